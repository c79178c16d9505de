// pa_text.cpp -- host-side event packer: VCD-like activity text to per-pin
// event streams (see pa_text.h; the format is the one of pa_pack_text in
// include/pa.h).
#include "pa_text.h"

#include <locale.h>
#include <stdlib.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <limits>

#include "pa.h"

namespace pa::text {

namespace {

int bad(std::string &err, const char *fmt, ...) {
  char buf[256];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  err = buf;
  return PA_EDATA;
}

inline bool is_space(char c) { return c == ' ' || c == '\t' || c == '\n' || c == '\r' || c == '\v' || c == '\f'; }
inline bool is_blank(char c) { return c == ' ' || c == '\t' || c == '\r'; }
inline bool is_digit(char c) { return (unsigned)(c - '0') <= 9u; }

// identifier characters 33..126, at most 8, packed first-character-lowest
inline bool pack_id(const char *p, size_t n, uint64_t &key) {
  if (n == 0 || n > 8) return false;
  key = 0;
  for (size_t i = 0; i < n; ++i) {
    const unsigned c = (unsigned char)p[i];
    if (c < 33 || c > 126) return false;
    key |= (uint64_t)c << (8 * i);
  }
  return true;
}

// the value of eight decimal digits c[0..8) (c[0] most significant), or
// false if any of them is not a digit: every byte of w - '0' must be below 10
inline bool eight_digits(const char *c, uint64_t &v) {
  uint64_t w;
  std::memcpy(&w, c, 8);
  const uint64_t d = w - 0x3030303030303030ull;
  if (((w | (w + 0x4646464646464646ull)) & 0x8080808080808080ull) != 0 || (d & 0xF0F0F0F0F0F0F0F0ull) != 0)
    return false;
  // pairs, quads, then all eight (the first character is the low byte)
  uint64_t x = (d * 10 + (d >> 8)) & 0x00FF00FF00FF00FFull;
  x = (x * 100 + (x >> 16)) & 0x0000FFFF0000FFFFull;
  v = (x * 10000 + (x >> 32)) & 0xFFFFFFFFull;
  return true;
}

// nonnegative decimal integer [p, e) (at most 18 digits)
inline bool parse_time(const char *p, const char *e, int64_t &v) {
  if (p == e || e - p > 18) return false;
  int64_t x = 0;
  uint64_t v8;
  while (e - p >= 8 && eight_digits(p, v8)) {
    x = x * 100000000 + (int64_t)v8;
    p += 8;
  }
  for (; p < e; ++p) {
    if (!is_digit(*p)) return false;
    x = x * 10 + (*p - '0');
  }
  v = x;
  return true;
}

struct Tok {
  const char *s = nullptr;
  size_t n = 0, at = 0;
  bool is(const char *lit) const { return n == std::strlen(lit) && std::memcmp(s, lit, n) == 0; }
};

class Lexer {
 public:
  Lexer(const char *s, size_t n) : s_(s), n_(n) {}
  bool next(Tok &t) {
    while (i_ < n_ && is_space(s_[i_])) ++i_;
    if (i_ >= n_) return false;
    t.s = s_ + i_;
    t.at = i_;
    while (i_ < n_ && !is_space(s_[i_])) ++i_;
    t.n = (size_t)(s_ + i_ - t.s);
    return true;
  }
  size_t pos() const { return i_; }

 private:
  const char *s_;
  size_t n_, i_ = 0;
};

// skip the tokens of a "$keyword ... $end" section up to and including $end
bool skip_section(Lexer &lx) {
  Tok e;
  do {
    if (!lx.next(e)) return false;
  } while (!e.is("$end"));
  return true;
}

// exact powers of ten representable in a double
constexpr double kPow10[23] = {1e0,  1e1,  1e2,  1e3,  1e4,  1e5,  1e6,  1e7,  1e8,  1e9,  1e10, 1e11,
                               1e12, 1e13, 1e14, 1e15, 1e16, 1e17, 1e18, 1e19, 1e20, 1e21, 1e22};

bool parse_float_slow(const char *a, const char *b, float &out) {
  static locale_t c_locale = newlocale(LC_NUMERIC_MASK, "C", (locale_t)0);
  char buf[96];
  const size_t n = (size_t)(b - a);
  if (n == 0 || n >= sizeof buf || !c_locale) return false;
  std::memcpy(buf, a, n);
  buf[n] = 0;
  char *end = nullptr;
  out = strtof_l(buf, &end, c_locale);
  return end == buf + n;
}

}  // namespace

// A decimal number [digits][.digits][(e|E)[+-]digits] (at least one digit
// before the exponent) read as the nearest float; false for any other form.
// Fast path (Clinger, "How to read floating point numbers
// accurately", 1990): with at most 19 significant digits whose integer m is
// below 2^53 and a power of ten 10^q, |q| <= 22, the double m * 10^q (or
// m / 10^-q) is one correctly rounded operation on exact operands.  Rounding
// that double to float is then correct unless the double lies exactly halfway
// between two floats (a double rounding could then break the tie the wrong
// way); that case, and the numbers outside the fast path, go to strtof in
// the C locale, which rounds correctly.
bool parse_float(const char *a, const char *b, float &out) {
  const char *p = a;
  uint64_t m = 0;
  int nd = 0, q = 0;  // digits taken into m (leading zeros included), power of ten
  bool any = false, lost = false;
  uint64_t v8;
  if (b - p >= 8 && eight_digits(p, v8)) {  // the first eight digits at once
    m = v8;
    nd = 8;
    p += 8;
    any = true;
  }
  for (; p < b && is_digit(*p); ++p) {
    any = true;
    if (nd < 19) {
      m = m * 10 + (uint64_t)(*p - '0');
      ++nd;
    } else {
      ++q;
      lost |= *p != '0';
    }
  }
  if (p < b && *p == '.') {
    for (++p; p < b && is_digit(*p); ++p) {
      any = true;
      if (nd < 19) {
        m = m * 10 + (uint64_t)(*p - '0');
        ++nd;
        --q;
      } else {
        lost |= *p != '0';
      }
    }
  }
  if (!any) return false;
  if (p < b && (*p == 'e' || *p == 'E')) {
    ++p;
    int sign = 1;
    if (p < b && (*p == '+' || *p == '-')) sign = *p++ == '-' ? -1 : 1;
    if (p == b || !is_digit(*p)) return false;
    int x = 0;
    for (; p < b && is_digit(*p); ++p) x = std::min(x * 10 + (*p - '0'), 100000);
    q += sign * x;
  }
  if (p != b) return false;  // not of the decimal form
  if (lost) return parse_float_slow(a, b, out);
  if (m == 0) {
    out = 0.0f;
    return true;
  }
  if (m >= (uint64_t(1) << 53) || q < -22 || q > 22) return parse_float_slow(a, b, out);
  const double d = q >= 0 ? (double)m * kPow10[q] : (double)m / kPow10[-q];
  // a double in the range of normal floats lies halfway between two floats
  // exactly when its 29 significand bits below float precision are 1000...0;
  // outside that range (and for those) the slow path decides
  uint64_t bits;
  std::memcpy(&bits, &d, sizeof bits);
  const uint64_t ex = (bits >> 52) & 0x7FF;
  if (ex < 1023 - 125 || ex > 1023 + 127 || (bits & ((uint64_t(1) << 29) - 1)) == (uint64_t(1) << 28))
    return parse_float_slow(a, b, out);
  out = (float)d;
  return true;
}

// ------------------------------------------------------------------ Pool --

Pool::Pool(int n) : n_(std::max(1, n)) {
  for (int i = 1; i < n_; ++i) th_.emplace_back([this] { worker(); });
}

Pool::~Pool() {
  {
    std::lock_guard<std::mutex> g(mu_);
    stop_ = true;
  }
  cv_go_.notify_all();
  for (auto &t : th_) t.join();
}

void Pool::drain() {
  for (;;) {
    const std::function<void(int)> *fn;
    int i;
    {
      std::lock_guard<std::mutex> g(mu_);
      if (next_ >= tasks_) return;
      i = next_++;
      fn = fn_;
    }
    (*fn)(i);
  }
}

void Pool::worker() {
  uint64_t seen = 0;
  for (;;) {
    {
      std::unique_lock<std::mutex> lk(mu_);
      cv_go_.wait(lk, [&] { return stop_ || gen_ != seen; });
      if (stop_) return;
      seen = gen_;
      ++busy_;
    }
    drain();
    {
      std::lock_guard<std::mutex> g(mu_);
      if (--busy_ == 0) cv_done_.notify_all();
    }
  }
}

void Pool::run(int tasks, const std::function<void(int)> &fn) {
  if (tasks <= 0) return;
  if (n_ == 1 || tasks == 1) {
    for (int i = 0; i < tasks; ++i) fn(i);
    return;
  }
  {
    std::lock_guard<std::mutex> g(mu_);
    fn_ = &fn;
    tasks_ = tasks;
    next_ = 0;
    ++gen_;
  }
  cv_go_.notify_all();
  drain();
  std::unique_lock<std::mutex> lk(mu_);
  cv_done_.wait(lk, [&] { return next_ >= tasks_ && busy_ == 0; });
  fn_ = nullptr;
  tasks_ = 0;
  next_ = 0;
}

// ----------------------------------------------------------------- IdMap --

void IdMap::reset(int64_t n) {
  size_t cap = 16;
  int bits = 4;
  while ((int64_t)cap < 2 * n) {
    cap <<= 1;
    ++bits;
  }
  keys_.assign(cap, 0);
  pins_.assign(cap, -1);
  mask_ = cap - 1;
  shift_ = 64 - bits;
}

bool IdMap::insert(uint64_t key, int32_t pin) {
  size_t i = (size_t)((key * 0x9E3779B97F4A7C15ull) >> shift_);
  while (keys_[i] != 0) {
    if (keys_[i] == key) return false;
    i = (i + 1) & mask_;
  }
  keys_[i] = key;
  pins_[i] = pin;
  return true;
}

// ---------------------------------------------------------------- header --

int parse_header(const char *s, size_t n, Header &h, std::string &err) {
  Lexer lx(s, n);
  Tok t;
  std::vector<uint64_t> keys;
  bool defs_done = false;
  while (lx.next(t)) {
    if (t.is("$var")) {
      Tok type, width, id, name;
      if (!lx.next(type) || !lx.next(width) || !lx.next(id) || !lx.next(name))
        return bad(err, "$var at byte %zu is cut short", t.at);
      if (!width.is("1")) return bad(err, "$var at byte %zu: width must be 1 (one variable per pin)", t.at);
      uint64_t key;
      if (!pack_id(id.s, id.n, key))
        return bad(err, "$var at byte %zu: the identifier must be 1-8 characters in '!'..'~'", t.at);
      if (name.is("$end")) return bad(err, "$var at byte %zu has no name", t.at);
      keys.push_back(key);
      if (!skip_section(lx)) return bad(err, "$var at byte %zu has no $end", t.at);
    } else if (t.is("$enddefinitions")) {
      Tok e;
      if (!lx.next(e) || !e.is("$end")) return bad(err, "$enddefinitions at byte %zu has no $end", t.at);
      defs_done = true;
      break;
    } else if (t.n > 1 && t.s[0] == '$' && !t.is("$end")) {
      if (!skip_section(lx)) return bad(err, "section at byte %zu has no $end", t.at);
    } else {
      return bad(err, "unexpected token at byte %zu in the definitions", t.at);
    }
  }
  if (!defs_done) return bad(err, "no $enddefinitions");
  const int64_t P = (int64_t)keys.size();
  if (P >= (int64_t(1) << 31)) return bad(err, "too many variables");
  h.n_pins = P;
  h.ids.reset(P);
  for (int64_t i = 0; i < P; ++i)
    if (!h.ids.insert(keys[i], (int32_t)i)) return bad(err, "the identifier of variable %lld is declared twice", (long long)i);
  h.init.assign((size_t)P, 2);
  bool dumped = false;
  while (lx.next(t)) {
    if (t.s[0] == '#') {
      int64_t v;
      if (!parse_time(t.s + 1, t.s + t.n, v) || v != 0)
        return bad(err, "the initial values ($dumpvars) must come at time 0 (byte %zu)", t.at);
      continue;
    }
    if (t.is("$dumpvars")) {
      Tok v;
      for (;;) {
        if (!lx.next(v)) return bad(err, "$dumpvars at byte %zu has no $end", t.at);
        if (v.is("$end")) break;
        if (v.s[0] != '0' && v.s[0] != '1') return bad(err, "initial value at byte %zu must be 0 or 1", v.at);
        uint64_t key;
        if (!pack_id(v.s + 1, v.n - 1, key)) return bad(err, "bad identifier at byte %zu", v.at);
        const int32_t p = h.ids.find(key);
        if (p < 0) return bad(err, "unknown identifier at byte %zu", v.at);
        h.init[(size_t)p] = (uint8_t)(v.s[0] - '0');
      }
      dumped = true;
      break;
    }
    if (t.n > 1 && t.s[0] == '$' && !t.is("$end")) {
      if (!skip_section(lx)) return bad(err, "section at byte %zu has no $end", t.at);
      continue;
    }
    return bad(err, "value change at byte %zu before the initial values ($dumpvars)", t.at);
  }
  if (!dumped) return bad(err, "no $dumpvars section with the initial values");
  for (int64_t p = 0; p < P; ++p)
    if (h.init[(size_t)p] > 1) return bad(err, "variable %lld has no initial value in $dumpvars", (long long)p);
  h.body = lx.pos();
  return 0;
}

// ----------------------------------------------------------- segmentation --

namespace {
struct PieceIndex {
  std::vector<std::pair<size_t, int64_t>> starts;  // (byte of a time line, its segment) where the segment changes
  std::vector<std::pair<int64_t, int64_t>> counts; // (segment, value changes) in order
  int64_t pre = 0;                                 // value changes before the piece's first time line
  int64_t first_t = -1, last_t = -1;
  std::string err;
  size_t err_at = 0;
};

// the first '\n' in [p, e), or e: eight bytes at a time (a byte of w ^ '\n'
// that is zero gives the lowest flag of the borrow trick exactly)
inline const char *find_nl(const char *p, const char *e) {
  while (e - p >= 8) {
    uint64_t w;
    std::memcpy(&w, p, 8);
    const uint64_t x = w ^ 0x0A0A0A0A0A0A0A0Aull;
    const uint64_t t = (x - 0x0101010101010101ull) & ~x & 0x8080808080808080ull;
    if (t) return p + (__builtin_ctzll(t) >> 3);
    p += 8;
  }
  while (p < e && *p != '\n') ++p;
  return p;
}

// the first byte at or after c (and after b0) that starts a line
size_t line_start_at_or_after(const char *s, size_t b0, size_t b1, size_t c) {
  if (c <= b0) return b0;
  const void *nl = std::memchr(s + c - 1, '\n', b1 - (c - 1));
  return nl ? (size_t)((const char *)nl - s) + 1 : b1;
}

// the first line start at or after c whose first byte is '#' (b1 if none)
size_t time_line_at_or_after(const char *s, size_t b0, size_t b1, size_t c) {
  size_t i = line_start_at_or_after(s, b0, b1, c);
  while (i < b1 && s[i] != '#') {
    const void *nl = std::memchr(s + i, '\n', b1 - i);
    if (!nl) return b1;
    i = (size_t)((const char *)nl - s) + 1;
  }
  return i;
}
}  // namespace

int index_segments(const char *s, size_t n, const Header &h, int64_t seg_ticks, int64_t n_seg, int64_t t_end,
                   Pool &pool, SegmentIndex &ix, std::string &err) {
  const size_t b0 = h.body;
  const int np = (int)std::max<int64_t>(1, std::min<int64_t>(4 * pool.size(), (int64_t)((n - b0) >> 18)));
  std::vector<size_t> cut(np + 1);
  cut[0] = b0;
  cut[np] = n;
  for (int i = 1; i < np; ++i)
    cut[i] = std::max(cut[i - 1], line_start_at_or_after(s, b0, n, b0 + (n - b0) * (size_t)i / (size_t)np));
  std::vector<PieceIndex> pc(np);
  pool.run(np, [&](int i) {
    PieceIndex &X = pc[i];
    const char *p = s + cut[i], *e = s + cut[i + 1];
    int64_t seg = -1, cnt = 0, sg = -1, seg_lo = 0, seg_hi = -1;
    while (p < e) {
      const char *line = p;
      const char *le = find_nl(p, e);
      p = le < e ? le + 1 : e;
      const char *q = line;
      while (q < le && is_blank(*q)) ++q;
      if (q == le) continue;
      if (*q != '#') {
        ++cnt;
        continue;
      }
      const char *d = q + 1, *de = d;
      while (de < le && is_digit(*de)) ++de;
      const char *r = de;
      while (r < le && is_blank(*r)) ++r;
      int64_t tv;
      if (!parse_time(d, de, tv) || r != le) {
        X.err = "bad timestamp line";
        X.err_at = (size_t)(q - s);
        return;
      }
      if (tv < X.last_t) {
        X.err = "timestamps decrease";
        X.err_at = (size_t)(q - s);
        return;
      }
      if (X.first_t < 0) X.first_t = tv;
      X.last_t = tv;
      // the segment of tv (a division only when tv leaves the current one)
      if (tv < seg_lo || tv >= seg_hi) {
        const int64_t k = tv >= t_end ? n_seg : std::min(tv / seg_ticks, n_seg);
        seg_lo = k < n_seg ? k * seg_ticks : t_end;
        seg_hi = k < n_seg - 1 ? seg_lo + seg_ticks : (k < n_seg ? t_end : std::numeric_limits<int64_t>::max());
        sg = k;
      }
      if (sg != seg) {
        if (seg < 0)
          X.pre = cnt;
        else if (cnt)
          X.counts.emplace_back(seg, cnt);
        X.starts.emplace_back((size_t)(line - s), sg);
        seg = sg;
        cnt = 0;
      }
    }
    if (seg < 0)
      X.pre = cnt;
    else if (cnt)
      X.counts.emplace_back(seg, cnt);
  });
  ix.begin.assign((size_t)n_seg + 1, n);
  ix.events.assign((size_t)n_seg + 1, 0);
  ix.begin[0] = b0;
  int64_t cur = 0, last_t = 0;  // the body starts at time 0
  for (int i = 0; i < np; ++i) {
    const PieceIndex &X = pc[i];
    if (!X.err.empty()) return bad(err, "%s at byte %zu", X.err.c_str(), X.err_at);
    if (X.first_t >= 0) {
      if (X.first_t < last_t) return bad(err, "timestamps decrease at byte %zu", X.starts.front().first);
      last_t = X.last_t;
    }
    ix.events[(size_t)cur] += X.pre;
    for (const auto &st : X.starts) {
      for (int64_t k = cur + 1; k <= st.second; ++k) ix.begin[(size_t)k] = st.first;
      cur = std::max(cur, st.second);
    }
    for (const auto &c : X.counts) ix.events[(size_t)c.first] += c.second;
  }
  if (ix.events[(size_t)n_seg] != 0) return bad(err, "value change at or after the end of the analysis window");
  ix.events.resize((size_t)n_seg);
  return 0;
}

// ---------------------------------------------------------------- packing --

int Packer::pack(const char *s, size_t b0, size_t b1, const Header &h, int64_t n_events, int64_t t_origin,
                 const uint8_t *init_in, const Csr &out, uint8_t *init_out, std::string &err) {
  const int64_t P = h.n_pins;
  if (n_events >= (int64_t(1) << 31)) return bad(err, "more than 2^31 - 1 value changes in one segment");
  const int np = (int)std::max<int64_t>(1, std::min<int64_t>(pool_.size(), (int64_t)((b1 - b0) >> 18)));
  if ((int)loc_.size() < np) loc_.resize(np);
  cut_.assign(np + 1, b1);
  cut_[0] = b0;
  for (int i = 1; i < np; ++i)
    cut_[i] = std::max(cut_[i - 1], time_line_at_or_after(s, b0, b1, b0 + (b1 - b0) * (size_t)i / (size_t)np));
  // 1. parse every piece into its own records and per-pin counts
  pool_.run(np, [&](int i) {
    Local &L = loc_[i];
    L.err.clear();
    L.cnt.assign((size_t)P, 0u);
    L.pin.clear();
    L.t.clear();
    L.slew.clear();
    L.val.clear();
    const size_t guess = (cut_[i + 1] - cut_[i]) / 12 + 16;
    L.pin.reserve(guess);
    L.t.reserve(guess);
    L.slew.reserve(guess);
    L.val.reserve(guess);
    const char *p = s + cut_[i], *e = s + cut_[i + 1];
    int64_t tcur = 0;
    auto fail_at = [&](const char *msg, const char *where) {
      L.err = msg;
      L.err_at = (size_t)(where - s);
    };
    while (p < e) {
      const char c = *p;
      if (c == '\n' || is_blank(c)) {
        ++p;
        continue;
      }
      if (c == '#') {
        const char *q = p + 1, *d = q;
        while (q < e && is_digit(*q)) ++q;
        if (!parse_time(d, q, tcur)) return fail_at("bad timestamp", p);
        while (q < e && is_blank(*q)) ++q;
        if (q < e && *q != '\n') return fail_at("text after a timestamp", p);
        p = q;
        continue;
      }
      if (c != '0' && c != '1') return fail_at("value change must start with 0 or 1", p);
      const char *q = p + 1;
      uint64_t key = 0;
      int k = 0;
      for (; q < e && (unsigned char)*q > 32 && (unsigned char)*q < 127; ++q, ++k)
        if (k < 8) key |= (uint64_t)(unsigned char)*q << (8 * k);
      if (k == 0 || k > 8) return fail_at("bad identifier", p);
      const int32_t pin = h.ids.find(key);
      if (pin < 0) return fail_at("unknown identifier", p);
      while (q < e && is_blank(*q) && *q != '\r') ++q;
      const char *ss = q;
      while (q < e && (unsigned char)*q > 32) ++q;
      if (q == ss) return fail_at("value change without a slew", p);
      float sl;
      if (!parse_float(ss, q, sl)) return fail_at("bad slew", ss);
      while (q < e && is_blank(*q)) ++q;
      if (q < e && *q != '\n') return fail_at("text after the slew", p);
      L.pin.push_back((uint32_t)pin);
      L.t.push_back(tcur - t_origin);
      L.val.push_back((uint8_t)(c - '0'));
      L.slew.push_back(sl);
      ++L.cnt[(size_t)pin];
      p = q;
    }
  });
  int64_t total = 0;
  for (int i = 0; i < np; ++i) {
    if (!loc_[i].err.empty()) return bad(err, "%s at byte %zu", loc_[i].err.c_str(), loc_[i].err_at);
    total += (int64_t)loc_[i].pin.size();
  }
  if (total != n_events) return bad(err, "segment holds %lld value changes, %lld expected", (long long)total, (long long)n_events);
  // 2. CSR offsets: pin-major, pieces in text (= time) order inside a pin
  const int nr = pool_.size();
  range_sum_.assign((size_t)nr + 1, 0);
  auto range = [&](int r, int64_t &p0, int64_t &p1) {
    p0 = P * r / nr;
    p1 = P * (r + 1) / nr;
  };
  pool_.run(nr, [&](int r) {
    int64_t p0, p1, sum = 0;
    range(r, p0, p1);
    for (int i = 0; i < np; ++i) {
      const uint32_t *cnt = loc_[i].cnt.data();
      for (int64_t p = p0; p < p1; ++p) sum += cnt[p];
    }
    range_sum_[(size_t)r + 1] = sum;
  });
  for (int r = 0; r < nr; ++r) range_sum_[(size_t)r + 1] += range_sum_[(size_t)r];
  pool_.run(nr, [&](int r) {
    int64_t p0, p1;
    range(r, p0, p1);
    int64_t run = range_sum_[(size_t)r];
    for (int64_t p = p0; p < p1; ++p) {
      out.pin_ptr[p] = run;
      for (int i = 0; i < np; ++i) {
        uint32_t &c = loc_[i].cnt[(size_t)p];
        const uint32_t k = c;
        c = (uint32_t)run;
        run += k;
      }
    }
  });
  out.pin_ptr[P] = total;
  // 3. scatter every piece's records to their slots
  pool_.run(np, [&](int i) {
    Local &L = loc_[i];
    const size_t m = L.pin.size();
    for (size_t j = 0; j < m; ++j) {
      const uint32_t pos = L.cnt[L.pin[j]]++;
      out.t[pos] = L.t[j];
      out.val[pos] = L.val[j];
      out.slew[pos] = L.slew[j];
    }
  });
  // 4. the pin values at the segment start and at its end
  pool_.run(nr, [&](int r) {
    int64_t p0, p1;
    range(r, p0, p1);
    for (int64_t p = p0; p < p1; ++p) {
      const uint8_t v0 = init_in[p];
      out.pin_init[p] = v0;
      init_out[p] = out.pin_ptr[p + 1] > out.pin_ptr[p] ? out.val[out.pin_ptr[p + 1] - 1] : v0;
    }
  });
  return 0;
}

}  // namespace pa::text
