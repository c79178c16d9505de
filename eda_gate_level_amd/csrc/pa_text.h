// pa_text.h -- host-side event packer (internal): reads VCD-like activity
// text into the per-pin event streams the library loads, on host threads.
//
// The paper's GPU flow packs events on the CPU and overlaps that with the
// GPU's power computation ("GPU-Accelerated Gate-Level Time-Based Power
// Analysis via Event-Density-Aware Partitioning and Kernel Fusion",
// end-to-end runtime breakdown, Fig. 13).  The text format is described in
// include/pa.h (pa_pack_text).  Everything here is plain C++ (no HIP).
#pragma once
#include <condition_variable>
#include <cstddef>
#include <cstdint>
#include <functional>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

namespace pa::text {

// A fixed set of worker threads that run fn(0..tasks-1) and return when all
// are done; the calling thread takes part.
class Pool {
 public:
  explicit Pool(int n_threads);
  ~Pool();
  Pool(const Pool &) = delete;
  Pool &operator=(const Pool &) = delete;
  int size() const { return n_; }
  void run(int tasks, const std::function<void(int)> &fn);

 private:
  void worker();
  void drain();
  int n_;
  std::vector<std::thread> th_;
  std::mutex mu_;
  std::condition_variable cv_go_, cv_done_;
  const std::function<void(int)> *fn_ = nullptr;
  int tasks_ = 0, next_ = 0, busy_ = 0;
  uint64_t gen_ = 0;
  bool stop_ = false;
};

// Identifier codes (1..8 characters in 33..126) packed into 64 bits, the
// first character in the low byte, mapped to pin indices.
class IdMap {
 public:
  void reset(int64_t n);
  bool insert(uint64_t key, int32_t pin);  // false if the key is there already
  int32_t find(uint64_t key) const {
    size_t i = (size_t)((key * 0x9E3779B97F4A7C15ull) >> shift_);
    for (;;) {
      const uint64_t k = keys_[i];
      if (k == key) return pins_[i];
      if (k == 0) return -1;
      i = (i + 1) & mask_;
    }
  }

 private:
  std::vector<uint64_t> keys_;
  std::vector<int32_t> pins_;
  size_t mask_ = 0;
  int shift_ = 64;
};

struct Header {
  int64_t n_pins = 0;
  std::vector<uint8_t> init;  // every pin's value at t = 0
  IdMap ids;
  size_t body = 0;            // byte offset of the value changes that follow $dumpvars
};

// Definitions and initial values.  Returns 0, or PA_EDATA with err set.
int parse_header(const char *s, size_t n, Header &h, std::string &err);

struct SegmentIndex {
  std::vector<size_t> begin;    // [n_seg + 1] first byte of segment k; begin[n_seg] = end of text
  std::vector<int64_t> events;  // [n_seg] value changes in segment k
};

// Cut the value changes into segments of seg_ticks ticks: segment k holds
// the times [k seg_ticks, (k + 1) seg_ticks).  Checks that timestamps never
// decrease and that no value change comes at or after t_end.
int index_segments(const char *s, size_t n, const Header &h, int64_t seg_ticks, int64_t n_seg, int64_t t_end,
                   Pool &pool, SegmentIndex &ix, std::string &err);

// One segment's events in the library's input layout (arrays owned by the caller).
struct Csr {
  int64_t *pin_ptr;  // [P + 1]
  uint8_t *pin_init; // [P]
  int64_t *t;        // [E]
  uint8_t *val;      // [E]
  float *slew;       // [E]
};

// Parses one segment's bytes on the pool's threads and packs them per pin.
class Packer {
 public:
  explicit Packer(Pool &pool) : pool_(pool) {}
  // [b0, b1): a segment of the body (starting at a time line, or at the body
  // start where the time is 0); n_events: its value changes per the index;
  // times are stored minus t_origin; init_in: pin values at the segment
  // start (copied to out.pin_init); init_out: the values at its end.
  int pack(const char *s, size_t b0, size_t b1, const Header &h, int64_t n_events, int64_t t_origin,
           const uint8_t *init_in, const Csr &out, uint8_t *init_out, std::string &err);

 private:
  struct Local {
    std::vector<uint32_t> pin;
    std::vector<int64_t> t;
    std::vector<float> slew;
    std::vector<uint8_t> val;
    std::vector<uint32_t> cnt;  // per pin: events, then the next output slot
    std::string err;
    size_t err_at = 0;
  };
  Pool &pool_;
  std::vector<Local> loc_;
  std::vector<size_t> cut_;
  std::vector<int64_t> range_sum_;
};

// Parses a slew token [a, b) as the float nearest to its decimal value.
bool parse_float(const char *a, const char *b, float &out);

}  // namespace pa::text
