"""Plain reader of VCD-like activity text (TEST INFRASTRUCTURE: the oracle of
the library's event packer).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this module; the product library never loads it.

The paper's GPU flow packs the events of its activity files on the host
while the GPU computes ("GPU-Accelerated Gate-Level Time-Based Power Analysis
via Event-Density-Aware Partitioning and Kernel Fusion", end-to-end runtime
breakdown, Fig. 13).  It does not print the file format, so the
format is a reading: a subset of VCD with one slew per value change,

    $var <type> 1 <id> <name> [...] $end    one pin, pins in declaration order
    $<keyword> ... $end                     other definition sections, skipped
    $enddefinitions $end
    [#0] $dumpvars <v><id> ... $end         every pin's value at t = 0
    #<t>                                    timestamp, ticks, nondecreasing
    <v><id> <slew>                          value change at the current time

with <v> in {0, 1}, <id> 1..8 characters in '!'..'~', value changes before
the body's first timestamp at t = 0, and each slew read as the float32
nearest to its decimal value (ties to even).

`parse` does this line by line in plain Python, with the slew rounded from
its exact rational value, and returns the per-pin streams in the layout of
the library's event load (CSR over pins, each pin's events in time order).
It raises ValueError for text outside the format.  It is slow: use it on
small texts.
"""
from __future__ import annotations

import re
from fractions import Fraction

import numpy as np

_NUMBER = re.compile(r"^(\d*)(?:\.(\d*))?(?:[eE]([+-]?\d+))?$")
_F32_MAX_ROUND = (Fraction(2 ** 25 - 1) / 2) * Fraction(2) ** 104  # halfway between FLT_MAX and 2^128


def nearest_float32(q: Fraction) -> np.float32:
    """The float32 nearest to the rational q >= 0, ties to even (IEEE 754
    round-to-nearest-even)."""
    if q < 0:
        raise ValueError("negative")
    if q == 0:
        return np.float32(0.0)
    if q >= _F32_MAX_ROUND:
        return np.float32(np.inf)
    e = q.numerator.bit_length() - q.denominator.bit_length()
    if Fraction(2) ** e > q:
        e -= 1
    e = max(e, -126)  # subnormals are spaced like the smallest binade
    ulp = Fraction(2) ** (e - 23)
    m = q / ulp
    n = m.numerator // m.denominator
    r = m - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return np.float32(float(n * ulp))


def read_decimal(tok: str) -> np.float32:
    """A slew token [digits][.digits][(e|E)[+-]digits] as the nearest float32."""
    m = _NUMBER.match(tok)
    if not m or not ((m.group(1) or "") + (m.group(2) or "")):
        raise ValueError(f"bad slew {tok!r}")
    digits = (m.group(1) or "") + (m.group(2) or "")
    q = Fraction(int(digits)) * Fraction(10) ** (int(m.group(3) or 0) - len(m.group(2) or ""))
    return nearest_float32(q)


def _id_ok(s: str) -> bool:
    return 1 <= len(s) <= 8 and all(33 <= ord(c) <= 126 for c in s)


def parse(text, n_pins: int) -> dict:
    """CSR event streams of the text: pin_ptr [P+1], pin_init [P], evt_t,
    evt_val, evt_slew (caller's pin order = declaration order)."""
    if isinstance(text, (bytes, bytearray)):
        text = bytes(text).decode("ascii")
    # ---- definitions: whitespace-separated tokens up to $enddefinitions $end
    toks = [(m.group(0), m.end()) for m in re.finditer(r"\S+", text)]
    i, ids = 0, {}
    while True:
        if i >= len(toks):
            raise ValueError("no $enddefinitions")
        tok = toks[i][0]
        if tok == "$var":
            if i + 4 >= len(toks):
                raise ValueError("$var cut short")
            width, ident, name = toks[i + 2][0], toks[i + 3][0], toks[i + 4][0]
            if width != "1" or not _id_ok(ident) or name == "$end":
                raise ValueError("bad $var")
            if ident in ids:
                raise ValueError("identifier declared twice")
            ids[ident] = len(ids)
            i += 5
            while i < len(toks) and toks[i][0] != "$end":
                i += 1
            if i >= len(toks):
                raise ValueError("$var without $end")
            i += 1
        elif tok == "$enddefinitions":
            if i + 1 >= len(toks) or toks[i + 1][0] != "$end":
                raise ValueError("$enddefinitions without $end")
            i += 2
            break
        elif tok.startswith("$") and tok != "$end" and len(tok) > 1:
            i += 1
            while i < len(toks) and toks[i][0] != "$end":
                i += 1
            if i >= len(toks):
                raise ValueError("section without $end")
            i += 1
        else:
            raise ValueError(f"unexpected token {tok!r} in the definitions")
    if len(ids) != n_pins:
        raise ValueError(f"{len(ids)} variables declared, {n_pins} pins expected")
    # ---- initial values
    init = [None] * n_pins
    while True:
        if i >= len(toks):
            raise ValueError("no $dumpvars")
        tok = toks[i][0]
        if tok.startswith("#"):
            if tok[1:] != "0" and not (tok[1:].isdigit() and int(tok[1:]) == 0):
                raise ValueError("initial values must come at time 0")
            i += 1
        elif tok == "$dumpvars":
            i += 1
            while True:
                if i >= len(toks):
                    raise ValueError("$dumpvars without $end")
                tok = toks[i][0]
                i += 1
                if tok == "$end":
                    break
                if tok[0] not in "01" or tok[1:] not in ids:
                    raise ValueError(f"bad initial value {tok!r}")
                init[ids[tok[1:]]] = int(tok[0])
            body = toks[i - 1][1]
            break
        elif tok.startswith("$") and tok != "$end" and len(tok) > 1:
            i += 1
            while i < len(toks) and toks[i][0] != "$end":
                i += 1
            if i >= len(toks):
                raise ValueError("section without $end")
            i += 1
        else:
            raise ValueError("value change before $dumpvars")
    if any(v is None for v in init):
        raise ValueError("a pin has no initial value")
    # ---- value changes, line by line
    per_pin = [[] for _ in range(n_pins)]
    t = 0
    for line in text[body:].split("\n"):
        s = line.strip(" \t\r")
        if not s:
            continue
        if s[0] == "#":
            if not s[1:].isdigit() or len(s) > 19 or not s[1:].isascii():
                raise ValueError(f"bad timestamp {s!r}")
            t_new = int(s[1:])
            if t_new < t:
                raise ValueError("timestamps decrease")
            t = t_new
            continue
        parts = s.split()
        if len(parts) != 2 or s[0] not in "01":
            raise ValueError(f"bad value change {s!r}")
        ident = parts[0][1:]
        if ident not in ids:
            raise ValueError(f"unknown identifier {ident!r}")
        per_pin[ids[ident]].append((t, int(s[0]), read_decimal(parts[1])))
    counts = np.array([len(p) for p in per_pin], dtype=np.int64)
    pin_ptr = np.zeros(n_pins + 1, dtype=np.int64)
    np.cumsum(counts, out=pin_ptr[1:])
    ev = [e for p in per_pin for e in p]
    return dict(pin_ptr=pin_ptr, pin_init=np.array(init, dtype=np.uint8),
                evt_t=np.array([e[0] for e in ev], dtype=np.int64),
                evt_val=np.array([e[1] for e in ev], dtype=np.uint8),
                evt_slew=np.array([e[2] for e in ev], dtype=np.float32))
