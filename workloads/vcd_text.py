"""Writes a synthetic event trace as VCD-like activity text.

This is an input generator: it turns a `synth.Trace` (per-pin CSR streams)
into the text that the library's event packer reads, and holds none of the
power arithmetic.  The paper's GPU flow packs events on the host from
activity files while the GPU computes ("GPU-Accelerated Gate-Level Time-
Based Power Analysis via Event-Density-Aware Partitioning and Kernel Fusion",
end-to-end runtime breakdown, Fig. 13); its activity files are not
available, so this text stands in for them.

Format (a subset of VCD, plus one slew per value change):

    $timescale 1 fs $end                one tick
    $scope module top $end
    $var wire 1 <id> <name> $end        one line per pin, in pin order
    $upscope $end
    $enddefinitions $end
    #0
    $dumpvars
    <v><id>                             the value of every pin at t = 0
    $end
    #<t>                                nondecreasing timestamps, ticks
    <v><id> <slew>                      value change at t with its slew, ticks

`<id>` is a string of printable ASCII characters 33..126 (at most 8 here);
`<v>` is 0 or 1.  This writer gives every pin an id of the same length
(base-94 digits of the pin index) and prints each slew with nine significant
digits, enough for every float32 value to read back exactly.
"""
from __future__ import annotations

import numpy as np

ID_FIRST = 33
ID_BASE = 94


def id_length(n_pins: int) -> int:
    n, length = ID_BASE, 1
    while n < n_pins:
        n *= ID_BASE
        length += 1
    return length


def pin_ids(n_pins: int) -> np.ndarray:
    """uint8 [n_pins, L]: every pin's id characters (base-94, most significant first)."""
    L = id_length(n_pins)
    p = np.arange(n_pins, dtype=np.int64)
    out = np.empty((n_pins, L), dtype=np.uint8)
    for j in range(L - 1, -1, -1):
        out[:, j] = ID_FIRST + p % ID_BASE
        p //= ID_BASE
    return out


def _header(n_pins: int, ids: np.ndarray, pin_init: np.ndarray) -> bytes:
    id_str = [bytes(r).decode() for r in ids]
    parts = ["$timescale 1 fs $end\n", "$scope module top $end\n"]
    parts += [f"$var wire 1 {s} p{i} $end\n" for i, s in enumerate(id_str)]
    parts += ["$upscope $end\n", "$enddefinitions $end\n", "#0\n", "$dumpvars\n"]
    parts += [f"{int(v)}{s}\n" for v, s in zip(pin_init.tolist(), id_str)]
    parts.append("$end\n")
    return "".join(parts).encode()


def _digits(x: np.ndarray) -> np.ndarray:
    """Decimal digit count of nonnegative int64 values (1 for 0)."""
    nd = np.ones(x.shape, dtype=np.int64)
    for k in range(1, 19):
        nd += x >= 10 ** k
    return nd


def _put_int(buf: np.ndarray, pos: np.ndarray, x: np.ndarray, nd: np.ndarray) -> None:
    """Write the decimal digits of x (nd of them) at buf[pos : pos + nd]."""
    last = pos + nd - 1
    lo = int(nd.min(initial=1))
    for k in range(int(nd.max(initial=1))):
        if k < lo:
            buf[last - k] = 48 + (x // 10 ** k) % 10
        else:
            m = nd > k
            buf[last[m] - k] = 48 + (x[m] // 10 ** k) % 10


def _slew_fields(s: np.ndarray):
    """Nine significant digits of every slew as (mantissa, exponent): the
    value is mantissa * 10^exponent, mantissa in [1e8, 1e9)."""
    v = s.astype(np.float64)
    if np.any(~np.isfinite(v)) or np.any(v <= 0):
        raise ValueError("slews must be finite and > 0")
    e = np.floor(np.log10(v)).astype(np.int64) - 8
    m = np.rint(v / np.power(10.0, e)).astype(np.int64)
    hi = m >= 1_000_000_000
    m[hi] = np.rint(v[hi] / np.power(10.0, e[hi] + 1)).astype(np.int64)
    e[hi] += 1
    lo = m < 100_000_000
    m[lo] = np.rint(v[lo] / np.power(10.0, e[lo] - 1)).astype(np.int64)
    e[lo] -= 1
    back = (m.astype(np.float64) * np.power(10.0, e)).astype(np.float32)
    if not np.array_equal(back, s.astype(np.float32)):
        raise AssertionError("nine-digit slew text does not read back")
    return m, e


def write(trace) -> bytes:
    """The VCD-like text of `trace` (a synth.Trace): value changes grouped by
    timestamp, the pins of one timestamp in pin order."""
    P, E = trace.n_pins, trace.n_events
    ids = pin_ids(P)
    L = ids.shape[1]
    head = _header(P, ids, trace.pin_init)
    if E == 0:
        return head
    pin = np.repeat(np.arange(P, dtype=np.int64), np.diff(trace.pin_ptr))
    order = np.lexsort((pin, trace.evt_t))
    pin = pin[order]
    t = trace.evt_t[order]
    val = trace.evt_val[order]
    m, e = _slew_fields(trace.evt_slew[order])
    # a time line before the first event of every timestamp ("#0" is already in the header)
    new_t = np.ones(E, dtype=bool)
    new_t[1:] = t[1:] != t[:-1]
    if t[0] == 0:
        new_t[0] = False
    nd_t = _digits(t)
    t_len = np.where(new_t, 2 + nd_t, 0)
    # event line: v, id, ' ', 9 mantissa digits, 'e', sign, exponent digits, '\n'
    ae = np.abs(e)
    nd_e = _digits(ae)
    ev_len = 1 + L + 1 + 9 + 2 + nd_e + 1
    line = t_len + ev_len
    start = np.zeros(E, dtype=np.int64)
    np.cumsum(line[:-1], out=start[1:])
    buf = np.empty(int(start[-1] + line[-1]), dtype=np.uint8)
    ts = start[new_t]
    buf[ts] = ord("#")
    _put_int(buf, ts + 1, t[new_t], nd_t[new_t])
    buf[ts + 1 + nd_t[new_t]] = ord("\n")
    p0 = start + t_len
    buf[p0] = (48 + val).astype(np.uint8)
    for j in range(L):
        buf[p0 + 1 + j] = ids[pin, j]
    buf[p0 + 1 + L] = ord(" ")
    _put_int(buf, p0 + 2 + L, m, np.full(E, 9, dtype=np.int64))
    buf[p0 + 11 + L] = ord("e")
    buf[p0 + 12 + L] = np.where(e < 0, ord("-"), ord("+")).astype(np.uint8)
    _put_int(buf, p0 + 13 + L, ae, nd_e)
    buf[p0 + 13 + L + nd_e] = ord("\n")
    return head + buf.tobytes()
