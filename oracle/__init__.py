"""CPU oracle for gate-level time-based power analysis (TEST INFRASTRUCTURE).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package.  The product library never loads it.

`build()` compiles pa_oracle.c with gcc into liboracle.so next to it;
`run()` calls the oracle on host numpy arrays.  See pa_oracle.c for what it
computes and which passage of "GPU-Accelerated Gate-Level Time-Based Power
Analysis via Event-Density-Aware Partitioning and Kernel Fusion" each step
follows.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "pa_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-ffp-contract=off", "-fno-fast-math", "-Wall",
          "-Wextra"]


def build(extra_flags=(), out=LIB) -> str:
    # compiled under a private name and renamed into place, so that a process
    # loading the library never sees a half-written file
    tmp = f"{out}.{os.getpid()}.tmp"
    cmd = ["gcc", *CFLAGS, *extra_flags, "-o", tmp, SRC, "-lm"]
    try:
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    finally:
        if os.path.exists(tmp):
            os.remove(tmp)
    return out


def host_threads(cap: int = 16) -> int:
    """Host cores this process may use, at most `cap` (the CPU share a GPU
    box gives one GPU is 16 cores, whatever the machine has)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(cap, n))


def cpu_model() -> str:
    """The host CPU's model name from /proc/cpuinfo ("unknown" if absent)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


class Totals(C.Structure):
    _fields_ = [("p_int_W", C.c_double), ("p_sw_W", C.c_double), ("p_gl_W", C.c_double),
                ("p_leak_W", C.c_double), ("e_int_J", C.c_double), ("e_sw_J", C.c_double),
                ("e_gl_J", C.c_double), ("e_leak_J", C.c_double), ("n_events", C.c_uint64),
                ("n_glitches", C.c_uint64), ("n_cycles", C.c_int64)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        L = C.CDLL(LIB)
        P = C.c_void_p
        L.pa_oracle_run.restype = C.c_int
        L.pa_oracle_run.argtypes = [C.c_int64, P, P, C.c_int32, P, C.c_int32, C.c_int32, P, P, P, P,
                                    C.c_double, C.c_int64, P, P, P, P, P, C.c_int64, C.c_int64,
                                    C.c_double, C.c_int64, C.c_int64, C.POINTER(Totals), P, P, P, P, P, P]
        L.pa_oracle_run_mt.restype = C.c_int
        L.pa_oracle_run_mt.argtypes = [C.c_int64, P, P, C.c_int32, P, C.c_int32, C.c_int32, P, P, P, P,
                                       C.c_double, C.c_int64, P, P, P, P, P, C.c_int64, C.c_int64,
                                       C.c_double, C.c_int64, C.c_int64, C.c_int32, C.POINTER(Totals), P, P, P,
                                       P, P, P]
        L.pa_oracle_bilerp.restype = C.c_double
        L.pa_oracle_bilerp.argtypes = [C.c_int, C.c_int, P, P, P, C.c_double, C.c_double]
        L.pa_oracle_n_cycles.restype = C.c_int64
        L.pa_oracle_n_cycles.argtypes = [C.c_int64, C.c_int64]
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def bilerp(slew_axis, cap_axis, table, x_slew, x_cap) -> float:
    sa, ca = _c(slew_axis, np.float64), _c(cap_axis, np.float64)
    tb = _c(table, np.float64)
    return lib().pa_oracle_bilerp(sa.shape[0], ca.shape[0], _p(sa), _p(ca), _p(tb), float(x_slew), float(x_cap))


class OracleError(RuntimeError):
    pass


def run(design, trace, gate_lo: int = 0, gate_hi: Optional[int] = None, per_event: bool = True,
        per_gate: bool = False, threads: int = 1) -> dict:
    """Run the oracle over gates [gate_lo, gate_hi).  Returns the totals, the
    per-cycle waveform/counts, (if per_event) the per-event glitch flags and
    states before each event, and (if per_gate) gate_J[G][4]: every gate's
    internal, switching, glitch and leakage energy (zero outside the range).
    threads > 1 walks contiguous gate ranges on that many host threads and
    merges their sums in range order (pa_oracle_run_mt)."""
    d, t = design, trace
    if gate_hi is None:
        gate_hi = d.n_gates
    arrs = dict(gc=_c(d.gate_cell, np.int32), cap=_c(d.gate_cap_F, np.float64), k=_c(d.cell_n_in, np.int32),
                sa=_c(d.slew_axis, np.float64), ca=_c(d.cap_axis, np.float64), lut=_c(d.lut_J, np.float64),
                leak=_c(d.leak_W, np.float64), pp=_c(t.pin_ptr, np.int64), pi=_c(t.pin_init, np.uint8),
                et=_c(t.evt_t, np.int64), ev=_c(t.evt_val, np.uint8), es=_c(t.evt_slew, np.float32))
    n_cyc = lib().pa_oracle_n_cycles(t.t_clk, t.t_max)
    if n_cyc <= 0:
        raise OracleError("bad clock or window")
    wave = np.zeros(n_cyc, np.float64)
    ce = np.zeros(n_cyc, np.uint64)
    cg = np.zeros(n_cyc, np.uint64)
    E = t.evt_t.shape[0]
    fl = np.zeros(E, np.uint8) if per_event else None
    st = np.zeros(E, np.uint8) if per_event else None
    gj = np.zeros((d.n_gates, 4), np.float64) if per_gate else None
    tot = Totals()
    a = arrs
    common = (d.n_gates, _p(a["gc"]), _p(a["cap"]), d.n_cells, _p(a["k"]), d.n_slew, d.n_cap, _p(a["sa"]),
              _p(a["ca"]), _p(a["lut"]), _p(a["leak"]), float(d.vdd_V), t.pin_init.shape[0], _p(a["pp"]),
              _p(a["pi"]), _p(a["et"]), _p(a["ev"]), _p(a["es"]), int(t.t_clk), int(t.t_max), float(t.tick_s),
              int(gate_lo), int(gate_hi))
    if threads > 1:
        rc = lib().pa_oracle_run_mt(*common, int(threads), C.byref(tot), _p(wave), _p(ce), _p(cg), _p(fl), _p(st),
                                    _p(gj))
    else:
        rc = lib().pa_oracle_run(*common, C.byref(tot), _p(wave), _p(ce), _p(cg), _p(fl), _p(st), _p(gj))
    if rc != 0:
        raise OracleError(f"oracle rejected the input (code {rc})")
    out = {f: getattr(tot, f) for f, _ in Totals._fields_}
    out.update(wave_J=wave, cyc_events=ce, cyc_glitches=cg)
    if per_event:
        out.update(evt_glitch=fl, evt_state_before=st)
    if per_gate:
        out.update(gate_J=gj)
    return out
