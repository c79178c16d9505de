"""Seeded synthetic designs and event traces for gate-level power analysis.

This module only draws random inputs.  It contains none of the power
arithmetic (no interpolation, no state tracking, no energies) and is the one
module that both the CPU oracle's tests and the HIP path's tests, smoke run
and benchmark take their inputs from.

The workloads stand in for the designs and activity traces that "GPU-
Accelerated Gate-Level Time-Based Power Analysis via Event-Density-Aware
Partitioning and Kernel Fusion" (arXiv 2609.05960) evaluates on (the benchmark
designs and traces of its Table 2, which are not available here).  Their shapes follow the paper's
problem statement: gates with k input pins and one output pin, per-pin
sorted event streams (Sec. 2.4.1/2.4.2), state-indexed internal-power LUTs
per input pin and state-indexed leakage (Figs. 2-3), and the skewed per-gate
event counts the paper reports (Sec. 3.2, Fig. 4).

Units: one tick is 1 fs (tick_s = 1e-15); timestamps, clock period, t_max
and slews are integers/floats in ticks; caps in F; LUT entries in J; leakage
in W; Vdd in V.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np

TICK_S = 1e-15
PS = 1000  # ticks per picosecond
NS = 1_000_000  # ticks per nanosecond
FF = 1e-15  # farad per femtofarad
FJ = 1e-15  # joule per femtojoule


@dataclasses.dataclass
class Design:
    gate_cell: np.ndarray  # int32 [G]
    gate_cap_F: np.ndarray  # float64 [G]
    cell_n_in: np.ndarray  # int32 [n_cells]
    n_slew: int
    n_cap: int
    slew_axis: np.ndarray  # float64 [n_cells, n_slew], ticks
    cap_axis: np.ndarray  # float64 [n_cells, n_cap], F
    lut_J: np.ndarray  # float64, per cell [2^k][k][n_slew][n_cap] concatenated
    leak_W: np.ndarray  # float64, per cell [2^k] concatenated
    vdd_V: float

    @property
    def n_gates(self) -> int:
        return int(self.gate_cell.shape[0])

    @property
    def n_cells(self) -> int:
        return int(self.cell_n_in.shape[0])

    def gate_k(self) -> np.ndarray:
        return self.cell_n_in[self.gate_cell].astype(np.int64)

    def pin_base(self) -> np.ndarray:
        """First pin id of every gate (gate-major pins, k inputs then the output)."""
        pb = np.zeros(self.n_gates + 1, dtype=np.int64)
        np.cumsum(self.gate_k() + 1, out=pb[1:])
        return pb

    def lut_base(self) -> np.ndarray:
        k = self.cell_n_in.astype(np.int64)
        sizes = (1 << k) * k * self.n_slew * self.n_cap
        return np.concatenate([[0], np.cumsum(sizes)[:-1]]).astype(np.int64)

    def leak_base(self) -> np.ndarray:
        k = self.cell_n_in.astype(np.int64)
        return np.concatenate([[0], np.cumsum(1 << k)[:-1]]).astype(np.int64)


@dataclasses.dataclass
class Trace:
    pin_ptr: np.ndarray  # int64 [P+1]
    pin_init: np.ndarray  # uint8 [P]
    evt_t: np.ndarray  # int64 [E], ticks, strictly increasing per pin
    evt_val: np.ndarray  # uint8 [E], alternating from not(init)
    evt_slew: np.ndarray  # float32 [E], ticks
    t_clk: int
    t_max: int
    tick_s: float = TICK_S

    @property
    def n_pins(self) -> int:
        return int(self.pin_init.shape[0])

    @property
    def n_events(self) -> int:
        return int(self.evt_t.shape[0])

    @property
    def n_cycles(self) -> int:
        return -(-self.t_max // self.t_clk)


@dataclasses.dataclass
class Workload:
    name: str
    design: Design
    trace: Trace
    info: Dict[str, float]


# --------------------------------------------------------------- library --

def make_library(rng: np.random.Generator, ks, cells_per_k: int = 8, n_axis: int = 7) -> Design:
    """A small cell library: `cells_per_k` cell types for every input count in
    `ks`.  Slew axis geometric 2..200 ps, cap axis geometric 0.5..100 fF, so
    the generated slews (5..100 ps) and caps (1..50 fF) stay inside the axes.
    LUT entries are fJ-scale, positive and monotone in slew and cap, and not
    bilinear (a sqrt term), per (cell, state, input pin):
        f = e0 + e1*s + e2*c + e3*s*c + e4*sqrt(s),  s = slew/100ps, c = cap/10fF,
    with e_i ~ U(0.1, 1) fJ.  Leakage per (cell, state) ~ U(1e-9, 1e-7) W.
    The gate arrays are left empty; callers fill them."""
    ks = sorted(set(int(k) for k in ks))
    cell_n_in = np.array([k for k in ks for _ in range(cells_per_k)], dtype=np.int32)
    n_cells = len(cell_n_in)
    slew_axis = np.geomspace(2 * PS, 200 * PS, n_axis)
    cap_axis = np.geomspace(0.5 * FF, 100 * FF, n_axis)
    slew_axes = np.tile(slew_axis, (n_cells, 1))
    cap_axes = np.tile(cap_axis, (n_cells, 1))
    s_hat = (slew_axis / (100 * PS))[:, None]
    c_hat = (cap_axis / (10 * FF))[None, :]
    luts, leaks = [], []
    for k in cell_n_in:
        nst = 1 << int(k)
        e = rng.uniform(0.1, 1.0, size=(nst, int(k), 5, 1, 1)) * FJ
        tab = (e[:, :, 0] + e[:, :, 1] * s_hat + e[:, :, 2] * c_hat + e[:, :, 3] * s_hat * c_hat
               + e[:, :, 4] * np.sqrt(s_hat))
        luts.append(tab.reshape(-1))
        leaks.append(rng.uniform(1e-9, 1e-7, size=nst))
    return Design(gate_cell=np.zeros(0, np.int32), gate_cap_F=np.zeros(0), cell_n_in=cell_n_in,
                  n_slew=n_axis, n_cap=n_axis, slew_axis=slew_axes, cap_axis=cap_axes,
                  lut_J=np.concatenate(luts).astype(np.float64),
                  leak_W=np.concatenate(leaks).astype(np.float64), vdd_V=0.8)


def assign_gates(rng: np.random.Generator, lib: Design, k_of_gate: np.ndarray, cap_ff_lo: float,
                 cap_ff_hi: float) -> Design:
    cells_by_k = {int(k): np.flatnonzero(lib.cell_n_in == k) for k in np.unique(lib.cell_n_in)}
    gate_cell = np.empty(k_of_gate.shape[0], dtype=np.int32)
    for k, cells in cells_by_k.items():
        sel = np.flatnonzero(k_of_gate == k)
        gate_cell[sel] = rng.choice(cells, size=sel.shape[0])
    cap = rng.uniform(cap_ff_lo, cap_ff_hi, size=k_of_gate.shape[0]) * FF
    return dataclasses.replace(lib, gate_cell=gate_cell, gate_cap_F=cap.astype(np.float64))


# ---------------------------------------------------------------- events --

def _finish_trace(rng: np.random.Generator, n_pins: int, pin_of: np.ndarray, t: np.ndarray, t_clk: int,
                  t_max: int) -> Trace:
    """Sort (pin, t), drop exact duplicates on a pin, draw init values and
    slews, and derive alternating values."""
    key = pin_of.astype(np.int64) * np.int64(t_max) + t.astype(np.int64)
    del pin_of, t
    key.sort(kind="stable")
    if key.shape[0] > 1:
        keep = np.empty(key.shape[0], dtype=bool)
        keep[0] = True
        np.not_equal(key[1:], key[:-1], out=keep[1:])
        key = key[keep]
        del keep
    pin = key // np.int64(t_max)
    evt_t = key - pin * np.int64(t_max)
    del key
    counts = np.bincount(pin, minlength=n_pins).astype(np.int64)
    pin_ptr = np.zeros(n_pins + 1, dtype=np.int64)
    np.cumsum(counts, out=pin_ptr[1:])
    pin_init = rng.integers(0, 2, size=n_pins, dtype=np.uint8)
    idx = np.arange(evt_t.shape[0], dtype=np.int64) - pin_ptr[pin]
    evt_val = (pin_init[pin] ^ ((idx + 1) & 1).astype(np.uint8)).astype(np.uint8)
    del idx, pin
    evt_slew = rng.uniform(5 * PS, 100 * PS, size=evt_t.shape[0]).astype(np.float32)
    return Trace(pin_ptr=pin_ptr, pin_init=pin_init, evt_t=evt_t, evt_val=evt_val, evt_slew=evt_slew,
                 t_clk=int(t_clk), t_max=int(t_max))


def poisson_trace(rng: np.random.Generator, rate_per_pin_cycle: np.ndarray, n_cycles: int, t_clk: int,
                  extra_pin: Optional[np.ndarray] = None, extra_t: Optional[np.ndarray] = None) -> Trace:
    """Per-pin Poisson processes: N_p ~ Poisson(rate_p * n_cycles), event times
    uniform on [0, t_max) in integer ticks.  Optional extra (pin, t) events are
    merged in before sorting."""
    t_max = int(n_cycles) * int(t_clk)
    n_pins = rate_per_pin_cycle.shape[0]
    n_per_pin = rng.poisson(rate_per_pin_cycle * n_cycles)
    pin_of = np.repeat(np.arange(n_pins, dtype=np.int64), n_per_pin)
    t = rng.integers(0, t_max, size=pin_of.shape[0], dtype=np.int64)
    if extra_pin is not None:
        pin_of = np.concatenate([pin_of, extra_pin.astype(np.int64)])
        t = np.concatenate([t, extra_t.astype(np.int64)])
    return _finish_trace(rng, n_pins, pin_of, t, t_clk, t_max)


# --------------------------------------------------------------- configs --

def _scaled(rates: np.ndarray, target_events: float, n_cycles: int) -> np.ndarray:
    return rates * (target_events / (rates.sum() * n_cycles))


def tiny(seed: int = 0) -> Workload:
    """1,000 two-input gates (4 states, 7x7 LUTs), 200 cycles of 1 ns, Poisson
    0.1 events/pin/cycle (~60k events), slews 5-100 ps, caps 1-20 fF, Vdd 0.8 V."""
    rng = np.random.default_rng(seed)
    lib = make_library(rng, [2])
    G, C, T = 1000, 200, NS
    des = assign_gates(rng, lib, np.full(G, 2, np.int64), 1.0, 20.0)
    P = int(des.pin_base()[-1])
    tr = poisson_trace(rng, np.full(P, 0.1), C, T)
    return Workload("tiny", des, tr, {"nominal_rate": 0.1, "effective_rate": 0.1})


def uniform_mixed(name: str, seed: int, G: int, C: int, T: int, target_events: float, n_axis: int = 7,
                  nominal_rate: float = 0.01) -> Workload:
    rng = np.random.default_rng(seed)
    lib = make_library(rng, [1, 2, 3, 4], n_axis=n_axis)
    k = rng.integers(1, 5, size=G)
    des = assign_gates(rng, lib, k, 1.0, 50.0)
    P = int(des.pin_base()[-1])
    rates = _scaled(np.full(P, nominal_rate), target_events, C)
    tr = poisson_trace(rng, rates, C, T)
    return Workload(name, des, tr, {"nominal_rate": nominal_rate, "effective_rate": float(rates[0])})


def medium(seed: int = 0) -> Workload:
    """100,000 gates with 1-4 inputs (2^k states, 7x7 LUTs), 10,000 cycles of
    1 ns, uniform activity scaled so the expected total is 10M events
    (nominal 0.01/pin/cycle, effective ~0.00286), caps 1-50 fF."""
    return uniform_mixed("medium", seed, 100_000, 10_000, NS, 10e6)


def skewed(seed: int = 0) -> Workload:
    """200,000 gates (1-4 inputs), 10,000 cycles of 1 ns; per-gate activity
    ~ Pareto(alpha=1.2) split evenly over the gate's pins, scaled to an
    expected 20M events (top 1% of gates hold ~46% of events)."""
    rng = np.random.default_rng(seed)
    G, C, T = 200_000, 10_000, NS
    lib = make_library(rng, [1, 2, 3, 4])
    k = rng.integers(1, 5, size=G)
    des = assign_gates(rng, lib, k, 1.0, 50.0)
    gate_rate = rng.pareto(1.2, size=G) + 1.0
    pin_rate = np.repeat(gate_rate / (k + 1), k + 1)
    rates = _scaled(pin_rate, 20e6, C)
    tr = poisson_trace(rng, rates, C, T)
    return Workload("skewed", des, tr, {"pareto_alpha": 1.2})


def glitch_heavy(seed: int = 0) -> Workload:
    """100,000 four-input gates (16 states), 5,000 cycles of 1 ns, ~15M
    events: 70% background Poisson, 30% in clusters of m ~ U{2,3,4}
    transitions on one random pin inside one random cycle, with gaps
    ~ U(10, 300) ps and a start drawn so the cluster ends inside the cycle."""
    rng = np.random.default_rng(seed)
    G, C, T = 100_000, 5_000, NS
    lib = make_library(rng, [4])
    des = assign_gates(rng, lib, np.full(G, 4, np.int64), 1.0, 50.0)
    P = int(des.pin_base()[-1])
    total = 15e6
    clustered = 0.3 * total
    n_clusters = int(round(clustered / 3.0))
    m = rng.integers(2, 5, size=n_clusters)
    c_pin = rng.integers(0, P, size=n_clusters)
    c_cyc = rng.integers(0, C, size=n_clusters)
    gaps = rng.integers(10 * PS, 300 * PS + 1, size=(n_clusters, 3))
    gaps = np.where(np.arange(3)[None, :] < (m - 1)[:, None], gaps, 0)
    span = gaps.sum(axis=1)
    start = c_cyc * T + (rng.random(n_clusters) * (T - span)).astype(np.int64)
    offs = np.concatenate([np.zeros((n_clusters, 1), np.int64), np.cumsum(gaps, axis=1)], axis=1)
    valid = np.arange(4)[None, :] < m[:, None]
    ex_t = (start[:, None] + offs)[valid]
    ex_pin = np.repeat(c_pin, m)
    rates = np.full(P, (total - clustered) / (P * C))
    tr = poisson_trace(rng, rates, C, T, extra_pin=ex_pin, extra_t=ex_t)
    return Workload("glitch_heavy", des, tr, {"clusters": n_clusters})


def large(seed: int = 0) -> Workload:
    """2,000,000 gates (1-4 inputs, 8x8 LUTs), 20,000 cycles of 0.5 ns; per-pin
    activity lognormal (mean 0.005/pin/cycle, sigma 1) scaled to ~200M events."""
    rng = np.random.default_rng(seed)
    G, C, T = 2_000_000, 20_000, NS // 2
    lib = make_library(rng, [1, 2, 3, 4], n_axis=8)
    k = rng.integers(1, 5, size=G)
    des = assign_gates(rng, lib, k, 1.0, 50.0)
    P = int(des.pin_base()[-1])
    sigma = 1.0
    rates = rng.lognormal(math.log(0.005) - 0.5 * sigma * sigma, sigma, size=P)
    rates = _scaled(rates, 200e6, C)
    tr = poisson_trace(rng, rates, C, T)
    return Workload("large", des, tr, {"lognormal_sigma": sigma})


def toggle_trace(rng: np.random.Generator, n_pins: int, n_cycles: int, t_clk: int, m: int) -> Trace:
    """Every pin toggles m times in every clock cycle: the cycle is cut into m
    equal slots and toggle j falls uniformly inside slot j, so the times of a
    pin are strictly increasing.  Values alternate from a random initial
    value; slews ~ U(5, 100) ps."""
    slot = t_clk // m
    per_pin = n_cycles * m
    grid = (np.arange(n_cycles, dtype=np.int64)[:, None] * t_clk
            + np.arange(m, dtype=np.int64)[None, :] * slot).reshape(-1)
    evt_t = rng.integers(0, slot, size=(n_pins, per_pin), dtype=np.int64)
    evt_t += grid[None, :]
    evt_t = evt_t.reshape(-1)
    pin_ptr = np.arange(n_pins + 1, dtype=np.int64) * per_pin
    pin_init = rng.integers(0, 2, size=n_pins, dtype=np.uint8)
    alt = np.resize(np.array([1, 0], dtype=np.uint8), per_pin)  # toggle i gives !init for even i
    evt_val = (np.tile(alt, n_pins) ^ np.repeat(pin_init, per_pin)).astype(np.uint8)
    evt_slew = rng.random(evt_t.shape[0], dtype=np.float32)
    evt_slew *= np.float32(95 * PS)
    evt_slew += np.float32(5 * PS)
    return Trace(pin_ptr=pin_ptr, pin_init=pin_init, evt_t=evt_t, evt_val=evt_val, evt_slew=evt_slew,
                 t_clk=int(t_clk), t_max=int(n_cycles) * int(t_clk))


def contention(m: int, seed: int = 0, G: int = 32, C: int = 100_000) -> Workload:
    """Waveform-bin stress: 32 two-input gates (96 pins), 100,000 cycles of
    1 ns, every pin toggling m times per cycle (m = 1, 2, 4, 8: 9.6M to
    76.8M events, 96 m events in every waveform bin).  Every event of a cycle lands in the same waveform bin and
    every toggle after a pin's first in a cycle is a glitch, so this is the
    worst case for the per-bin accumulation (the paper's atomic stress test
    on high-activity synthetic waveforms, in its evaluation of the
    waveform-bin atomic overhead)."""
    rng = np.random.default_rng(seed)
    lib = make_library(rng, [2])
    des = assign_gates(rng, lib, np.full(G, 2, np.int64), 1.0, 50.0)
    P = int(des.pin_base()[-1])
    tr = toggle_trace(rng, P, C, NS, m)
    return Workload(f"contention{m}", des, tr, {"toggles_per_cycle": m})


CONFIGS = {"tiny": tiny, "medium": medium, "skewed": skewed, "glitch_heavy": glitch_heavy, "large": large,
           "contention1": lambda seed=0: contention(1, seed), "contention2": lambda seed=0: contention(2, seed),
           "contention4": lambda seed=0: contention(4, seed), "contention8": lambda seed=0: contention(8, seed)}


def make(name: str, seed: int = 0) -> Workload:
    return CONFIGS[name](seed)


def subset_gates(w: Workload, g_lo: int, g_hi: int) -> Workload:
    """The sub-design made of gates [g_lo, g_hi) with their pins and events
    (same library, same clock and window)."""
    d, t = w.design, w.trace
    pb = d.pin_base()
    p_lo, p_hi = int(pb[g_lo]), int(pb[g_hi])
    e_lo, e_hi = int(t.pin_ptr[p_lo]), int(t.pin_ptr[p_hi])
    des = dataclasses.replace(d, gate_cell=d.gate_cell[g_lo:g_hi].copy(), gate_cap_F=d.gate_cap_F[g_lo:g_hi].copy())
    tr = dataclasses.replace(t, pin_ptr=(t.pin_ptr[p_lo:p_hi + 1] - e_lo).copy(),
                             pin_init=t.pin_init[p_lo:p_hi].copy(), evt_t=t.evt_t[e_lo:e_hi].copy(),
                             evt_val=t.evt_val[e_lo:e_hi].copy(), evt_slew=t.evt_slew[e_lo:e_hi].copy())
    return Workload(f"{w.name}[{g_lo}:{g_hi}]", des, tr, dict(w.info))


def select_gates(w: Workload, gates) -> Workload:
    """The sub-design made of the given gates (in increasing order) with their
    pins and events (same library, clock and window)."""
    d, t = w.design, w.trace
    gates = np.unique(np.asarray(gates, dtype=np.int64))
    pb = d.pin_base()
    npin = pb[gates + 1] - pb[gates]
    pins = np.repeat(pb[gates], npin) + (np.arange(int(npin.sum())) - np.repeat(np.cumsum(npin) - npin, npin))
    cnt = t.pin_ptr[pins + 1] - t.pin_ptr[pins]
    ptr = np.zeros(pins.shape[0] + 1, dtype=np.int64)
    np.cumsum(cnt, out=ptr[1:])
    ev = np.repeat(t.pin_ptr[pins], cnt) + (np.arange(int(cnt.sum())) - np.repeat(ptr[:-1], cnt))
    des = dataclasses.replace(d, gate_cell=d.gate_cell[gates].copy(), gate_cap_F=d.gate_cap_F[gates].copy())
    tr = dataclasses.replace(t, pin_ptr=ptr, pin_init=t.pin_init[pins].copy(), evt_t=t.evt_t[ev].copy(),
                             evt_val=t.evt_val[ev].copy(), evt_slew=t.evt_slew[ev].copy())
    return Workload(f"{w.name}[{gates.shape[0]} gates]", des, tr, dict(w.info))
