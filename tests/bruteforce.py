"""Independent numpy/scipy formulations used to pin the CPU oracle.

Nothing here shares code with the oracle (pa_oracle.c) or with the HIP
library.  Each function restates one part of the method in a different
formulation from the oracle's per-gate time-ordered walk:
  - glitch flags/counts from per-(pin, cycle) event counts (bincount);
  - states before events from sorted-key searches (searchsorted), not a merge;
  - internal energies from scipy's RegularGridInterpolator, not hand bilerp;
  - leakage by summing the state of every single tick (tiny windows only).
The method follows "GPU-Accelerated Gate-Level Time-Based Power Analysis via
Event-Density-Aware Partitioning and Kernel Fusion" (Sec. 2.4.1, 2.4.2,
Eqs. 1-4, Figs. 2, 3, 7).
"""
import numpy as np
from scipy.interpolate import RegularGridInterpolator


def event_pins(trace):
    counts = np.diff(trace.pin_ptr)
    return np.repeat(np.arange(trace.n_pins, dtype=np.int64), counts)


def pin_roles(design):
    """For every pin: its gate, its index inside the gate, and whether it is the output."""
    k = design.gate_k()
    pb = design.pin_base()
    P = int(pb[-1])
    gate_of_pin = np.repeat(np.arange(design.n_gates, dtype=np.int64), k + 1)
    local = np.arange(P, dtype=np.int64) - pb[gate_of_pin]
    is_out = local == k[gate_of_pin]
    return gate_of_pin, local, is_out


def glitch_flags(trace):
    """Event e is a glitch iff the previous event on its pin falls in the same
    clock cycle (a running per-pin count of 2 or more inside the cycle)."""
    pin = event_pins(trace)
    cyc = trace.evt_t // trace.t_clk
    flag = np.zeros(trace.n_events, np.uint8)
    if trace.n_events > 1:
        same = (pin[1:] == pin[:-1]) & (cyc[1:] == cyc[:-1])
        flag[1:] = same
    return flag


def glitch_count(trace):
    """sum over (pin, cycle) of max(0, n - 1), via one bincount."""
    pin = event_pins(trace)
    ncyc = trace.n_cycles
    key = pin * ncyc + trace.evt_t // trace.t_clk
    _, n = np.unique(key, return_counts=True)
    return int(np.maximum(n - 1, 0).sum())


def cycle_counts(trace):
    cyc = trace.evt_t // trace.t_clk
    return np.bincount(cyc, minlength=trace.n_cycles).astype(np.uint64)


def state_before(design, trace):
    """S(t-) for every input-pin event (0 for output-pin events): bit j is the
    value of input pin j just before t = init_j xor parity(#events on pin j
    strictly before t)."""
    pin = event_pins(trace)
    gate_of_pin, local, is_out = pin_roles(design)
    pb = design.pin_base()
    k = design.gate_k()
    keys = pin * np.int64(trace.t_max) + trace.evt_t  # globally sorted (pin-major, t ascending)
    g = gate_of_pin[pin]
    S = np.zeros(trace.n_events, np.int64)
    for j in range(int(k.max()) if k.size else 0):
        has = j < k[g]
        pj = np.where(has, pb[g] + j, 0)
        before = np.searchsorted(keys, pj * np.int64(trace.t_max) + trace.evt_t, side="left") - trace.pin_ptr[pj]
        vj = trace.pin_init[pj].astype(np.int64) ^ (before & 1)
        S += np.where(has, vj << j, 0)
    S[is_out[pin]] = 0
    return S.astype(np.uint8)


def dynamic(design, trace):
    """Per-event dynamic energy and its split into internal / switching /
    glitch, and the dynamic part of the per-cycle waveform."""
    pin = event_pins(trace)
    gate_of_pin, local, is_out = pin_roles(design)
    g = gate_of_pin[pin]
    i = local[pin]
    out = is_out[pin]
    cell = design.gate_cell[g].astype(np.int64)
    kk = design.cell_n_in[cell].astype(np.int64)
    cap = design.gate_cap_F[g]
    slew = trace.evt_slew.astype(np.float64)
    S = state_before(design, trace).astype(np.int64)
    E = np.zeros(trace.n_events)
    # switching: 0->1 on the output pin
    E[out] = np.where(trace.evt_val[out] == 1, 0.5 * cap[out] * design.vdd_V ** 2, 0.0)
    # internal: interpolate the (cell, state, pin) table with scipy
    lb = design.lut_base()
    ns, nc = design.n_slew, design.n_cap
    inp = np.flatnonzero(~out)
    grp = (cell[inp] * 256 + S[inp]) * 16 + i[inp]
    order = np.argsort(grp, kind="stable")
    uniq, starts = np.unique(grp[order], return_index=True)
    bounds = list(starts) + [order.shape[0]]
    for u in range(uniq.shape[0]):
        ev = inp[order[bounds[u]:bounds[u + 1]]]
        c, s, ii = int(cell[ev[0]]), int(S[ev[0]]), int(i[ev[0]])
        k_c = int(design.cell_n_in[c])
        base = lb[c] + (s * k_c + ii) * ns * nc
        tab = design.lut_J[base:base + ns * nc].reshape(ns, nc)
        f = RegularGridInterpolator((design.slew_axis[c], design.cap_axis[c]), tab, method="linear",
                                    bounds_error=False, fill_value=None)
        E[ev] = f(np.stack([slew[ev], cap[ev]], axis=1))
    flag = glitch_flags(trace).astype(bool)
    r = np.zeros(trace.n_events)
    idx = np.flatnonzero(flag)
    pw = (trace.evt_t[idx] - trace.evt_t[idx - 1]).astype(np.float64)
    r[idx] = np.minimum(1.0, pw / (0.5 * (slew[idx] + slew[idx - 1])))
    contrib = np.where(flag, r * E, E)
    cyc = trace.evt_t // trace.t_clk
    wave = np.bincount(cyc, weights=contrib, minlength=trace.n_cycles)
    G = design.n_gates
    gate_dyn = np.stack([np.bincount(g, weights=np.where(~out & ~flag, E, 0.0), minlength=G),
                         np.bincount(g, weights=np.where(out & ~flag, E, 0.0), minlength=G),
                         np.bincount(g, weights=np.where(flag, r * E, 0.0), minlength=G)], axis=1)
    return dict(E=E, e_int=float(E[~out & ~flag].sum()), e_sw=float(E[out & ~flag].sum()),
                e_gl=float((r * E)[flag].sum()), wave_dyn=wave, gate_dyn=gate_dyn, _kk=kk)


def leakage_per_tick(design, trace, per_gate=False):
    """Leakage by brute force over every tick of a tiny window: the energy of
    tick x is leak[cell][S(x)] * tick_s where S(x) holds after all events at
    times <= x.  Returns (e_leak, per-cycle leakage bins), plus every gate's
    leakage energy when per_gate."""
    assert trace.t_max <= 200_000, "per-tick brute force is for tiny windows"
    ticks = np.arange(trace.t_max, dtype=np.int64)
    k = design.gate_k()
    pb = design.pin_base()
    kb = design.leak_base()
    ncyc = trace.n_cycles
    bins_ticks = np.zeros(ncyc)
    total = 0.0
    gate_total = np.zeros(design.n_gates)
    cyc_of_tick = ticks // trace.t_clk
    for g in range(design.n_gates):
        S = np.zeros(trace.t_max, np.int64)
        for j in range(int(k[g])):
            p = pb[g] + j
            times = trace.evt_t[trace.pin_ptr[p]:trace.pin_ptr[p + 1]]
            n_le = np.searchsorted(times, ticks, side="right")
            S |= (int(trace.pin_init[p]) ^ (n_le & 1)) << j
        p_tick = design.leak_W[kb[design.gate_cell[g]] + S]
        # integer tick counts per (bin, state) times the power, i.e. one multiply per term
        per_bin = np.bincount(cyc_of_tick, weights=p_tick, minlength=ncyc)
        bins_ticks += per_bin
        gate_total[g] = p_tick.sum()
        total += gate_total[g]
    if per_gate:
        return total * trace.tick_s, bins_ticks * trace.tick_s, gate_total * trace.tick_s
    return total * trace.tick_s, bins_ticks * trace.tick_s
