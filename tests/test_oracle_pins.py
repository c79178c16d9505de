"""Pins for the CPU oracle, against values and formulations that do not come
from the oracle itself: hand-worked circuits (tests/golden), closed forms,
textbook/library interpolation (scipy), brute force over ticks and over
(pin, cycle) counts, and invariants of the method.

Method: "GPU-Accelerated Gate-Level Time-Based Power Analysis via
Event-Density-Aware Partitioning and Kernel Fusion" (Sec. 2.4.1, 2.4.2,
Eqs. 1-4, Figs. 2, 3, 7).
"""
import dataclasses
import math

import numpy as np
import pytest
from scipy.interpolate import RegularGridInterpolator

import bruteforce as bf
import golden_util
from workloads import synth

REL_HAND = 1e-12


def _close(a, b, rel=REL_HAND, abs_=1e-30):
    return abs(a - b) <= max(rel * max(abs(a), abs(b)), abs_)


@pytest.mark.parametrize("path", golden_util.fixtures(), ids=lambda p: p.split("/")[-1])
def test_hand_circuit(oracle_lib, path):
    spec, d, t = golden_util.load(path)
    r = oracle_lib.run(d, t)
    exp = spec["expect"]
    for key in ("e_int_J", "e_sw_J", "e_gl_J", "e_leak_J", "p_int_W", "p_leak_W"):
        if key in exp:
            assert _close(r[key], exp[key]), (key, r[key], exp[key])
    np.testing.assert_allclose(r["wave_J"], exp["wave_J"], rtol=REL_HAND, atol=1e-30)
    assert r["cyc_events"].tolist() == exp["cyc_events"]
    assert r["cyc_glitches"].tolist() == exp["cyc_glitches"]
    assert r["evt_glitch"].tolist() == exp["evt_glitch"]
    assert r["evt_state_before"].tolist() == exp["evt_state_before"]
    assert r["n_events"] == exp["n_events"] and r["n_glitches"] == exp["n_glitches"]
    window = t.t_max * t.tick_s
    for comp in ("int", "sw", "gl", "leak"):
        assert _close(r[f"p_{comp}_W"], r[f"e_{comp}_J"] / window)


# ------------------------------------------------------------ bilinear --

def _rand_table(rng, ns=7, nc=7):
    sa = np.sort(rng.uniform(1.0, 100.0, ns)) + np.arange(ns)
    ca = np.sort(rng.uniform(0.1, 10.0, nc)) + np.arange(nc) * 0.1
    tab = rng.uniform(0.1, 1.0, (ns, nc))
    return sa, ca, tab


def test_bilerp_grid_points_exact(oracle_lib):
    rng = np.random.default_rng(1)
    sa, ca, tab = _rand_table(rng)
    for i in range(sa.shape[0]):
        for j in range(ca.shape[0]):
            assert oracle_lib.bilerp(sa, ca, tab, sa[i], ca[j]) == tab[i, j]


def test_bilerp_reproduces_bilinear_function(oracle_lib):
    """A table sampled from f = a + b s + c x + d s x is reproduced at any
    query, inside the axes or extrapolated (linear extrapolation)."""
    rng = np.random.default_rng(2)
    sa, ca, _ = _rand_table(rng)
    a, b, c, d = rng.uniform(-1, 1, 4)
    f = lambda s, x: a + b * s + c * x + d * s * x
    tab = f(sa[:, None], ca[None, :])
    qs = np.concatenate([rng.uniform(sa[0], sa[-1], 200), rng.uniform(sa[0] - 30, sa[0], 20),
                         rng.uniform(sa[-1], sa[-1] + 30, 20)])
    qc = np.concatenate([rng.uniform(ca[0], ca[-1], 200), rng.uniform(ca[-1], ca[-1] + 5, 20),
                         rng.uniform(ca[0] - 5, ca[0], 20)])
    for s, x in zip(qs, qc):
        assert abs(oracle_lib.bilerp(sa, ca, tab, s, x) - f(s, x)) <= 1e-12 * (1 + abs(f(s, x)))


def test_bilerp_matches_scipy(oracle_lib):
    rng = np.random.default_rng(3)
    sa, ca, tab = _rand_table(rng)
    rgi = RegularGridInterpolator((sa, ca), tab, method="linear", bounds_error=False, fill_value=None)
    qs = np.concatenate([rng.uniform(sa[0], sa[-1], 300), rng.uniform(sa[-1], sa[-1] + 20, 30)])
    qc = np.concatenate([rng.uniform(ca[0], ca[-1], 300), rng.uniform(ca[0] - 2, ca[0], 30)])
    ref = rgi(np.stack([qs, qc], 1))
    got = np.array([oracle_lib.bilerp(sa, ca, tab, s, x) for s, x in zip(qs, qc)])
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-15)


# ------------------------------------------------- closed forms, brute force --

def _small_random(seed, G=40, C=20, T=1000, rate=0.3, ks=(1, 2, 3, 4)):
    """A small random workload whose window is short enough for per-tick
    brute force (t_max = C * T ticks)."""
    rng = np.random.default_rng(seed)
    lib = synth.make_library(rng, ks, cells_per_k=2, n_axis=5)
    k = rng.choice(np.array(ks), size=G)
    des = synth.assign_gates(rng, lib, k, 1.0, 50.0)
    P = int(des.pin_base()[-1])
    tr = synth.poisson_trace(rng, np.full(P, rate), C, T)
    # slews of the order of the clock so that r_gl takes values below and at 1
    tr = dataclasses.replace(tr, evt_slew=rng.uniform(50, 900, tr.n_events).astype(np.float32))
    return des, tr


def test_constant_state_gate_closed_form(oracle_lib):
    """A gate whose input pins never switch leaks leak[S0] over the whole
    window: E_leak = leak * t_max * tick_s, every full bin without output
    events gets leak * T * tick_s, and the partial last bin gets leak times
    its length (Sec. 2.4.2, Eq. 4; leakage is always present)."""
    rng = np.random.default_rng(5)
    lib = synth.make_library(rng, (1, 2, 3, 4), cells_per_k=2, n_axis=5)
    G, T, C = 30, 997, 13
    des = synth.assign_gates(rng, lib, rng.integers(1, 5, G), 1.0, 50.0)
    _, _, is_out = bf.pin_roles(des)
    t_max = C * T - 300  # the last bin is partial
    rates = np.where(is_out, 0.5, 0.0)  # only output pins switch
    tr = synth.poisson_trace(rng, rates, C, T)
    tr = dataclasses.replace(tr, t_max=t_max)
    keep = tr.evt_t < t_max
    pin = bf.event_pins(tr)[keep]
    counts = np.bincount(pin, minlength=tr.n_pins)
    pp = np.zeros(tr.n_pins + 1, np.int64)
    pp[1:] = np.cumsum(counts)
    tr = dataclasses.replace(tr, pin_ptr=pp, evt_t=tr.evt_t[keep], evt_val=tr.evt_val[keep],
                             evt_slew=tr.evt_slew[keep])
    kb, pb, k = des.leak_base(), des.pin_base(), des.gate_k()
    n_full = t_max // T
    for g in range(G):
        r = oracle_lib.run(des, tr, g, g + 1)
        S0 = sum(int(tr.pin_init[pb[g] + j]) << j for j in range(int(k[g])))
        leak = des.leak_W[kb[des.gate_cell[g]] + S0]
        assert r["e_int_J"] == 0.0
        assert _close(r["e_leak_J"], leak * t_max * tr.tick_s)
        out_pin = pb[g] + k[g]
        busy = set((tr.evt_t[pp[out_pin]:pp[out_pin + 1]] // T).tolist())
        for c in range(n_full + 1):
            if c in busy:
                continue
            length = T if c < n_full else t_max - n_full * T
            assert _close(r["wave_J"][c], leak * length * tr.tick_s), (g, c)


@pytest.mark.parametrize("seed", [11, 12, 13])
def test_leakage_matches_per_tick_bruteforce(oracle_lib, seed):
    des, tr = _small_random(seed)
    r = oracle_lib.run(des, tr)
    e_leak, bins = bf.leakage_per_tick(des, tr)
    assert _close(r["e_leak_J"], e_leak, rel=1e-11)
    dyn = bf.dynamic(des, tr)
    np.testing.assert_allclose(r["wave_J"], bins + dyn["wave_dyn"], rtol=1e-11)


@pytest.mark.parametrize("seed", [21, 22])
def test_small_random_dynamic_and_states(oracle_lib, seed):
    des, tr = _small_random(seed, G=60, C=30, T=700, rate=0.6)
    r = oracle_lib.run(des, tr)
    assert r["evt_state_before"].tolist() == bf.state_before(des, tr).tolist()
    assert r["evt_glitch"].tolist() == bf.glitch_flags(tr).tolist()
    dyn = bf.dynamic(des, tr)
    for comp in ("int", "sw", "gl"):
        assert _close(r[f"e_{comp}_J"], dyn[f"e_{comp}"], rel=1e-11), comp
    assert r["n_glitches"] == bf.glitch_count(tr) > 0


@pytest.mark.parametrize("seed", [31, 32])
def test_per_gate_energies_bruteforce(oracle_lib, seed):
    """Every gate's internal, switching, glitch and leakage energy (the
    per-gate output that hotspot ranking uses) against the brute-force
    per-event energies (scipy interpolation) and per-tick leakage, gate by gate."""
    des, tr = _small_random(seed, G=40, C=25, T=800, rate=0.5)
    r = oracle_lib.run(des, tr, per_gate=True)
    gj = r["gate_J"]
    dyn = bf.dynamic(des, tr)
    _, _, leak_g = bf.leakage_per_tick(des, tr, per_gate=True)
    ref = np.concatenate([dyn["gate_dyn"], leak_g[:, None]], axis=1)
    np.testing.assert_allclose(gj, ref, rtol=1e-11, atol=1e-30)
    assert np.all(gj[:, 3] > 0) and np.count_nonzero(gj[:, 2]) > 0


@pytest.fixture(scope="module")
def tiny_run(oracle_lib):
    w = synth.tiny()
    return w, oracle_lib.run(w.design, w.trace)


def test_tiny_glitch_count_bruteforce(tiny_run):
    w, r = tiny_run
    assert r["n_glitches"] == bf.glitch_count(w.trace)
    assert r["evt_glitch"].tolist() == bf.glitch_flags(w.trace).tolist()
    cyc = w.trace.evt_t // w.trace.t_clk
    np.testing.assert_array_equal(r["cyc_glitches"], np.bincount(cyc, weights=bf.glitch_flags(w.trace),
                                                                 minlength=w.trace.n_cycles).astype(np.uint64))
    np.testing.assert_array_equal(r["cyc_events"], bf.cycle_counts(w.trace))
    assert r["n_events"] == w.trace.n_events


def test_tiny_states_bruteforce(tiny_run):
    w, r = tiny_run
    np.testing.assert_array_equal(r["evt_state_before"], bf.state_before(w.design, w.trace))


def test_tiny_dynamic_totals_bruteforce(tiny_run):
    w, r = tiny_run
    dyn = bf.dynamic(w.design, w.trace)
    for comp in ("int", "sw", "gl"):
        assert _close(r[f"e_{comp}_J"], dyn[f"e_{comp}"], rel=1e-11), comp


def test_waveform_sums_to_totals(tiny_run):
    w, r = tiny_run
    tot = r["e_int_J"] + r["e_sw_J"] + r["e_gl_J"] + r["e_leak_J"]
    assert _close(float(np.sum(r["wave_J"])), tot, rel=1e-12)
    assert np.all(r["wave_J"] > 0)


def test_gate_subsets_add_up(oracle_lib, tiny_run):
    w, r = tiny_run
    a = oracle_lib.run(w.design, w.trace, 0, 377)
    b = oracle_lib.run(w.design, w.trace, 377, w.design.n_gates)
    for key in ("e_int_J", "e_sw_J", "e_gl_J", "e_leak_J"):
        assert _close(a[key] + b[key], r[key], rel=1e-12)
    np.testing.assert_allclose(a["wave_J"] + b["wave_J"], r["wave_J"], rtol=1e-12)
    assert a["n_glitches"] + b["n_glitches"] == r["n_glitches"]


def test_per_gate_sums_to_totals(oracle_lib, tiny_run):
    w, r = tiny_run
    gj = oracle_lib.run(w.design, w.trace, per_event=False, per_gate=True)["gate_J"]
    for c, key in enumerate(("e_int_J", "e_sw_J", "e_gl_J", "e_leak_J")):
        assert _close(float(gj[:, c].sum()), r[key], rel=1e-12), key
    sub = oracle_lib.run(w.design, w.trace, 100, 101, per_event=False)
    assert [sub[k] for k in ("e_int_J", "e_sw_J", "e_gl_J", "e_leak_J")] == gj[100].tolist()


@pytest.mark.parametrize("threads", [1, 2, 7, 64])
def test_threaded_oracle_equals_single_thread(oracle_lib, tiny_run, threads):
    """The threaded driver (contiguous gate ranges on host threads, merged in
    order) against the single-threaded walk: integer outputs, per-event
    outputs and per-gate rows identical; totals and bins equal up to the
    order of the fp64 additions.  Also on a gate sub-range, and with more
    threads than gates."""
    w, r = tiny_run
    m = oracle_lib.run(w.design, w.trace, per_gate=True, threads=threads)
    g1 = oracle_lib.run(w.design, w.trace, per_event=False, per_gate=True)["gate_J"]
    for key in ("e_int_J", "e_sw_J", "e_gl_J", "e_leak_J", "p_int_W", "p_sw_W", "p_gl_W", "p_leak_W"):
        assert _close(m[key], r[key], rel=1e-14), key
    for key in ("n_events", "n_glitches", "n_cycles"):
        assert m[key] == r[key], key
    for key in ("cyc_events", "cyc_glitches", "evt_glitch", "evt_state_before"):
        np.testing.assert_array_equal(m[key], r[key], err_msg=key)
    np.testing.assert_allclose(m["wave_J"], r["wave_J"], rtol=1e-14, atol=0)
    np.testing.assert_array_equal(m["gate_J"], g1)
    a = oracle_lib.run(w.design, w.trace, 123, 321, per_event=False)
    b = oracle_lib.run(w.design, w.trace, 123, 321, per_event=False, threads=threads)
    np.testing.assert_array_equal(a["cyc_events"], b["cyc_events"])
    np.testing.assert_allclose(a["wave_J"], b["wave_J"], rtol=1e-14, atol=0)
    assert _close(a["e_leak_J"], b["e_leak_J"], rel=1e-14) and a["n_glitches"] == b["n_glitches"]
    few = synth.subset_gates(w, 0, 3)
    c = oracle_lib.run(few.design, few.trace, per_event=False)
    d = oracle_lib.run(few.design, few.trace, per_event=False, threads=threads)
    assert _close(c["e_int_J"], d["e_int_J"], rel=1e-14)
    np.testing.assert_array_equal(c["cyc_glitches"], d["cyc_glitches"])


def test_threaded_oracle_rejects_bad_input(oracle_lib):
    des, tr = _small_random(31)
    tt = tr.evt_t.copy()
    tt[-1] = tr.t_max
    with pytest.raises(Exception):
        oracle_lib.run(des, dataclasses.replace(tr, evt_t=tt), threads=4)


@pytest.mark.parametrize("m", [1, 3, 8])
def test_contention_generator_and_glitch_count(oracle_lib, m):
    """The waveform-bin stress trace: every pin toggles exactly m times in
    every cycle, times strictly increasing, values alternating; so every bin
    holds P*m events of which P*(m-1) are glitches, in closed form."""
    w = synth.contention(m, G=5, C=40)
    d, t = w.design, w.trace
    P = t.n_pins
    cyc = t.evt_t // t.t_clk
    pin = bf.event_pins(t)
    assert t.n_events == P * 40 * m
    assert np.all(np.bincount(pin * 40 + cyc, minlength=P * 40) == m)
    for p in range(P):
        tt = t.evt_t[t.pin_ptr[p]:t.pin_ptr[p + 1]]
        assert np.all(np.diff(tt) > 0)
        vv = t.evt_val[t.pin_ptr[p]:t.pin_ptr[p + 1]].astype(int)
        assert vv[0] == 1 - int(t.pin_init[p]) and np.all(vv[1:] != vv[:-1])
    r = oracle_lib.run(d, t, per_event=False)
    assert np.all(r["cyc_events"] == P * m) and np.all(r["cyc_glitches"] == P * (m - 1))
    assert r["n_glitches"] == P * 40 * (m - 1)


def test_tiny_generator_statistics(tiny_run):
    """Tiny draws Poisson(0.1) events per pin-cycle: expected glitches =
    N_pin_cycles * (lambda - 1 + e^-lambda) ~ 2,902, expected events 60,000."""
    w, r = tiny_run
    lam = 0.1
    n_pc = w.trace.n_pins * w.trace.n_cycles
    exp_gl = n_pc * (lam - 1 + math.exp(-lam))
    assert abs(r["n_glitches"] - exp_gl) < 6 * math.sqrt(exp_gl)
    assert abs(w.trace.n_events - 60_000) < 6 * math.sqrt(60_000)


# -------------------------------------------------------------- rejection --

@pytest.mark.parametrize("mutate", ["unsorted", "bad_value", "t_max", "slew", "clock", "pins"])
def test_oracle_rejects_bad_input(oracle_lib, mutate):
    des, tr = _small_random(31)
    pin = bf.event_pins(tr)
    e = int(np.flatnonzero(np.diff(pin) == 0)[0]) + 1  # an event with a predecessor on its pin
    if mutate == "unsorted":
        tt = tr.evt_t.copy(); tt[e] = tt[e - 1]; tr = dataclasses.replace(tr, evt_t=tt)
    elif mutate == "bad_value":
        vv = tr.evt_val.copy(); vv[e] ^= 1; tr = dataclasses.replace(tr, evt_val=vv)
    elif mutate == "t_max":
        tt = tr.evt_t.copy(); tt[-1] = tr.t_max; tr = dataclasses.replace(tr, evt_t=tt)
    elif mutate == "slew":
        ss = tr.evt_slew.copy(); ss[e] = 0.0; tr = dataclasses.replace(tr, evt_slew=ss)
    elif mutate == "clock":
        tr = dataclasses.replace(tr, t_clk=0)
    elif mutate == "pins":
        tr = dataclasses.replace(tr, pin_init=tr.pin_init[:-1], pin_ptr=tr.pin_ptr[:-1])
    with pytest.raises(Exception):
        oracle_lib.run(des, tr)
