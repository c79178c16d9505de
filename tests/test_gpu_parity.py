"""GPU parity: the HIP path through the C ABI against the CPU oracle, element
by element on the same seeded inputs.

Cases: the hand circuits; small random designs over every input count 1..8,
forced same-timestamp collisions and several chunk lengths (results must
not depend on the layout's chunking or the launch grid); edge cases (no
events, one gate, partial last bin, events at t = 0 and t = t_max - 1, a
dense glitch train); and the Tiny, Medium, Skewed and Glitch-heavy workloads
at full size in the default launch configuration.
"""
import dataclasses

import numpy as np
import pytest

import golden_util
import parity_util as pu
from workloads import synth

pytestmark = pytest.mark.gpu


def _oracle(d, t, **kw):
    import oracle

    return oracle.run(d, t, **kw)


def _print_case(name):
    print(f"[case] {name}", flush=True)


@pytest.mark.parametrize("path", golden_util.fixtures(), ids=lambda p: p.split("/")[-1])
def test_hand_circuits(path):
    spec, d, t = golden_util.load(path)
    _print_case(path)
    g = pu.gpu_run(d, t)
    pu.assert_parity(g, _oracle(d, t), label=path)
    exp = spec["expect"]
    for key in ("e_int_J", "e_sw_J", "e_gl_J", "e_leak_J"):
        assert pu.rel_err(g[key], exp[key]) <= 1e-12 or abs(g[key] - exp[key]) < 1e-30, key
    assert g["evt_glitch"].tolist() == exp["evt_glitch"]
    assert g["evt_state_before"].tolist() == exp["evt_state_before"]


def _random(seed, G=200, C=40, T=1000, rate=0.3, ks=(1, 2, 3, 4), collide=0, t_max=None):
    rng = np.random.default_rng(seed)
    lib = synth.make_library(rng, ks, cells_per_k=2, n_axis=5)
    k = rng.choice(np.array(ks), size=G)
    des = synth.assign_gates(rng, lib, k, 1.0, 50.0)
    P = int(des.pin_base()[-1])
    tr = synth.poisson_trace(rng, np.full(P, rate), C, T)
    pin = np.repeat(np.arange(P), np.diff(tr.pin_ptr))
    tt = tr.evt_t
    if collide:
        tt = (tt // collide) * collide
    if t_max is not None:
        tt = np.minimum(tt, t_max - 1)
    tr = synth._finish_trace(rng, P, pin, tt, T, t_max if t_max is not None else C * T)
    tr = dataclasses.replace(tr, evt_slew=rng.uniform(50, 900, tr.n_events).astype(np.float32))
    return des, tr


RANDOM_CASES = [
    dict(seed=1),
    dict(seed=2, ks=(5, 6, 7, 8), G=60, rate=0.2),
    dict(seed=3, collide=50, rate=0.8, G=120),
    dict(seed=4, collide=1000, rate=0.6, G=80),  # events on cycle boundaries
    dict(seed=5, t_max=39 * 1000 + 217),  # partial last bin
    dict(seed=6, G=3000, C=300, rate=0.05),
]


@pytest.mark.parametrize("case", RANDOM_CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
@pytest.mark.parametrize("chunk", [0, 1, 3, 16])
def test_random_designs_any_chunking(case, chunk):
    d, t = _random(**case)
    _print_case(f"random {case} chunk {chunk}")
    o = _oracle(d, t)
    g = pu.gpu_run(d, t, chunk_cycles=chunk)
    pu.assert_parity(g, o, label=f"{case} chunk {chunk}")
    if chunk:
        pow2 = 1
        while pow2 * 2 <= chunk:
            pow2 *= 2
        assert g["_info"]["chunk_cycles"] == pow2


@pytest.mark.parametrize("grid", [1, 3, 64, 256])
def test_launch_grid_does_not_change_results(grid):
    d, t = _random(seed=7, G=2000, C=200, rate=0.1)
    _print_case(f"grid {grid}")
    pu.assert_parity(pu.gpu_run(d, t, grid_blocks=grid), _oracle(d, t), label=f"grid {grid}")


@pytest.mark.parametrize("n_fix", [1, 4, 32])
def test_fixed_windows_do_not_change_results(n_fix):
    """Fixed-length windows (the layout the paper's density-aware windows
    replace) give the same results; with one-cycle windows every (gate,
    cycle, pin kind) run is a window (a gate's input events and its output
    events go to windows of their own), so the window count is the number of
    such runs."""
    import eda_gate_level_amd as pa

    d, t = _random(seed=9, G=400, C=120, rate=0.3)
    _print_case(f"fixed windows {n_fix}")
    pu.assert_parity(pu.gpu_run(d, t, fixed_window_cycles=n_fix), _oracle(d, t), label=f"fixed {n_fix}")
    an = pa.PowerAnalysis(fixed_window_cycles=n_fix)
    try:
        an.load(d, t)
        st = an.window_stats()
    finally:
        an.close()
    pb = d.pin_base()
    gate = np.repeat(np.repeat(np.arange(d.n_gates), np.diff(pb)), np.diff(t.pin_ptr))
    pin = np.repeat(np.arange(t.n_pins), np.diff(t.pin_ptr))
    is_out = (pin == pb[1:][gate] - 1).astype(np.int64)  # the gate's last pin is its output
    run = (gate.astype(np.int64) * t.n_cycles + t.evt_t // t.t_clk) * 2 + is_out
    if n_fix == 1:
        assert st["n_windows"] == np.unique(run).shape[0]
        assert st["max"] == np.bincount(np.unique(run, return_inverse=True)[1]).max()
    assert st["p50"] <= st["p90"] <= st["p99"] <= st["max"]
    assert abs(st["mean"] * st["n_windows"] - t.n_events) < 1e-6 * t.n_events


def _many_cells(seed, cells_per_k, ks, G, C, rate, n_axis=5):
    rng = np.random.default_rng(seed)
    lib = synth.make_library(rng, ks, cells_per_k=cells_per_k, n_axis=n_axis)
    k = rng.choice(np.array(ks), size=G)
    des = synth.assign_gates(rng, lib, k, 1.0, 50.0)
    tr = synth.poisson_trace(rng, np.full(int(des.pin_base()[-1]), rate), C, 1000)
    return des, dataclasses.replace(tr, evt_slew=rng.uniform(50, 900, tr.n_events).astype(np.float32))


LUT_CASES = {
    "eight-cells": lambda: _random(seed=1),
    "wide-cells": lambda: _random(seed=2, ks=(5, 6, 7, 8), G=60, rate=0.2),  # 8-input LUTs never fit
    "eighty-cells": lambda: _many_cells(11, 40, (1, 2), G=600, C=50, rate=0.3),  # > 8 cells per block
    "tiny-7x7": lambda: (lambda w: (w.design, w.trace))(synth.make("tiny")),
}


@pytest.mark.parametrize("name", list(LUT_CASES))
def test_lut_copies_in_lds(name):
    """Each block copies the LUTs of the cells most of its events use into
    LDS and reads the rest through the caches.  With no copies, with room for
    the smallest tables only, and with all the spare LDS, the results must
    meet the parity bar, in both the plain and the per-event kernels.  The
    event energies are the same arithmetic on the same table values; where
    two settings share the lane layout (the cached and the partly copied
    tables) they are summed in the same order and agree bit for bit, and the
    default setting (the walk kernel, whose layout deals the windows to the
    lanes by its own cost) agrees to rounding.  The bins and the leakage
    built from them are LDS atomics, whose order between waves is free, so
    they match to rounding."""
    d, t = LUT_CASES[name]()
    _print_case(f"lut copies {name}")
    o = _oracle(d, t)
    for per_event in (False, True):
        ref = None
        for kib in (-1, 1, 0):
            g = pu.gpu_run(d, t, per_event=per_event, lut_lds_kib=kib)
            pu.assert_parity(g, o, per_event=per_event, label=f"lut {name} {kib} {per_event}")
            if ref is None:
                ref = g
                continue
            same_layout = kib != 0
            for key in ("e_int_J", "e_sw_J", "e_gl_J"):
                if same_layout:
                    assert g[key] == ref[key], (key, kib, per_event)
                else:
                    assert pu.rel_err(g[key], ref[key]) <= 1e-13, (key, kib, per_event)
            assert g["n_glitches"] == ref["n_glitches"]
            assert pu.rel_err(g["e_leak_J"], ref["e_leak_J"]) <= 1e-13, (kib, per_event)
            np.testing.assert_allclose(g["wave_J"], ref["wave_J"], rtol=1e-13, atol=0)
            assert np.array_equal(g["cyc_events"], ref["cyc_events"])


@pytest.mark.parametrize("name", ["tiny-7x7", "eight-cells"])
def test_event_energies_repeat_bit_for_bit(name):
    """The internal, switching and glitch energies are summed in a fixed
    order (per lane in stream order, then fixed-order reductions), so runs of
    one configuration on the loaded data repeat them bit for bit, as they do
    the integer outputs; the bins and the leakage match to rounding."""
    import eda_gate_level_amd as pa

    d, t = LUT_CASES[name]()
    _print_case(f"repeat {name}")
    an = pa.PowerAnalysis()
    try:
        an.load(d, t)
        r = [an.run() for _ in range(3)]
    finally:
        an.close()
    for x in r[1:]:
        for key in ("e_int_J", "e_sw_J", "e_gl_J", "n_glitches", "n_events"):
            assert x["totals"][key] == r[0]["totals"][key], key
        assert np.array_equal(x["cyc_events"].cpu().numpy(), r[0]["cyc_events"].cpu().numpy())
        assert np.array_equal(x["cyc_glitches"].cpu().numpy(), r[0]["cyc_glitches"].cpu().numpy())
        np.testing.assert_allclose(x["wave_J"].cpu().numpy(), r[0]["wave_J"].cpu().numpy(), rtol=1e-13, atol=0)


def test_load_frees_its_scratch():
    """The event load's scratch (sort keys, indexes, the radix sort's storage)
    and the previous load's buffers are freed when the load returns: loading
    the same events again keeps the footprint, and it stays within the
    events' own arrays (key, slew, caller index: 16 B per slot of the lane
    streams, 4 B per window), the per-block bins and the design."""
    import eda_gate_level_amd as pa

    d, t = _random(seed=12, G=3000, C=300, rate=0.05)
    _print_case("load scratch")
    an = pa.PowerAnalysis()
    try:
        an.load(d, t)
        i1 = an.info()
        an.load(d, t)
        i2 = an.info()
        an.run(per_event=False)
        i3 = an.info()
    finally:
        an.close()
    assert i2["device_bytes"] == i1["device_bytes"] == i3["device_bytes"]
    print(f"events {t.n_events} windows {i1['n_windows']} slots {i1['n_slots']}", flush=True)
    assert t.n_events <= i1["n_slots"] <= 2 * t.n_events + 128 * i1["n_windows"]
    bound = (16 * i1["n_slots"] + 4 * i1["n_windows"] + 16 * i1["grid_blocks"] * i1["chunk_cycles"] + 64 * d.n_gates
             + 16 * int(d.pin_base()[-1]) + d.lut_J.nbytes + (1 << 20))
    assert i1["device_bytes"] <= bound, (i1["device_bytes"], bound)


def test_no_events():
    d, t = _random(seed=8, G=50, rate=0.0)
    assert t.n_events == 0
    _print_case("no events")
    pu.assert_parity(pu.gpu_run(d, t), _oracle(d, t), label="no events")


def test_single_gate_and_window_edges():
    d, t = _random(seed=9, G=1, C=5, T=100, rate=3.0, ks=(3,))
    # force events at t = 0 and t = t_max - 1 on the first input pin
    ev = t.evt_t.copy()
    p0 = slice(t.pin_ptr[0], t.pin_ptr[1])
    if ev[p0].size >= 2:
        ev[t.pin_ptr[0]] = 0
        ev[t.pin_ptr[1] - 1] = t.t_max - 1
    pin = np.repeat(np.arange(t.n_pins), np.diff(t.pin_ptr))
    t2 = synth._finish_trace(np.random.default_rng(1), t.n_pins, pin, ev, t.t_clk, t.t_max)
    _print_case("single gate")
    pu.assert_parity(pu.gpu_run(d, t2), _oracle(d, t2), label="single gate")


def test_cycle_bits_above_the_gate_id():
    """A 1 ns clock in 1 fs ticks leaves 9 bits of the low key word for the
    cycle in the chunk: 1024- and 2048-cycle chunks need the cycle bits the
    gate id leaves free in the high word (2048 is the default)."""
    d, t = _random(seed=12, G=300, C=4500, T=1_000_000, rate=0.01)
    _print_case("cycle high bits")
    o = _oracle(d, t)
    for chunk in (0, 512, 1024, 2048):
        g = pu.gpu_run(d, t, chunk_cycles=chunk)
        pu.assert_parity(g, o, label=f"high cycle bits chunk {chunk}")
        assert g["_info"]["chunk_cycles"] == (chunk or 2048)


def test_widest_gate_ids_and_clock():
    """2^21 + 5 gates (22-bit gate ids, no free bits in the high word) and a
    clock of 2^31 - 5 ticks for one-input cells (the pin code and the time
    in the cycle fill the low word): every chunk is one cycle."""
    rng = np.random.default_rng(13)
    lib = synth.make_library(rng, (1,), cells_per_k=2, n_axis=4)
    G = (1 << 21) + 5
    des = synth.assign_gates(rng, lib, np.ones(G, dtype=np.int64), 1.0, 50.0)
    P = 2 * G
    T, C = (1 << 31) - 5, 6
    rates = np.zeros(P)
    hot = rng.choice(P, size=400, replace=False)
    rates[hot] = 2.0
    rates[-2:] = 3.0  # the last gate, the largest id
    tr = synth.poisson_trace(rng, rates, C, T)
    tr = dataclasses.replace(tr, evt_slew=rng.uniform(50, 900, tr.n_events).astype(np.float32))
    _print_case(f"widest ids E={tr.n_events}")
    o = _oracle(des, tr)
    g = pu.gpu_run(des, tr)
    pu.assert_parity(g, o, label="widest ids")
    assert g["_info"]["chunk_cycles"] == 1


def test_dense_glitch_train():
    """One gate with thousands of events, about 70 of them per clock cycle
    (time windows of single cycles), many inside single cycles."""
    rng = np.random.default_rng(10)
    lib = synth.make_library(rng, (2,), cells_per_k=1, n_axis=4)
    des = synth.assign_gates(rng, lib, np.array([2, 2]), 1.0, 50.0)
    T, C = 10_000, 30
    P = 6
    rates = np.array([25.0, 15.0, 30.0, 0.5, 0.1, 0.2])
    tr = synth.poisson_trace(rng, rates, C, T)
    tr = dataclasses.replace(tr, evt_slew=rng.uniform(50, 900, tr.n_events).astype(np.float32))
    _print_case("dense train")
    o = _oracle(des, tr)
    assert o["n_glitches"] > 1000
    for chunk in (0, 2):
        pu.assert_parity(pu.gpu_run(des, tr, chunk_cycles=chunk), o, label=f"dense chunk {chunk}")


def test_hundreds_of_events_of_one_gate_in_one_cycle():
    """A gate with about 200 events inside single clock cycles (two pins at
    100 events per cycle each): a lane walks the whole run, with no limit on
    its length."""
    rng = np.random.default_rng(3)
    lib = synth.make_library(rng, (1,), cells_per_k=1, n_axis=3)
    des = synth.assign_gates(rng, lib, np.array([1]), 1.0, 5.0)
    tr = synth.poisson_trace(rng, np.array([100.0, 100.0]), 4, 100_000)
    _print_case("200 events per gate-cycle")
    o = _oracle(des, tr)
    assert tr.n_events > 600 and o["n_glitches"] > 500
    for chunk in (0, 1):
        pu.assert_parity(pu.gpu_run(des, tr, chunk_cycles=chunk), o, label=f"dense cycle chunk {chunk}")


def test_repeated_runs_agree():
    """Accumulators are reset between passes: two passes give the same integers
    and the same energies within the fp64 tolerance."""
    import eda_gate_level_amd as pa

    d, t = _random(seed=11, G=1500, C=120, rate=0.2)
    _print_case("repeated")
    an = pa.PowerAnalysis()
    try:
        an.load(d, t)
        outs = [an.run(per_event=True) for _ in range(3)]
    finally:
        pass
    o = _oracle(d, t)
    for r in outs:
        g = dict(r["totals"])
        g.update(wave_J=r["wave_J"].cpu().numpy(), cyc_events=r["cyc_events"].cpu().numpy().astype(np.uint64),
                 cyc_glitches=r["cyc_glitches"].cpu().numpy().astype(np.uint64),
                 evt_glitch=r["evt_glitch"][:t.n_events].cpu().numpy(),
                 evt_state_before=r["evt_state_before"][:t.n_events].cpu().numpy())
        pu.assert_parity(g, o, label="repeat")
    an.close()


@pytest.mark.parametrize("m", [1, 2, 4, 8])
def test_contention_small(m):
    """Every pin toggling m times per cycle: all events of a cycle share one
    waveform bin and most are glitches (the stress workload, reduced)."""
    w = synth.contention(m, G=12, C=700)
    _print_case(f"contention m={m}")
    pu.assert_parity(pu.gpu_run(w.design, w.trace), _oracle(w.design, w.trace), label=f"contention {m}")


@pytest.mark.parametrize("name", ["tiny", "medium", "skewed", "glitch_heavy"])
def test_workload_full_size(name):
    w = synth.make(name)
    _print_case(f"workload {name} E={w.trace.n_events}")
    o = _oracle(w.design, w.trace)
    g = pu.gpu_run(w.design, w.trace)
    pu.assert_parity(g, o, label=name)


@pytest.mark.parametrize("m", [1, 8])
def test_contention_full_size(m):
    """The waveform-bin stress workload at the shape the bench times (32
    two-input gates, 100,000 cycles, m toggles per pin and cycle: every event
    of a cycle in one bin, every toggle after a pin's first in a cycle a
    glitch) through the bench's pass: every total, bin and count against the
    threaded oracle."""
    import oracle

    w = synth.contention(m)
    _print_case(f"contention full size m={m} events={w.trace.n_events}")
    o = oracle.run(w.design, w.trace, per_event=False, threads=oracle.host_threads())
    g = pu.gpu_run(w.design, w.trace, per_event=False)
    pu.assert_parity(g, o, per_event=False, label=f"contention {m} full")


def test_plain_bins_is_a_timing_aid():
    """plain_bins = 1 or 2 swaps the bin atomics for plain adds or plain
    stores (the no-atomic variants of the stress test): the per-lane energy
    sums do not touch the bins, so they stay exact; 3 is refused."""
    import eda_gate_level_amd as pa

    d, t = LUT_CASES["tiny-7x7"]()
    _print_case("plain bins")
    ref = pu.gpu_run(d, t, per_event=False)
    for mode in (1, 2):
        g = pu.gpu_run(d, t, per_event=False, plain_bins=mode)
        for key in ("e_int_J", "e_sw_J", "e_gl_J", "n_events"):
            assert g[key] == ref[key], (mode, key)
        assert np.isfinite(g["wave_J"]).all()
    with pytest.raises(pa.PaError) as ei:
        pa.PowerAnalysis(plain_bins=3)
    assert ei.value.code == pa.PA_EINVAL


@pytest.mark.parametrize("name", ["medium", "skewed"])
def test_window_count_against_the_additive_law(name):
    """The paper sizes a gate's work items by an additive law, about
    events / target + a floor.  The library's windows, 2^s per (gate, time
    chunk) with s the smallest level whose expected events per window are
    at most 32, split by pin kind, must land between half the law's count
    (target 32, floor one per (gate, chunk)) and four times it (twice for
    the power of two, twice for the two kinds)."""
    import eda_gate_level_amd as pa

    w = synth.make(name)
    d, t = w.design, w.trace
    _print_case(f"window law {name}")
    an = pa.PowerAnalysis()
    try:
        an.load(d, t)
        st = an.window_stats()
        info = an.info()
    finally:
        an.close()
    Cc = info["chunk_cycles"]
    pb = d.pin_base()
    gate = np.repeat(np.repeat(np.arange(d.n_gates), np.diff(pb)), np.diff(t.pin_ptr))
    chunk = (t.evt_t // t.t_clk) // Cc
    per = np.bincount(gate.astype(np.int64) * info["n_chunks"] + chunk)
    per = per[per > 0]
    law = float(np.sum(per / 32.0 + 1.0))
    print(f"windows {st['n_windows']} law {law:.0f} ratio {st['n_windows'] / law:.3f}", flush=True)
    assert 0.5 * law <= st["n_windows"] <= 4.0 * law
