"""GPU parity of the walk kernel, the pass without per-event outputs on 7- and
8-point LUT axes, on the edge cases the per-event kernel meets elsewhere:
input counts 1..5 (pin records in registers up to four inputs, in LDS
above; a block's cells' LUTs must fit its LDS, which wider cells' do not),
forced same-timestamp collisions, events on cycle boundaries, a
partial last bin, several chunk lengths and launch grids, fixed windows,
one gate with events at t = 0 and t = t_max - 1, 22-bit gate ids, cycle bits
above the gate id, dense glitch trains and hundreds of events of one gate in
one cycle.  Every case checks that the walk kernel is the one that ran, then
compares every total, bin and count with the oracle.

Slews are drawn log-uniform over 0.05..300 ps, so they fall below, inside
(every segment) and above the 2..200 ps slew axis.  Libraries are chosen
so that every block's LUT range fits its LDS: the walk kernel runs in every
case (the general kernel takes over otherwise, which the per-event parity
tests cover).
"""
import dataclasses

import numpy as np
import pytest

import parity_util as pu
from workloads import synth

pytestmark = pytest.mark.gpu


def _oracle(d, t):
    import oracle

    return oracle.run(d, t, per_event=False)


def _print_case(name):
    print(f"[case] {name}", flush=True)


def _slews(rng, n):
    return np.exp(rng.uniform(np.log(50.0), np.log(300_000.0), n)).astype(np.float32)


def _case(seed, G=200, C=40, T=1000, rate=0.3, ks=(1, 2, 3, 4), collide=0, t_max=None, n_axis=7, cpk=2, hot=()):
    """A random design and Poisson trace; hot = ((gate, rate), ...) gives those
    gates' pins their own rate (events per pin per cycle)."""
    rng = np.random.default_rng(seed)
    lib = synth.make_library(rng, ks, cells_per_k=cpk, n_axis=n_axis)
    k = rng.choice(np.array(ks), size=G)
    des = synth.assign_gates(rng, lib, k, 1.0, 50.0)
    pb = des.pin_base()
    P = int(pb[-1])
    rates = np.full(P, rate)
    for g, r in hot:
        rates[pb[g]:pb[g + 1]] = r
    tr = synth.poisson_trace(rng, rates, C, T)
    pin = np.repeat(np.arange(P), np.diff(tr.pin_ptr))
    tt = tr.evt_t
    if collide:
        tt = (tt // collide) * collide
    if t_max is not None:
        tt = np.minimum(tt, t_max - 1)
    tr = synth._finish_trace(rng, P, pin, tt, T, t_max if t_max is not None else C * T)
    return des, dataclasses.replace(tr, evt_slew=_slews(rng, tr.n_events))


def _walk_run(d, t, label, **kw):
    g = pu.gpu_run(d, t, per_event=False, **kw)
    if t.n_events > 0:
        assert g["_info"]["walk_kernel"] == 1, f"{label}: the walk kernel did not run"
    return g


CASES = [
    dict(seed=1),
    dict(seed=2, ks=(1, 5), cpk=1, G=60, rate=0.2),  # five inputs: pin records in LDS
    dict(seed=3, collide=50, rate=0.8, G=120),
    dict(seed=4, collide=1000, rate=0.6, G=80),  # events on cycle boundaries
    dict(seed=5, t_max=39 * 1000 + 217),  # partial last bin
    dict(seed=6, G=3000, C=300, rate=0.05),
    dict(seed=14, ks=(2, 3), G=150, rate=0.4, n_axis=8),
    dict(seed=15, ks=(5,), cpk=1, G=400, C=60, rate=0.5, collide=10),
    dict(seed=17, G=3000, C=300, rate=0.05, n_axis=8),  # the library does not fit one block's LDS
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
@pytest.mark.parametrize("chunk", [0, 1, 3, 16])
def test_walk_random_designs_any_chunking(case, chunk):
    d, t = _case(**case)
    label = f"walk {case} chunk {chunk}"
    _print_case(label)
    pu.assert_parity(_walk_run(d, t, label, chunk_cycles=chunk), _oracle(d, t), per_event=False, label=label)


@pytest.mark.parametrize("grid", [1, 3, 64, 256])
def test_walk_launch_grid(grid):
    d, t = _case(seed=7, G=2000, C=200, rate=0.1)
    label = f"walk grid {grid}"
    _print_case(label)
    pu.assert_parity(_walk_run(d, t, label, grid_blocks=grid), _oracle(d, t), per_event=False, label=label)


@pytest.mark.parametrize("n_fix", [1, 4, 32])
def test_walk_fixed_windows(n_fix):
    d, t = _case(seed=9, G=400, C=120, rate=0.3)
    label = f"walk fixed windows {n_fix}"
    _print_case(label)
    g = _walk_run(d, t, label, fixed_window_cycles=n_fix)
    pu.assert_parity(g, _oracle(d, t), per_event=False, label=label)


def test_walk_no_events():
    d, t = _case(seed=8, G=50, rate=0.0)
    assert t.n_events == 0
    _print_case("walk no events")
    pu.assert_parity(_walk_run(d, t, "no events"), _oracle(d, t), per_event=False, label="walk no events")


def test_walk_single_gate_and_window_edges():
    d, t = _case(seed=9, G=1, C=5, T=100, rate=3.0, ks=(3,))
    ev = t.evt_t.copy()
    assert t.pin_ptr[1] - t.pin_ptr[0] >= 2
    ev[t.pin_ptr[0]] = 0
    ev[t.pin_ptr[1] - 1] = t.t_max - 1
    pin = np.repeat(np.arange(t.n_pins), np.diff(t.pin_ptr))
    rng = np.random.default_rng(1)
    t2 = synth._finish_trace(rng, t.n_pins, pin, ev, t.t_clk, t.t_max)
    t2 = dataclasses.replace(t2, evt_slew=_slews(rng, t2.n_events))
    _print_case("walk single gate")
    for chunk in (0, 1):
        label = f"walk single gate chunk {chunk}"
        pu.assert_parity(_walk_run(d, t2, label, chunk_cycles=chunk), _oracle(d, t2), per_event=False, label=label)


def test_walk_cycle_bits_above_the_gate_id():
    """A 1 ns clock in 1 fs ticks: 2048-cycle chunks keep the cycle's high
    bits above the gate id in the sort key; the walk kernel's 32-bit key
    holds 20 bits of time in the cycle and up to 12 of cycle."""
    d, t = _case(seed=12, G=300, C=4500, T=1_000_000, rate=0.01)
    o = _oracle(d, t)
    for chunk in (0, 512, 1024):
        label = f"walk high cycle bits chunk {chunk}"
        _print_case(label)
        g = _walk_run(d, t, label, chunk_cycles=chunk)
        pu.assert_parity(g, o, per_event=False, label=label)
        assert g["_info"]["chunk_cycles"] == (chunk or 2048)


def test_walk_widest_gate_ids():
    """2^21 + 5 one-input gates (22-bit gate ids, no free bits in the sort
    key's high word), events on 400 random pins and on the last gate."""
    rng = np.random.default_rng(13)
    lib = synth.make_library(rng, (1,), cells_per_k=2, n_axis=7)
    G = (1 << 21) + 5
    des = synth.assign_gates(rng, lib, np.ones(G, dtype=np.int64), 1.0, 50.0)
    P = 2 * G
    rates = np.zeros(P)
    rates[rng.choice(P, size=400, replace=False)] = 2.0
    rates[-2:] = 3.0
    tr = synth.poisson_trace(rng, rates, 300, 1000)
    tr = dataclasses.replace(tr, evt_slew=_slews(rng, tr.n_events))
    _print_case(f"walk widest ids E={tr.n_events}")
    o = _oracle(des, tr)
    for chunk in (0, 1):
        label = f"walk widest ids chunk {chunk}"
        pu.assert_parity(_walk_run(des, tr, label, chunk_cycles=chunk), o, per_event=False, label=label)


def test_walk_dense_glitch_train():
    """Two two-input gates, about 70 events per clock cycle on the first."""
    rng = np.random.default_rng(10)
    lib = synth.make_library(rng, (2,), cells_per_k=1, n_axis=7)
    des = synth.assign_gates(rng, lib, np.array([2, 2]), 1.0, 50.0)
    rates = np.array([25.0, 15.0, 30.0, 0.5, 0.1, 0.2])
    tr = synth.poisson_trace(rng, rates, 30, 10_000)
    tr = dataclasses.replace(tr, evt_slew=_slews(rng, tr.n_events))
    o = _oracle(des, tr)
    assert o["n_glitches"] > 500
    for chunk in (0, 2):
        label = f"walk dense train chunk {chunk}"
        _print_case(label)
        pu.assert_parity(_walk_run(des, tr, label, chunk_cycles=chunk), o, per_event=False, label=label)


def test_walk_hundreds_of_events_of_one_gate_in_one_cycle():
    """About 200 events of one gate inside single clock cycles: one lane
    walks the whole window."""
    rng = np.random.default_rng(3)
    lib = synth.make_library(rng, (1,), cells_per_k=1, n_axis=8)
    des = synth.assign_gates(rng, lib, np.array([1]), 1.0, 5.0)
    tr = synth.poisson_trace(rng, np.array([100.0, 100.0]), 4, 100_000)
    tr = dataclasses.replace(tr, evt_slew=_slews(rng, tr.n_events))
    o = _oracle(des, tr)
    assert tr.n_events > 600
    for chunk in (0, 1):
        label = f"walk 200 events per gate-cycle chunk {chunk}"
        _print_case(label)
        pu.assert_parity(_walk_run(des, tr, label, chunk_cycles=chunk), o, per_event=False, label=label)


@pytest.mark.parametrize("m", [1, 2, 4, 8])
def test_walk_contention_small(m):
    w = synth.contention(m, G=12, C=700)
    label = f"walk contention m={m}"
    _print_case(label)
    pu.assert_parity(_walk_run(w.design, w.trace, label), _oracle(w.design, w.trace), per_event=False, label=label)


def test_walk_matches_the_general_kernel():
    """The walk kernel and the general kernel agree: integer outputs bit for
    bit, energies and bins to rounding (they sum in different orders).  The
    walk kernel takes the leakage's in-bin time corrections from the bins'
    sum less the dynamic energies, so its leakage total carries a rounding
    error of about 1e-16 times the dynamic energy: the bar for the leakage
    is 1e-15 of the dynamic energy, not of the leakage itself."""
    d, t = _case(seed=16, G=1500, C=100, rate=0.3, ks=(1, 2, 5), cpk=1)
    _print_case("walk vs general kernel")
    a = _walk_run(d, t, "walk vs general")
    b = pu.gpu_run(d, t, per_event=True, lut_lds_kib=-1)  # no LUT copies: the general kernel
    assert b["_info"]["walk_kernel"] == 0
    for key in ("n_events", "n_glitches"):
        assert a[key] == b[key], key
    assert np.array_equal(a["cyc_events"], b["cyc_events"])
    assert np.array_equal(a["cyc_glitches"], b["cyc_glitches"])
    for key in ("e_int_J", "e_sw_J", "e_gl_J", "p_int_W", "p_sw_W", "p_gl_W"):
        assert pu.rel_err(a[key], b[key]) <= 1e-12, key
    e_dyn = b["e_int_J"] + b["e_sw_J"] + b["e_gl_J"]
    assert abs(a["e_leak_J"] - b["e_leak_J"]) <= 1e-15 * e_dyn, (a["e_leak_J"], b["e_leak_J"], e_dyn)
    assert pu.rel_err(a["p_leak_W"], b["p_leak_W"]) <= 1e-15 * e_dyn / b["e_leak_J"] + 1e-15
    np.testing.assert_allclose(a["wave_J"], b["wave_J"], rtol=1e-12, atol=0)


@pytest.mark.parametrize("case", [dict(seed=1), dict(seed=2, ks=(1, 5), cpk=1, G=60, rate=0.2),
                                  dict(seed=3, collide=50, rate=0.8, G=120), dict(seed=14, ks=(2, 3), G=150, n_axis=8)],
                         ids=["k1-4", "k1-5", "collide", "8x8"])
@pytest.mark.parametrize("chunk", [0, 1])
def test_walk_per_event_outputs(case, chunk):
    """Per-event outputs from the walk kernel (written in stream order, moved
    into the caller's order through every event's slot): the glitch flags and
    the states before every event bit for bit against the oracle and against
    the general kernel, with every total, bin and count."""
    d, t = _case(**case)
    label = f"walk per-event {case} chunk {chunk}"
    _print_case(label)
    g = pu.gpu_run(d, t, per_event=True, chunk_cycles=chunk)
    assert g["_info"]["walk_kernel"] == 1, label
    import oracle

    pu.assert_parity(g, oracle.run(d, t), per_event=True, label=label)
    ref = pu.gpu_run(d, t, per_event=True, chunk_cycles=chunk, lut_lds_kib=-1)
    np.testing.assert_array_equal(g["evt_glitch"], ref["evt_glitch"])
    np.testing.assert_array_equal(g["evt_state_before"], ref["evt_state_before"])


def _walk_gates(d, t, **kw):
    import eda_gate_level_amd as pa

    an = pa.PowerAnalysis(**kw)
    try:
        an.load(d, t)
        outs = an.alloc_outputs(per_gate=True)
        r = an.run(outs)
        g = dict(r["totals"])
        g["gate_J"] = r["gate_J"][:d.n_gates].cpu().numpy()
        # a second run into rows filled with NaN: every row rewritten, the same bits
        outs["gate_J"].fill_(float("nan"))
        g["gate_J_again"] = an.run(outs)["gate_J"][:d.n_gates].cpu().numpy()
        g["wave_J"] = r["wave_J"].cpu().numpy()
        g["cyc_events"] = r["cyc_events"].cpu().numpy().astype(np.uint64)
        g["cyc_glitches"] = r["cyc_glitches"].cpu().numpy().astype(np.uint64)
        g["_info"] = an.info()
        return g
    finally:
        an.close()


@pytest.mark.parametrize("case", [dict(seed=1), dict(seed=2, ks=(1, 5), cpk=1, G=60, rate=0.2),
                                  dict(seed=4, collide=1000, rate=0.6, G=80), dict(seed=14, ks=(2, 3), G=150, n_axis=8),
                                  dict(seed=21, G=40, C=600, rate=0.2,
                                       hot=((0, 0.0), (7, 40.0), (8, 3.0), (20, 0.0), (30, 12.0), (39, 0.0)))],
                         ids=["k1-4", "k1-5", "cycle-edges", "8x8", "hot-gates"])
@pytest.mark.parametrize("chunk", [0, 3])
def test_walk_per_gate_rows(case, chunk):
    """Per-gate rows from the walk kernel (each window's energies and the
    leakage of its power changes to t_max, stored at the window's rank in
    gate order and added up per gate after the walk): every entry within
    1e-9 of the oracle's per-gate energies, the rows adding up to the
    totals, every total, bin and count, and a second run giving the same
    rows bit for bit."""
    import oracle
    from test_gpu_gates import _assert_gates

    d, t = _case(**case)
    label = f"walk per-gate {case} chunk {chunk}"
    _print_case(label)
    g = _walk_gates(d, t, chunk_cycles=chunk)
    assert g["_info"]["walk_kernel"] == 1, label
    o = oracle.run(d, t, per_event=False, per_gate=True)
    pu.assert_parity(g, o, per_event=False, label=label)
    _assert_gates(g, o, label)
    assert np.array_equal(g["gate_J"], g["gate_J_again"]), label
