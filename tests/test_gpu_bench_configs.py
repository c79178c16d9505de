"""GPU parity in the configurations the benchmark times, against the oracle.

The timed pass is pa_run without per-event or per-gate outputs, in the
default layout (2048-cycle chunks, one 1024-thread block per compute unit);
it runs the plain (non-diagnostic) kernel template chosen by the LUT axis
length: 7-point axes for the 10M-event workload, 8-point axes for the
200M-event one.  Here those exact configurations are compared with the
oracle element by element (every bin, every count, every total), plus the
cases the generated workloads never reach: loads and slews outside the LUT
axes (linear extrapolation, the NLDM reading of the paper's LUT
interpolation, Sec. 2.4.1 and Fig. 2) and cell libraries whose tables do not
fit in a block's LDS (the global-table kernel templates).
"""
import dataclasses
import math

import numpy as np
import pytest

import parity_util as pu
from workloads import synth

pytestmark = pytest.mark.gpu


def _oracle(d, t, **kw):
    import oracle

    return oracle.run(d, t, per_event=False, threads=oracle.host_threads(), **kw)


def _print_case(name):
    print(f"[case] {name}", flush=True)


def test_medium_bench_configuration():
    """The 10M-event workload exactly as the benchmark runs it."""
    w = synth.make("medium")
    _print_case(f"medium bench config E={w.trace.n_events}")
    o = _oracle(w.design, w.trace)
    g = pu.gpu_run(w.design, w.trace, per_event=False)
    assert g["_info"]["chunk_cycles"] == 2048 and g["_info"]["tables_in_lds"] == 1
    pu.assert_parity(g, o, per_event=False, label="medium bench config")


def test_large_bench_configuration_full_size():
    """The 200M-event, 2M-gate workload (8x8 LUTs, 0.5 ns clock, 20,000
    cycles) through the pass the benchmark times, against the oracle run on
    all host cores: the 8 totals, every one of the 20,000 bins and the
    per-cycle counts."""
    w = synth.make("large")
    d, t = w.design, w.trace
    _print_case(f"large bench config E={t.n_events}")
    g = pu.gpu_run(d, t, per_event=False)
    assert d.n_slew == 8
    print(f"[large] gpu done (chunks of {g['_info']['chunk_cycles']} cycles), oracle on "
          f"{__import__('oracle').host_threads()} threads", flush=True)
    o = _oracle(d, t)
    pu.assert_parity(g, o, per_event=False, label="large bench config")
    print(f"[large] {t.n_events} events, {int(o['n_glitches'])} glitches, {t.n_cycles} bins checked", flush=True)


def _large_shaped(seed, G, C, cap_ff=(1.0, 50.0), slew_ps=(5.0, 100.0), n_axis=8):
    """A reduced 200M-event-workload shape: 1-4 input cells with 8x8 LUTs,
    0.5 ns clock, per-pin rates lognormal (sigma 1), several 2048-cycle
    chunks.  Loads and slews are drawn from the given ranges (the library's
    axes span 0.5-100 fF and 2-200 ps)."""
    rng = np.random.default_rng(seed)
    lib = synth.make_library(rng, [1, 2, 3, 4], n_axis=n_axis)
    k = rng.integers(1, 5, size=G)
    des = synth.assign_gates(rng, lib, k, *cap_ff)
    P = int(des.pin_base()[-1])
    rates = rng.lognormal(math.log(0.005) - 0.5, 1.0, size=P)
    tr = synth.poisson_trace(rng, rates, C, synth.NS // 2)
    slew = rng.uniform(slew_ps[0] * synth.PS, slew_ps[1] * synth.PS, tr.n_events).astype(np.float32)
    return des, dataclasses.replace(tr, evt_slew=slew)


@pytest.mark.parametrize("per_event", [False, True])
def test_large_shaped_reduced(per_event):
    d, t = _large_shaped(21, G=20_000, C=7000)
    _print_case(f"large-shaped E={t.n_events} per_event {per_event}")
    import oracle

    o = oracle.run(d, t, per_event=per_event, threads=oracle.host_threads())
    g = pu.gpu_run(d, t, per_event=per_event)
    assert g["_info"]["n_chunks"] >= 4
    pu.assert_parity(g, o, per_event=per_event, label=f"large-shaped per_event {per_event}")


@pytest.mark.parametrize("n_axis", [7, 8, 5])
def test_loads_and_slews_outside_the_axes(n_axis):
    """Loads of 0.05-400 fF and slews of 0.3-600 ps against axes of 0.5-100
    fF and 2-200 ps: bilinear extrapolation on both axes, in the plain
    templates (7- and 8-point axes) and the generic one."""
    d, t = _large_shaped(22, G=3000, C=2500, cap_ff=(0.05, 400.0), slew_ps=(0.3, 600.0), n_axis=n_axis)
    caps = d.gate_cap_F
    assert (caps < d.cap_axis[0, 0]).any() and (caps > d.cap_axis[0, -1]).any()
    assert (t.evt_slew < d.slew_axis[0, 0]).any() and (t.evt_slew > d.slew_axis[0, -1]).any()
    _print_case(f"extrapolation n_axis {n_axis} E={t.n_events}")
    o = _oracle(d, t)
    for chunk in (0, 64):
        g = pu.gpu_run(d, t, per_event=False, chunk_cycles=chunk)
        pu.assert_parity(g, o, per_event=False, label=f"extrapolation {n_axis} chunk {chunk}")


def _big_library(seed, cells_per_k, G=4000, C=600, rate=0.05):
    rng = np.random.default_rng(seed)
    lib = synth.make_library(rng, [1, 2, 3, 4], cells_per_k=cells_per_k)
    k = rng.integers(1, 5, size=G)
    des = synth.assign_gates(rng, lib, k, 1.0, 50.0)
    tr = synth.poisson_trace(rng, np.full(int(des.pin_base()[-1]), rate), C, synth.NS)
    return des, tr


@pytest.mark.parametrize("chunk", [0, 128, 7])
def test_cell_tables_beyond_lds(chunk):
    """A library of 480 cells (120 per input count, 7x7 LUTs): its per-cell
    tables do not fit in a block's LDS next to the bins and pin records, so
    the pass reads them through the caches (the global-table templates,
    plain and diagnostic), at several chunk lengths."""
    d, t = _big_library(23, cells_per_k=120)
    assert d.n_cells == 480
    _print_case(f"480 cells chunk {chunk} E={t.n_events}")
    import oracle

    o = oracle.run(d, t, per_event=True, threads=oracle.host_threads())
    for per_event in (False, True):
        g = pu.gpu_run(d, t, per_event=per_event, chunk_cycles=chunk)
        assert g["_info"]["tables_in_lds"] == 0
        pu.assert_parity(g, o, per_event=per_event, label=f"480 cells chunk {chunk} per_event {per_event}")
