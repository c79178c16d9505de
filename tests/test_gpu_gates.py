"""GPU per-gate power output (pa_run_gates) against the oracle's per-gate
energies, and hotspot ranking on the full-size workloads.

The paper ranks gates by power to judge spatial accuracy (its Fig. 10 and
Table 3: rank correlation and the overlap of the top hotspots).  Here the reference ranking
is the oracle's; both sides compute every gate's internal, switching, glitch
and leakage energy in fp64, so the per-gate values must agree within the
energy bar (1e-9 relative) and the rankings must coincide.
"""
import numpy as np
import pytest

import parity_util as pu
from test_gpu_parity import RANDOM_CASES, _random
from workloads import synth

pytestmark = pytest.mark.gpu

REL_GATE = 1e-9
COMPONENTS = ("e_int_J", "e_sw_J", "e_gl_J", "e_leak_J")


def _oracle_gates(d, t):
    import oracle

    return oracle.run(d, t, per_event=False, per_gate=True)


def _gpu_gates(d, t, **kw):
    import eda_gate_level_amd as pa

    an = pa.PowerAnalysis(**kw)
    try:
        an.load(d, t)
        outs = an.alloc_outputs(per_gate=True)
        r = an.run(outs)
        g = dict(r["totals"])
        g["gate_J"] = r["gate_J"][:d.n_gates].cpu().numpy()
        g["wave_J"] = r["wave_J"].cpu().numpy()
        g["cyc_events"] = r["cyc_events"].cpu().numpy().astype(np.uint64)
        g["cyc_glitches"] = r["cyc_glitches"].cpu().numpy().astype(np.uint64)
        return g
    finally:
        an.close()


def _assert_gates(g, o, label):
    gj, oj = g["gate_J"], o["gate_J"]
    assert gj.shape == oj.shape
    den = np.maximum(np.abs(gj), np.abs(oj))
    bad = np.abs(gj - oj) > REL_GATE * den
    assert not bad.any(), f"{label}: {int(bad.sum())} gate entries off, first {np.argwhere(bad)[:3].tolist()}"
    # the rows add up to the totals of the same pass
    for c, key in enumerate(COMPONENTS):
        assert pu.rel_err(gj[:, c].sum(), g[key]) <= REL_GATE, (label, key)


@pytest.mark.parametrize("case", RANDOM_CASES[:4], ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_per_gate_energies_random(case):
    d, t = _random(**case)
    print(f"[case] per-gate {case}", flush=True)
    o = _oracle_gates(d, t)
    g = _gpu_gates(d, t, chunk_cycles=16)
    pu.assert_parity(g, o, per_event=False, label=f"gates {case}")
    _assert_gates(g, o, f"{case}")


def test_per_gate_no_events():
    d, t = _random(seed=8, G=50, rate=0.0)
    print("[case] per-gate no events", flush=True)
    o = _oracle_gates(d, t)
    g = _gpu_gates(d, t)
    _assert_gates(g, o, "no events")
    assert np.all(g["gate_J"][:, :3] == 0.0)


def _ranking(p_gpu, p_ref, frac=0.01):
    from scipy.stats import kendalltau

    tau = kendalltau(p_gpu, p_ref).statistic
    n = max(1, int(round(frac * p_ref.shape[0])))
    top_g = set(np.argsort(-p_gpu, kind="stable")[:n].tolist())
    top_r = set(np.argsort(-p_ref, kind="stable")[:n].tolist())
    return tau, len(top_g & top_r) / n


@pytest.mark.parametrize("name", ["medium", "skewed", "glitch_heavy"])
def test_hotspot_ranking_full_size(name):
    """Per-gate total power on the full workloads: every gate within the
    energy bar, Kendall tau of the two rankings at least 0.99999 and the top
    1% of gates the same set (overlap@1% = 1)."""
    w = synth.make(name)
    d, t = w.design, w.trace
    print(f"[case] hotspots {name}", flush=True)
    o = _oracle_gates(d, t)
    g = _gpu_gates(d, t)
    _assert_gates(g, o, name)
    window = float(t.t_max) * t.tick_s
    p_gpu = g["gate_J"].sum(axis=1) / window
    p_ref = o["gate_J"].sum(axis=1) / window
    tau, overlap = _ranking(p_gpu, p_ref)
    print(f"[hotspots] {name}: kendall tau {tau:.9f}, overlap@1% {overlap:.4f}", flush=True)
    assert tau >= 0.99999 and overlap == 1.0


def test_large_full_size_sampled():
    """The 200M-event, 2M-gate workload at full size through pa_run_gates
    (the diagnostic kernel template, which also adds every gate's own
    energies), checked against definitions and a sample of gates:
      - per-cycle event counts against a histogram of the event cycles;
      - glitch flags per cycle against the definition (an event whose pin has
        an earlier event in the same clock cycle);
      - the waveform adds up to the totals;
      - 256 random gates and the 16 busiest: their per-gate energies from the
        full run against the oracle run on just those gates (gates are
        independent, so the sub-design's rows are the same rows)."""
    import oracle

    w = synth.make("large")
    d, t = w.design, w.trace
    print(f"[case] large full size E={t.n_events}", flush=True)
    g = _gpu_gates(d, t)
    assert int(g["n_events"]) == t.n_events
    cyc = t.evt_t // t.t_clk
    C = t.n_cycles
    np.testing.assert_array_equal(g["cyc_events"], np.bincount(cyc, minlength=C).astype(np.uint64))
    first = np.zeros(t.n_events, dtype=bool)
    first[t.pin_ptr[:-1][np.diff(t.pin_ptr) > 0]] = True
    gl = np.zeros(t.n_events, dtype=bool)
    gl[1:] = ~first[1:] & (cyc[1:] == cyc[:-1])
    assert int(g["n_glitches"]) == int(gl.sum())
    np.testing.assert_array_equal(g["cyc_glitches"], np.bincount(cyc[gl], minlength=C).astype(np.uint64))
    total = sum(g[k] for k in COMPONENTS)
    assert pu.rel_err(g["wave_J"].sum(), total) <= REL_GATE
    rng = np.random.default_rng(3)
    counts = np.diff(t.pin_ptr)
    per_gate = np.add.reduceat(counts, d.pin_base()[:-1]) if d.n_gates else counts
    pick = np.unique(np.concatenate([rng.choice(d.n_gates, size=256, replace=False),
                                     np.argsort(-per_gate, kind="stable")[:16]]))
    sub = synth.select_gates(w, pick)
    o = oracle.run(sub.design, sub.trace, per_event=False, per_gate=True)
    gj, oj = g["gate_J"][pick], o["gate_J"]
    den = np.maximum(np.abs(gj), np.abs(oj))
    bad = np.abs(gj - oj) > REL_GATE * den
    assert not bad.any(), f"{int(bad.sum())} sampled gate entries off"
    print(f"[large] {t.n_events} events, {int(gl.sum())} glitches, {pick.size} gates checked", flush=True)
