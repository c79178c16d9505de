"""GPU power analysis of activity text (pa_run_text): host threads pack the
text segment by segment while the GPU loads and computes the previous
segment (the paper's CPU-side event packing overlapped with the GPU,
"GPU-Accelerated Gate-Level Time-Based Power Analysis via Event-Density-
Aware Partitioning and Kernel Fusion", Fig. 13).

The oracle side reads the same text with the plain reader (oracle.vcd_text)
and runs the CPU oracle on the result; the totals, waveform and counts must
meet the usual parity bar whatever the segment length, thread count and
overlap mode.
"""
import numpy as np
import pytest

import parity_util as pu
from test_gpu_parity import RANDOM_CASES, _random
from workloads import synth, vcd_text

pytestmark = pytest.mark.gpu


def _oracle_text(d, text, t):
    import oracle
    from oracle import vcd_text as ov

    tr = ov.parse(text, int(d.pin_base()[-1]))
    tt = synth.Trace(pin_ptr=tr["pin_ptr"], pin_init=tr["pin_init"], evt_t=tr["evt_t"], evt_val=tr["evt_val"],
                     evt_slew=tr["evt_slew"], t_clk=t.t_clk, t_max=t.t_max, tick_s=t.tick_s)
    return oracle.run(d, tt, per_event=False), tt


def _gpu_text(d, text, t, **kw):
    import eda_gate_level_amd as pa

    an = pa.PowerAnalysis()
    try:
        an.load_design(d)
        r = an.run_text(text, t.t_clk, t.t_max, t.tick_s, **kw)
        g = dict(r["totals"])
        g["wave_J"] = r["wave_J"].cpu().numpy()
        g["cyc_events"] = r["cyc_events"].cpu().numpy().astype(np.uint64)
        g["cyc_glitches"] = r["cyc_glitches"].cpu().numpy().astype(np.uint64)
        g["stats"] = r["stats"]
        return g
    finally:
        an.close()


@pytest.mark.parametrize("case", RANDOM_CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
@pytest.mark.parametrize("seg,threads,serial", [(1, 1, False), (3, 4, False), (16, 16, True), (1000, 2, False)])
def test_text_random_designs(case, seg, threads, serial):
    d, t = _random(**case)
    text = vcd_text.write(t)
    print(f"[case] text {case} segment {seg} threads {threads} serial {serial}", flush=True)
    o, tt = _oracle_text(d, text, t)
    for k in ("pin_ptr", "pin_init", "evt_t", "evt_val", "evt_slew"):
        assert np.array_equal(getattr(tt, k), getattr(t, k)), k
    g = _gpu_text(d, text, t, segment_cycles=seg, n_threads=threads, serial=serial)
    pu.assert_parity(g, o, per_event=False, label=f"text {case} seg {seg}")
    assert g["stats"]["n_segments"] == -(-t.n_cycles // seg)
    assert g["stats"]["n_events"] == t.n_events


def test_text_gaps_and_boundaries():
    """Segments with no events, events on segment starts and at t = 0, a
    window that ends inside a cycle."""
    d, t = _random(seed=21, G=150, C=64, rate=0.5, collide=1000, t_max=63 * 1000 + 7)
    keep = (t.evt_t < 8_000) | (t.evt_t >= 40_000)  # cycles 8..39 silent
    pin = np.repeat(np.arange(t.n_pins), np.diff(t.pin_ptr))[keep]
    counts = np.bincount(pin, minlength=t.n_pins)
    ptr = np.zeros(t.n_pins + 1, np.int64)
    np.cumsum(counts, out=ptr[1:])
    idx = np.arange(pin.size) - ptr[pin]
    val = (t.pin_init[pin] ^ ((idx + 1) & 1)).astype(np.uint8)
    t2 = synth.Trace(pin_ptr=ptr, pin_init=t.pin_init, evt_t=t.evt_t[keep], evt_val=val,
                     evt_slew=t.evt_slew[keep], t_clk=t.t_clk, t_max=t.t_max)
    text = vcd_text.write(t2)
    print("[case] text gaps and boundaries", flush=True)
    o, _ = _oracle_text(d, text, t2)
    for seg in (4, 8, 5):
        g = _gpu_text(d, text, t2, segment_cycles=seg, n_threads=3)
        pu.assert_parity(g, o, per_event=False, label=f"gaps seg {seg}")


def test_text_no_events():
    d, t = _random(seed=22, G=40, rate=0.0)
    text = vcd_text.write(t)
    print("[case] text no events", flush=True)
    o, _ = _oracle_text(d, text, t)
    g = _gpu_text(d, text, t, segment_cycles=7)
    pu.assert_parity(g, o, per_event=False, label="no events")


def test_text_errors():
    import eda_gate_level_amd as pa

    d, t = _random(seed=23, G=30, C=20, rate=0.4)
    text = vcd_text.write(t)
    print("[case] text errors", flush=True)
    an = pa.PowerAnalysis()
    try:
        with pytest.raises(pa.PaError) as e:
            an.run_text(text, t.t_clk, t.t_max)
        assert e.value.code == pa.PA_ESTATE
        an.load_design(d)
        # an event at or after t_max
        with pytest.raises(pa.PaError) as e:
            an.run_text(text, t.t_clk, int(t.evt_t.max()), segment_cycles=4)
        assert e.value.code == pa.PA_EDATA
        # values that do not alternate: the load of the segment rejects them
        t_bad = synth.Trace(pin_ptr=t.pin_ptr, pin_init=t.pin_init ^ 1, evt_t=t.evt_t, evt_val=t.evt_val,
                            evt_slew=t.evt_slew, t_clk=t.t_clk, t_max=t.t_max)
        with pytest.raises(pa.PaError) as e:
            an.run_text(vcd_text.write(t_bad), t.t_clk, t.t_max, segment_cycles=4)
        assert e.value.code == pa.PA_EDATA
        # a parse error in a late segment, behind segments already computed
        bad = text + b"#%d\nq! 1.0\n" % (t.t_max - 1)
        for serial in (False, True):
            with pytest.raises(pa.PaError) as e:
                an.run_text(bad, t.t_clk, t.t_max, segment_cycles=2, serial=serial)
            assert e.value.code == pa.PA_EDATA
        # the context is usable afterwards
        g = an.run_text(text, t.t_clk, t.t_max, segment_cycles=4)
        assert g["totals"]["n_events"] == t.n_events
        with pytest.raises(pa.PaError) as e:
            an.run()
        assert e.value.code == pa.PA_ESTATE
    finally:
        an.close()


def test_text_medium_full_size():
    """The 10M-event workload through text, segments of 1,024 cycles, both
    modes, against the oracle on the trace the text was written from."""
    import oracle

    w = synth.make("medium")
    d, t = w.design, w.trace
    text = vcd_text.write(t)
    print(f"[case] text medium {len(text)} bytes", flush=True)
    o = oracle.run(d, t, per_event=False)
    for serial in (False, True):
        g = _gpu_text(d, text, t, serial=serial)
        pu.assert_parity(g, o, per_event=False, label=f"medium text serial {serial}")
        st = g["stats"]
        print(f"[text] medium serial={serial}: wall {st['wall_s']:.3f}s parse {st['parse_s']:.3f}s "
              f"gpu {st['gpu_s']:.3f}s index {st['index_s']:.3f}s header {st['header_s']:.3f}s", flush=True)
