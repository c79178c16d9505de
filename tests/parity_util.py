"""Helpers of the GPU-vs-oracle parity tests.

Bars (per the project contract): integer outputs -- per-event glitch flags,
per-event states before the event, per-cycle event and glitch counts, event
and glitch totals -- are compared bit for bit; energies and powers are fp64
and must agree within a relative error of 1e-9 per total and 1e-7 per
waveform bin (fp64 atomics make the GPU summation order nondeterministic).
"""
import numpy as np

REL_TOTAL = 1e-9
REL_BIN = 1e-7
TOTAL_KEYS = ("e_int_J", "e_sw_J", "e_gl_J", "e_leak_J", "p_int_W", "p_sw_W", "p_gl_W", "p_leak_W")


def gpu_run(design, trace, per_event=True, **ctx_kw):
    """Load and run through the C ABI; returns host numpy results."""
    import eda_gate_level_amd as pa

    an = pa.PowerAnalysis(**ctx_kw)
    try:
        an.load(design, trace)
        r = an.run(per_event=per_event)
        out = dict(r["totals"])
        E = trace.n_events
        out["wave_J"] = r["wave_J"].cpu().numpy()
        out["cyc_events"] = r["cyc_events"].cpu().numpy().astype(np.uint64)
        out["cyc_glitches"] = r["cyc_glitches"].cpu().numpy().astype(np.uint64)
        if per_event:
            out["evt_glitch"] = r["evt_glitch"][:E].cpu().numpy()
            out["evt_state_before"] = r["evt_state_before"][:E].cpu().numpy()
        out["_info"] = an.info()
        return out
    finally:
        an.close()


def rel_err(a, b):
    a, b = float(a), float(b)
    den = max(abs(a), abs(b))
    return 0.0 if den == 0.0 else abs(a - b) / den


def assert_parity(g, o, per_event=True, label=""):
    for k in TOTAL_KEYS:
        e = rel_err(g[k], o[k])
        assert e <= REL_TOTAL, f"{label} {k}: gpu {g[k]!r} oracle {o[k]!r} rel {e:.3g}"
    assert int(g["n_events"]) == int(o["n_events"]), label
    assert int(g["n_glitches"]) == int(o["n_glitches"]), label
    np.testing.assert_array_equal(g["cyc_events"], o["cyc_events"], err_msg=f"{label} cyc_events")
    np.testing.assert_array_equal(g["cyc_glitches"], o["cyc_glitches"], err_msg=f"{label} cyc_glitches")
    gw, ow = np.asarray(g["wave_J"]), np.asarray(o["wave_J"])
    den = np.maximum(np.abs(gw), np.abs(ow))
    bad = np.abs(gw - ow) > REL_BIN * den
    assert not bad.any(), f"{label} wave bins off: first {np.flatnonzero(bad)[:5]} gpu {gw[bad][:3]} oracle {ow[bad][:3]}"
    if per_event:
        np.testing.assert_array_equal(g["evt_glitch"], o["evt_glitch"], err_msg=f"{label} evt_glitch")
        np.testing.assert_array_equal(g["evt_state_before"], o["evt_state_before"], err_msg=f"{label} states")
