"""Failure handling of the C ABI on the GPU: bad call order, bad arguments
and bad data are reported with the documented codes, and a failing load
leaves the previously loaded data usable.  Every error is detected on the
host or by the load kernels' own validation; no kernel is made to fault."""
import dataclasses

import numpy as np
import pytest

import parity_util as pu
from workloads import synth

pytestmark = pytest.mark.gpu


def _small():
    w = synth.subset_gates(synth.tiny(), 0, 50)
    return w.design, w.trace


def test_call_order():
    import eda_gate_level_amd as pa

    an = pa.PowerAnalysis()
    try:
        with pytest.raises(pa.PaError) as ei:
            an.n_cycles, an.n_events = 4, 4
            an.run()
        assert ei.value.code == pa.PA_ESTATE
        d, t = _small()
        with pytest.raises(pa.PaError) as ei:
            an.load_events(t)
        assert ei.value.code == pa.PA_ESTATE
    finally:
        an.close()


def _mut(t, kind):
    pin = np.repeat(np.arange(t.n_pins), np.diff(t.pin_ptr))
    e = int(np.flatnonzero(np.diff(pin) == 0)[0]) + 1
    if kind == "unsorted":
        tt = t.evt_t.copy(); tt[e] = tt[e - 1]; return dataclasses.replace(t, evt_t=tt)
    if kind == "value":
        v = t.evt_val.copy(); v[e] ^= 1; return dataclasses.replace(t, evt_val=v)
    if kind == "value2":
        v = t.evt_val.copy(); v[e] = 2; return dataclasses.replace(t, evt_val=v)
    if kind == "t_max":
        tt = t.evt_t.copy(); tt[-1] = t.t_max; return dataclasses.replace(t, evt_t=tt)
    if kind == "negative":
        tt = t.evt_t.copy(); tt[t.pin_ptr[pin[e]]] = -5; return dataclasses.replace(t, evt_t=tt)
    if kind == "slew":
        s = t.evt_slew.copy(); s[e] = 0.0; return dataclasses.replace(t, evt_slew=s)
    if kind == "slew_nan":
        s = t.evt_slew.copy(); s[e] = np.nan; return dataclasses.replace(t, evt_slew=s)
    if kind == "init":
        i = t.pin_init.copy(); i[0] = 3; return dataclasses.replace(t, pin_init=i)
    if kind == "pin_ptr":
        pp = t.pin_ptr.copy(); pp[3], pp[4] = pp[4], pp[3]
        if pp[3] == pp[4]:
            pp[3] += 1
        return dataclasses.replace(t, pin_ptr=pp)
    if kind == "ptr_first":  # pin_ptr[0] != 0
        pp = t.pin_ptr.copy(); pp[0] = 1
        return dataclasses.replace(t, pin_ptr=pp)
    if kind == "ptr_last":  # pin_ptr[P] != n_events
        pp = t.pin_ptr.copy(); pp[-1] -= 1
        return dataclasses.replace(t, pin_ptr=pp)
    if kind == "ptr_far":  # offsets far outside the events: the owner scatter must skip them
        pp = t.pin_ptr.copy(); pp[5] = 1 << 40; pp[7] = -7
        return dataclasses.replace(t, pin_ptr=pp)
    raise ValueError(kind)


@pytest.mark.parametrize("kind", ["unsorted", "value", "value2", "t_max", "negative", "slew", "slew_nan", "init",
                                  "pin_ptr", "ptr_first", "ptr_last", "ptr_far"])
def test_bad_events_rejected_and_previous_data_kept(kind):
    import eda_gate_level_amd as pa
    import oracle

    d, t = _small()
    an = pa.PowerAnalysis()
    try:
        an.load(d, t)
        with pytest.raises(pa.PaError) as ei:
            an.load_events(_mut(t, kind))
        assert ei.value.code == pa.PA_EDATA, str(ei.value)
        an.n_cycles, an.n_events = t.n_cycles, t.n_events
        r = an.run(per_event=True)
        g = dict(r["totals"])
        g.update(wave_J=r["wave_J"].cpu().numpy(), cyc_events=r["cyc_events"].cpu().numpy().astype(np.uint64),
                 cyc_glitches=r["cyc_glitches"].cpu().numpy().astype(np.uint64),
                 evt_glitch=r["evt_glitch"][:t.n_events].cpu().numpy(),
                 evt_state_before=r["evt_state_before"][:t.n_events].cpu().numpy())
        pu.assert_parity(g, oracle.run(d, t), label=f"after rejected {kind}")
    finally:
        an.close()


def test_bad_arguments():
    import torch

    import eda_gate_level_amd as pa

    d, t = _small()
    an = pa.PowerAnalysis()
    try:
        an.load_design(d)
        dev = an.device
        ok = dict(pin_ptr=torch.from_numpy(t.pin_ptr).to(dev), pin_init=torch.from_numpy(t.pin_init).to(dev),
                  evt_t=torch.from_numpy(t.evt_t).to(dev), evt_val=torch.from_numpy(t.evt_val).to(dev),
                  evt_slew=torch.from_numpy(t.evt_slew).to(dev))
        # pin count that does not match the design
        with pytest.raises(pa.PaError) as ei:
            pa.pa_load_events(an.ctx, ok["pin_ptr"][:-1], ok["pin_init"][:-1], ok["evt_t"], ok["evt_val"],
                              ok["evt_slew"], t.t_clk, t.t_max, t.tick_s)
        assert ei.value.code == pa.PA_EINVAL
        for t_clk, t_max, tick in ((0, t.t_max, t.tick_s), (1 << 32, t.t_max, t.tick_s), (t.t_clk, 0, t.tick_s),
                                   (t.t_clk, t.t_max, 0.0)):
            with pytest.raises(pa.PaError) as ei:
                pa.pa_load_events(an.ctx, ok["pin_ptr"], ok["pin_init"], ok["evt_t"], ok["evt_val"], ok["evt_slew"],
                                  t_clk, t_max, tick)
            assert ei.value.code == pa.PA_EINVAL
        # NULL output array
        an.load_events(t)
        with pytest.raises(pa.PaError) as ei:
            pa.pa_run(an.ctx, None, torch.empty(t.n_cycles, dtype=torch.uint64, device=dev),
                      torch.empty(t.n_cycles, dtype=torch.uint64, device=dev))
        assert ei.value.code == pa.PA_EINVAL
        # timing modes: 0..2 only; the pass-only mode fills the whole-pass time alone; the
        # per-kernel mode times each kernel's own execution, inside the whole pass
        for mode in (-1, 3):
            with pytest.raises(pa.PaError) as ei:
                an.set_timing(mode)
            assert ei.value.code == pa.PA_EINVAL
        outs = an.alloc_outputs()
        an.set_timing(2)
        an.run(outs)
        km = an.info()["kernel_ms"]
        assert km[0] == 0.0 and km[1] == 0.0 and km[3] > 0.0
        an.set_timing(1)
        an.run(outs)
        km = an.info()["kernel_ms"]
        assert km[0] > 0.0 and km[1] > 0.0 and km[3] >= km[0] + km[1]
    finally:
        an.close()
    with pytest.raises(pa.PaError) as ei:
        pa.PowerAnalysis(time_kernels=5)
    assert ei.value.code == pa.PA_EINVAL


@pytest.mark.parametrize("kind", ["cell_id", "k0", "k9", "axis"])
def test_bad_design_rejected(kind):
    import eda_gate_level_amd as pa

    d, t = _small()
    if kind == "cell_id":
        gc = d.gate_cell.copy(); gc[3] = d.n_cells; d = dataclasses.replace(d, gate_cell=gc)
    elif kind in ("k0", "k9"):
        k = d.cell_n_in.copy(); k[0] = 0 if kind == "k0" else 9; d = dataclasses.replace(d, cell_n_in=k)
    elif kind == "axis":
        sa = d.slew_axis.copy(); sa[0, 2] = sa[0, 1]; d = dataclasses.replace(d, slew_axis=sa)
    an = pa.PowerAnalysis()
    try:
        with pytest.raises(pa.PaError) as ei:
            an.load_design(d)
        assert ei.value.code == pa.PA_EDATA
    finally:
        an.close()


def test_device_memory_cap_gives_enomem_and_keeps_loaded_data():
    """The debug cap on the context's device memory (pa_tunables.device_mib_cap)
    makes an allocation fail as a real out-of-memory would: the load reports
    PA_ENOMEM, the events loaded before stay usable and give the same results,
    and an uncapped context runs the same trace."""
    import eda_gate_level_amd as pa
    import oracle

    d, t_small = _small()
    w = synth.tiny()
    d_big, t_big = w.design, w.trace
    print("[case] device memory cap", flush=True)
    an = pa.PowerAnalysis(device_mib_cap=1)
    try:
        an.load_design(d)
        an.load_events(t_small)
        before = an.run(per_event=False)
        wave_before = before["wave_J"].cpu().numpy().copy()
        # the same design with ten times the events: more than the 1 MiB cap allows
        tt = synth.poisson_trace(np.random.default_rng(5), np.full(t_small.n_pins, 1.0), 400, t_small.t_clk)
        with pytest.raises(pa.PaError) as ei:
            an.load_events(tt)
        assert ei.value.code == pa.PA_ENOMEM
        assert "out of device memory" in str(ei.value)
        after = an.run(per_event=False)
        # integers and the order-fixed energies repeat exactly; bins and leakage to rounding
        for key in ("n_events", "n_glitches", "e_int_J", "e_sw_J", "e_gl_J"):
            assert after["totals"][key] == before["totals"][key], key
        assert pu.rel_err(after["totals"]["e_leak_J"], before["totals"]["e_leak_J"]) <= 1e-13
        np.testing.assert_allclose(after["wave_J"].cpu().numpy(), wave_before, rtol=1e-13, atol=0)
        with pytest.raises(pa.PaError) as ei:
            an.load_design(d_big)
            an.load_events(t_big)
        assert ei.value.code == pa.PA_ENOMEM
    finally:
        an.close()
    g = pu.gpu_run(d_big, t_big, per_event=False, device_mib_cap=256)
    pu.assert_parity(g, oracle.run(d_big, t_big, per_event=False), per_event=False, label="uncapped")
    with pytest.raises(pa.PaError) as ei:
        pa.PowerAnalysis(device_mib_cap=-1)
    assert ei.value.code == pa.PA_EINVAL
