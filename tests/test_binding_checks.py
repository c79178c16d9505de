"""CPU checks of the binding's size checks: arrays whose lengths do not match
what the design and events imply are refused with ValueError before any
pointer crosses the C ABI (a short array would otherwise be read or written
out of bounds on the device).  Nothing here touches a GPU: the checks run
before the binding's device and dtype checks and before any library call."""
import numpy as np
import pytest
import torch

import eda_gate_level_amd as pa
from eda_gate_level_amd import _pa


def _design_arrays(n_cells=3, ks=(1, 2, 4), G=5, ns=7, nc=7):
    k = torch.tensor(list(ks), dtype=torch.int32)
    n_lut = sum((1 << x) * x * ns * nc for x in ks)
    n_leak = sum(1 << x for x in ks)
    return dict(gate_cell=torch.zeros(G, dtype=torch.int32), gate_cap_F=torch.ones(G, dtype=torch.float64),
                cell_n_in=k, n_slew=ns, n_cap=nc, slew_axis=torch.zeros(n_cells * ns, dtype=torch.float64),
                cap_axis=torch.zeros(n_cells * nc, dtype=torch.float64),
                lut_J=torch.zeros(n_lut, dtype=torch.float64), leak_W=torch.zeros(n_leak, dtype=torch.float64),
                vdd_V=0.8)


def _call_design(a):
    _pa.pa_load_design(None, a["gate_cell"], a["gate_cap_F"], a["cell_n_in"], a["n_slew"], a["n_cap"],
                       a["slew_axis"], a["cap_axis"], a["lut_J"], a["leak_W"], a["vdd_V"])


@pytest.mark.parametrize("field,delta", [("gate_cap_F", -1), ("slew_axis", 1), ("cap_axis", -1), ("lut_J", -1),
                                         ("lut_J", 1), ("leak_W", -1)])
def test_design_sizes_refused(field, delta):
    a = _design_arrays()
    n = a[field].numel() + delta
    a[field] = torch.zeros(n, dtype=a[field].dtype)
    with pytest.raises(ValueError, match=field):
        _call_design(a)


def test_design_sizes_consistent_reach_the_device_checks():
    # correct sizes pass the size checks and stop at the next check: CPU tensors
    with pytest.raises(ValueError, match="GPU tensor"):
        _call_design(_design_arrays())


def test_design_bad_input_count_left_to_the_library():
    # an input count outside 1..8 is the library's PA_EDATA (it rejects the
    # design before reading any table): the binding does not size the tables
    a = _design_arrays()
    a["cell_n_in"] = torch.tensor([1, 9, 2], dtype=torch.int32)
    a["lut_J"] = torch.zeros(3, dtype=torch.float64)
    with pytest.raises(ValueError, match="GPU tensor"):
        _call_design(a)


@pytest.mark.parametrize("field", ["pin_ptr", "evt_val", "evt_slew"])
def test_event_sizes_refused(field):
    P, E = 6, 10
    arrs = dict(pin_ptr=torch.zeros(P + 1, dtype=torch.int64), pin_init=torch.zeros(P, dtype=torch.uint8),
                evt_t=torch.zeros(E, dtype=torch.int64), evt_val=torch.zeros(E, dtype=torch.uint8),
                evt_slew=torch.zeros(E, dtype=torch.float32))
    arrs[field] = arrs[field][:-1].clone()
    with pytest.raises(ValueError, match=field):
        _pa.pa_load_events(None, arrs["pin_ptr"], arrs["pin_init"], arrs["evt_t"], arrs["evt_val"],
                           arrs["evt_slew"], 1000, 10000, 1e-15)


def _bare_analysis(C=12, E=30, G=4):
    an = object.__new__(pa.PowerAnalysis)
    an.ctx = None
    an.device = torch.device("cpu")
    an.n_cycles, an.n_events, an.n_gates = C, E, G
    return an


@pytest.mark.parametrize("key,n", [("wave_J", 11), ("cyc_events", 0), ("cyc_glitches", 5), ("evt_glitch", 29),
                                   ("evt_state_before", 1), ("gate_J", 15)])
def test_run_outputs_too_small(key, n):
    an = _bare_analysis()
    outs = dict(wave_J=torch.empty(12, dtype=torch.float64), cyc_events=torch.empty(12, dtype=torch.int64),
                cyc_glitches=torch.empty(12, dtype=torch.int64))
    outs[key] = torch.empty(n, dtype=torch.float64)
    with pytest.raises(ValueError, match=key):
        an.run(outs)


def test_run_unknown_output_refused():
    an = _bare_analysis()
    with pytest.raises(ValueError, match="unknown"):
        an.run(dict(wave=torch.empty(12, dtype=torch.float64)))


def test_text_outputs_too_small():
    w = torch.empty(9, dtype=torch.float64)
    c = torch.empty(10, dtype=torch.int64)
    with pytest.raises(ValueError, match="wave_J"):
        _pa.pa_run_text(None, b"", 100, 1000, 1e-15, w, c, c)
    assert np.ceil(1000 / 100) == 10
