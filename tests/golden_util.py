"""Build Design/Trace objects from the hand-circuit fixtures in tests/golden/.

Each fixture holds a tiny design and trace, the expected outputs worked out
by hand (see its "hand_derivation"), and the passage of the paper it pins.
"""
import glob
import json
import os

import numpy as np

from workloads.synth import Design, Trace

GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def fixtures():
    return sorted(glob.glob(os.path.join(GOLDEN_DIR, "hc*.json")))


def load(path):
    with open(path) as f:
        spec = json.load(f)
    d, t = spec["design"], spec["trace"]
    ns, nc = d["n_slew"], d["n_cap"]
    cells = d["cells"]
    cell_n_in = np.array([c["k"] for c in cells], np.int32)
    slew_axis = np.array([c["slew_axis"] for c in cells], np.float64)
    cap_axis = np.array([c["cap_axis"] for c in cells], np.float64)
    luts, leaks = [], []
    for c in cells:
        k = c["k"]
        if "lut_const_J" in c:
            const = np.array(c["lut_const_J"], np.float64)  # [2^k][k]
            tab = np.broadcast_to(const[:, :, None, None], (1 << k, k, ns, nc))
        else:
            tab = np.array(c["lut_J"], np.float64).reshape(1 << k, k, ns, nc)
        luts.append(np.ascontiguousarray(tab).reshape(-1))
        leaks.append(np.array(c["leak_W"], np.float64))
    design = Design(gate_cell=np.array([g["cell"] for g in d["gates"]], np.int32),
                    gate_cap_F=np.array([g["cap_F"] for g in d["gates"]], np.float64),
                    cell_n_in=cell_n_in, n_slew=ns, n_cap=nc, slew_axis=slew_axis, cap_axis=cap_axis,
                    lut_J=np.concatenate(luts), leak_W=np.concatenate(leaks), vdd_V=float(d["vdd_V"]))
    pins = t["pins"]
    counts = [len(p["events"]) for p in pins]
    pin_ptr = np.zeros(len(pins) + 1, np.int64)
    pin_ptr[1:] = np.cumsum(counts)
    ev_t, ev_v, ev_s = [], [], []
    for p in pins:
        v = p["init"]
        for tt, ss in p["events"]:
            v = 1 - v
            ev_t.append(tt)
            ev_v.append(v)
            ev_s.append(ss)
    trace = Trace(pin_ptr=pin_ptr, pin_init=np.array([p["init"] for p in pins], np.uint8),
                  evt_t=np.array(ev_t, np.int64), evt_val=np.array(ev_v, np.uint8),
                  evt_slew=np.array(ev_s, np.float32), t_clk=int(t["t_clk"]), t_max=int(t["t_max"]),
                  tick_s=float(t["tick_s"]))
    return spec, design, trace
