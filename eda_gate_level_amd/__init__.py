"""MI355X (gfx950) gate-level time-based power analysis.

The C ABI (include/pa.h) lives in libpa.so; `_pa` binds it with the same
names.  `PowerAnalysis` is a thin convenience holder of one context that
moves host arrays to the GPU and calls the ABI (marshalling only).

Method: "GPU-Accelerated Gate-Level Time-Based Power Analysis via
Event-Density-Aware Partitioning and Kernel Fusion" (arXiv 2609.05960).
"""
from __future__ import annotations

from typing import Optional

from ._pa import (EXPORTS, PA_EDATA, PA_EHIP, PA_EINVAL, PA_ENOMEM, PA_ESTATE, PA_OK, PaError, lib, pa_create,
                  pa_destroy, pa_get_info, pa_get_window_stats, pa_last_error, pa_load_design, pa_load_events,
                  pa_pack_text, pa_run, pa_run_gates, pa_run_text, pa_set_stream, pa_set_timing)

__all__ = ["PowerAnalysis", "PaError", "pa_create", "pa_destroy", "pa_set_stream", "pa_set_timing", "pa_last_error",
           "pa_load_design", "pa_load_events", "pa_run", "pa_run_gates", "pa_get_info", "pa_get_window_stats",
           "pa_pack_text", "pa_run_text",
           "lib", "EXPORTS", "PA_OK",
           "PA_EINVAL", "PA_EDATA",
           "PA_ENOMEM", "PA_EHIP", "PA_ESTATE"]


def _dev(a, dtype, device):
    import numpy as np
    import torch

    return torch.from_numpy(np.ascontiguousarray(a)).to(device=device, dtype=dtype)


class PowerAnalysis:
    """One library context on one GPU.  `load(design, trace)` takes host numpy
    arrays (the layout of include/pa.h), `run()` returns the totals and device
    output tensors."""

    def __init__(self, device: int = 0, stream=None, chunk_cycles: int = 0, grid_blocks: int = 0,
                 time_kernels=0, fixed_window_cycles: int = 0, lut_lds_kib: int = 0, device_mib_cap: int = 0,
                 plain_bins: int = 0):
        import torch

        self.device = torch.device("cuda", device)
        if stream is None:
            stream = torch.cuda.current_stream(self.device)
        self.ctx = pa_create(device, stream, chunk_cycles, grid_blocks, time_kernels, fixed_window_cycles,
                             lut_lds_kib, device_mib_cap, plain_bins)
        self.n_cycles = 0
        self.n_events = 0
        self.n_gates = 0

    def set_timing(self, time_kernels: int) -> None:
        """0: none; 1: fused, finalize and pass device times; 2: the pass only."""
        pa_set_timing(self.ctx, time_kernels)

    def close(self):
        if getattr(self, "ctx", None):
            pa_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def load_design(self, d) -> None:
        import torch

        dev = self.device
        pa_load_design(self.ctx, _dev(d.gate_cell, torch.int32, dev), _dev(d.gate_cap_F, torch.float64, dev),
                       _dev(d.cell_n_in, torch.int32, dev), d.n_slew, d.n_cap,
                       _dev(d.slew_axis, torch.float64, dev), _dev(d.cap_axis, torch.float64, dev),
                       _dev(d.lut_J, torch.float64, dev), _dev(d.leak_W, torch.float64, dev), d.vdd_V)
        self.n_gates = int(d.gate_cell.shape[0])

    def load_events(self, t) -> None:
        import torch

        dev = self.device
        pa_load_events(self.ctx, _dev(t.pin_ptr, torch.int64, dev), _dev(t.pin_init, torch.uint8, dev),
                       _dev(t.evt_t, torch.int64, dev), _dev(t.evt_val, torch.uint8, dev),
                       _dev(t.evt_slew, torch.float32, dev), t.t_clk, t.t_max, t.tick_s)
        self.n_cycles = -(-int(t.t_max) // int(t.t_clk))
        self.n_events = int(t.evt_t.shape[0])

    def load(self, design, trace) -> None:
        self.load_design(design)
        self.load_events(trace)

    def alloc_outputs(self, per_event: bool = False, per_gate: bool = False) -> dict:
        import torch

        C, E, dev = self.n_cycles, self.n_events, self.device
        out = dict(wave_J=torch.empty(C, dtype=torch.float64, device=dev),
                   cyc_events=torch.empty(C, dtype=torch.uint64, device=dev),
                   cyc_glitches=torch.empty(C, dtype=torch.uint64, device=dev))
        if per_event:
            out["evt_glitch"] = torch.empty(max(E, 1), dtype=torch.uint8, device=dev)
            out["evt_state_before"] = torch.empty(max(E, 1), dtype=torch.uint8, device=dev)
        if per_gate:
            out["gate_J"] = torch.empty((max(self.n_gates, 1), 4), dtype=torch.float64, device=dev)
        return out

    def run(self, outputs: Optional[dict] = None, per_event: bool = False) -> dict:
        if outputs is None:
            outputs = self.alloc_outputs(per_event)
        self._check_outputs(outputs)
        if "gate_J" in outputs:
            # per-gate energies (internal, switching, glitch, leakage) in a pass of their own
            tot = pa_run_gates(self.ctx, outputs["wave_J"], outputs["cyc_events"], outputs["cyc_glitches"],
                               outputs["gate_J"])
        else:
            tot = pa_run(self.ctx, outputs["wave_J"], outputs["cyc_events"], outputs["cyc_glitches"],
                         outputs.get("evt_glitch"), outputs.get("evt_state_before"))
        return dict(totals=tot, **outputs)

    def _check_outputs(self, outputs: dict) -> None:
        """Every output the pass writes must hold what the loaded data imply:
        C cycles, E events, G x 4 gate rows (ValueError before any launch)."""
        need = dict(wave_J=self.n_cycles, cyc_events=self.n_cycles, cyc_glitches=self.n_cycles,
                    evt_glitch=self.n_events, evt_state_before=self.n_events, gate_J=4 * self.n_gates)
        for key, t in outputs.items():
            if key not in need:
                raise ValueError(f"unknown output {key!r}")
            if t is not None and int(t.numel()) < need[key]:
                raise ValueError(f"{key}: {int(t.numel())} elements, needs at least {need[key]}")

    def run_text(self, text, t_clk: int, t_max: int, tick_s: float = 1e-15, segment_cycles: int = 0,
                 n_threads: int = 0, serial: bool = False) -> dict:
        """Power analysis of VCD-like activity text (host bytes), packed on host
        threads segment by segment while the GPU computes the previous one.
        Needs a loaded design; leaves no events loaded."""
        import torch

        C, dev = -(-int(t_max) // int(t_clk)), self.device
        outs = dict(wave_J=torch.empty(C, dtype=torch.float64, device=dev),
                    cyc_events=torch.empty(C, dtype=torch.uint64, device=dev),
                    cyc_glitches=torch.empty(C, dtype=torch.uint64, device=dev))
        tot, st = pa_run_text(self.ctx, text, t_clk, t_max, tick_s, outs["wave_J"], outs["cyc_events"],
                              outs["cyc_glitches"], segment_cycles, n_threads, serial)
        self.n_cycles, self.n_events = 0, 0
        return dict(totals=tot, stats=st, **outs)

    def window_stats(self) -> dict:
        """Events per (chunk, gate, window) of the loaded layout: count, mean, p50/p90/p99, max."""
        return pa_get_window_stats(self.ctx)

    def info(self) -> dict:
        return pa_get_info(self.ctx)
