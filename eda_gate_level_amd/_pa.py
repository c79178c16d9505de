"""ctypes binding of the C ABI in include/pa.h (argument marshalling only).

Every entry point keeps its C name.  Array arguments are torch tensors on the
context's GPU; the binding checks dtype, device and contiguity and passes
data pointers.  Every step of the power analysis runs in libpa.so's gfx950
kernels; there is no fallback: importing this module fails loudly when the
library is missing.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpa.so")

PA_OK, PA_EINVAL, PA_EDATA, PA_ENOMEM, PA_EHIP, PA_ESTATE = 0, -1, -2, -3, -4, -5
PA_NOALLOC_SCRATCH_BYTES = 16 * 1024 * 1024  # the fixed device scratch of pa_run_noalloc
_NAMES = {PA_EINVAL: "PA_EINVAL", PA_EDATA: "PA_EDATA", PA_ENOMEM: "PA_ENOMEM", PA_EHIP: "PA_EHIP",
          PA_ESTATE: "PA_ESTATE"}

EXPORTS = ("pa_create", "pa_destroy", "pa_set_stream", "pa_set_timing", "pa_last_error", "pa_load_design",
           "pa_load_events", "pa_run", "pa_run_noalloc", "pa_run_gates", "pa_get_info", "pa_get_window_stats",
           "pa_pack_text", "pa_run_text")


class PaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{_NAMES.get(code, code)}: {msg}")
        self.code = code


class pa_tunables(C.Structure):
    _fields_ = [("chunk_cycles", C.c_int32), ("grid_blocks", C.c_int32), ("time_kernels", C.c_int32),
                ("fixed_window_cycles", C.c_int32), ("lut_lds_kib", C.c_int32), ("device_mib_cap", C.c_int32),
                ("plain_bins", C.c_int32)]


class pa_totals(C.Structure):
    _fields_ = [("p_int_W", C.c_double), ("p_sw_W", C.c_double), ("p_gl_W", C.c_double), ("p_leak_W", C.c_double),
                ("e_int_J", C.c_double), ("e_sw_J", C.c_double), ("e_gl_J", C.c_double), ("e_leak_J", C.c_double),
                ("n_events", C.c_uint64), ("n_glitches", C.c_uint64), ("n_cycles", C.c_int64)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


class pa_window_stats(C.Structure):
    _fields_ = [("n_windows", C.c_int64), ("mean", C.c_double), ("p50", C.c_int64), ("p90", C.c_int64),
                ("p99", C.c_int64), ("max", C.c_int64)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


class pa_info(C.Structure):
    _fields_ = [("n_gates", C.c_int64), ("n_pins", C.c_int64), ("n_events", C.c_int64), ("n_cycles", C.c_int64),
                ("chunk_cycles", C.c_int32), ("n_chunks", C.c_int32), ("grid_blocks", C.c_int32),
                ("block_threads", C.c_int32), ("batch_events", C.c_int32), ("max_segment_events", C.c_int32),
                ("device_bytes", C.c_int64), ("kernel_ms", C.c_float * 4), ("n_windows", C.c_int64),
                ("n_slots", C.c_int64), ("wave_steps_max", C.c_int32), ("wave_steps_mean", C.c_float),
                ("tables_in_lds", C.c_int32), ("walk_kernel", C.c_int32)]

    def as_dict(self):
        d = {f: getattr(self, f) for f, _ in self._fields_ if f != "kernel_ms"}
        d["kernel_ms"] = list(self.kernel_ms)
        return d


class pa_text_opts(C.Structure):
    _fields_ = [("segment_cycles", C.c_int32), ("n_threads", C.c_int32), ("serial", C.c_int32),
                ("reserved", C.c_int32)]


class pa_text_stats(C.Structure):
    _fields_ = [("n_segments", C.c_int64), ("n_events", C.c_int64), ("max_segment_events", C.c_int64),
                ("text_bytes", C.c_int64), ("header_s", C.c_double), ("index_s", C.c_double),
                ("parse_s", C.c_double), ("gpu_s", C.c_double), ("wall_s", C.c_double)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


def load_library(path: str = LIB_PATH) -> C.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"libpa.so not built ({path}); run __graft_entry__.build() or python -m "
                          f"eda_gate_level_amd.build")
    L = C.CDLL(path)
    P = C.c_void_p
    i64, i32, dbl = C.c_int64, C.c_int32, C.c_double
    L.pa_create.argtypes = [C.POINTER(P), C.c_int, P, C.POINTER(pa_tunables)]
    L.pa_destroy.argtypes = [P]
    L.pa_destroy.restype = None
    L.pa_set_stream.argtypes = [P, P]
    L.pa_set_timing.argtypes = [P, i32]
    L.pa_last_error.restype = C.c_char_p
    L.pa_last_error.argtypes = []
    L.pa_load_design.argtypes = [P, i64, P, P, i32, P, i32, i32, P, P, P, P, dbl]
    L.pa_load_events.argtypes = [P, i64, i64, P, P, P, P, P, i64, i64, dbl]
    L.pa_run.argtypes = [P, C.POINTER(pa_totals), P, P, P, P, P]
    L.pa_run_noalloc.argtypes = [P, C.POINTER(pa_totals), P, P, P, P, P]
    L.pa_run_gates.argtypes = [P, C.POINTER(pa_totals), P, P, P, P]
    L.pa_get_info.argtypes = [P, C.POINTER(pa_info)]
    L.pa_get_window_stats.argtypes = [P, C.POINTER(pa_window_stats)]
    L.pa_pack_text.argtypes = [P, i64, i64, i32, i64, C.POINTER(i64), P, P, P, P, P]
    L.pa_run_text.argtypes = [P, P, i64, i64, i64, dbl, C.POINTER(pa_text_opts), C.POINTER(pa_totals), P, P, P,
                              C.POINTER(pa_text_stats)]
    for name in ("pa_create", "pa_set_stream", "pa_set_timing", "pa_load_design", "pa_load_events", "pa_run",
                 "pa_run_noalloc", "pa_run_gates", "pa_get_info", "pa_get_window_stats", "pa_pack_text", "pa_run_text"):
        getattr(L, name).restype = C.c_int
    return L


_lib: Optional[C.CDLL] = None


def lib() -> C.CDLL:
    global _lib
    if _lib is None:
        _lib = load_library()
    return _lib


def _check(rc: int):
    if rc != PA_OK:
        raise PaError(rc, lib().pa_last_error().decode(errors="replace"))


def _ptr(t, dtype, device=None, name="array"):
    import torch

    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, context is on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return C.c_void_p(t.data_ptr())


def _numel(t, name):
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    return int(t.numel())


def _need(t, n: int, name: str, exact: bool = True) -> None:
    """Size check before any pointer crosses the ABI: the library reads and
    writes these arrays by the sizes the loaded design and events imply, so a
    short array would be read or written out of bounds on the device."""
    if t is None:
        return
    m = _numel(t, name)
    if (m != n) if exact else (m < n):
        raise ValueError(f"{name}: {m} elements, {'expected' if exact else 'needs at least'} {n}")


def _design_sizes(cell_n_in, n_slew: int, n_cap: int):
    """LUT and leakage entries the cell library needs: sum over cells of
    2^k * k * n_slew * n_cap and of 2^k (k = input count, 1..8).  None when
    an input count is outside 1..8: the library then rejects the design
    (PA_EDATA) before it reads any table."""
    k = cell_n_in.detach().to("cpu").tolist()
    if any((not isinstance(x, int)) or x < 1 or x > 8 for x in k):
        return None
    return sum((1 << x) * x * n_slew * n_cap for x in k), sum(1 << x for x in k)


def _outputs_for(ctx):
    """(cycles, events, gates) of the context's loaded data."""
    info = pa_info()
    _check(lib().pa_get_info(ctx, C.byref(info)))
    return int(info.n_cycles), int(info.n_events), int(info.n_gates)


def _stream_handle(stream) -> C.c_void_p:
    if stream is None:
        return C.c_void_p(None)
    if isinstance(stream, int):
        return C.c_void_p(stream)
    return C.c_void_p(stream.cuda_stream)


def pa_create(device: int = 0, stream=None, chunk_cycles: int = 0, grid_blocks: int = 0,
              time_kernels=0, fixed_window_cycles: int = 0, lut_lds_kib: int = 0,
              device_mib_cap: int = 0, plain_bins: int = 0) -> C.c_void_p:
    t = pa_tunables(chunk_cycles, grid_blocks, int(time_kernels), int(fixed_window_cycles), int(lut_lds_kib),
                    int(device_mib_cap), int(plain_bins))
    h = C.c_void_p()
    _check(lib().pa_create(C.byref(h), int(device), _stream_handle(stream), C.byref(t)))
    return h


def pa_destroy(ctx) -> None:
    if ctx:
        lib().pa_destroy(ctx)


def pa_set_stream(ctx, stream) -> None:
    _check(lib().pa_set_stream(ctx, _stream_handle(stream)))


def pa_set_timing(ctx, time_kernels: int) -> None:
    _check(lib().pa_set_timing(ctx, int(time_kernels)))


def pa_last_error() -> str:
    return lib().pa_last_error().decode(errors="replace")


def pa_load_design(ctx, gate_cell, gate_cap_F, cell_n_in, n_slew: int, n_cap: int, slew_axis, cap_axis, lut_J,
                   leak_W, vdd_V: float) -> None:
    import torch

    G, nc = _numel(gate_cell, "gate_cell"), _numel(cell_n_in, "cell_n_in")
    _need(gate_cap_F, G, "gate_cap_F")
    _need(slew_axis, nc * int(n_slew), "slew_axis")
    _need(cap_axis, nc * int(n_cap), "cap_axis")
    if nc and 2 <= int(n_slew) <= 16 and 2 <= int(n_cap) <= 16:
        sizes = _design_sizes(cell_n_in, int(n_slew), int(n_cap))
        if sizes is not None:
            _need(lut_J, sizes[0], "lut_J")
            _need(leak_W, sizes[1], "leak_W")
    _check(lib().pa_load_design(ctx, int(gate_cell.numel()), _ptr(gate_cell, torch.int32, name="gate_cell"),
                                _ptr(gate_cap_F, torch.float64, name="gate_cap_F"), int(cell_n_in.numel()),
                                _ptr(cell_n_in, torch.int32, name="cell_n_in"), int(n_slew), int(n_cap),
                                _ptr(slew_axis, torch.float64, name="slew_axis"),
                                _ptr(cap_axis, torch.float64, name="cap_axis"),
                                _ptr(lut_J, torch.float64, name="lut_J"), _ptr(leak_W, torch.float64, name="leak_W"),
                                float(vdd_V)))


def pa_load_events(ctx, pin_ptr, pin_init, evt_t, evt_val, evt_slew, t_clk: int, t_max: int,
                   tick_s: float) -> None:
    import torch

    P, E = _numel(pin_init, "pin_init"), _numel(evt_t, "evt_t")
    _need(pin_ptr, P + 1, "pin_ptr")
    _need(evt_val, E, "evt_val")
    _need(evt_slew, E, "evt_slew")
    _check(lib().pa_load_events(ctx, int(pin_init.numel()), int(evt_t.numel()),
                                _ptr(pin_ptr, torch.int64, name="pin_ptr"), _ptr(pin_init, torch.uint8, name="pin_init"),
                                _ptr(evt_t, torch.int64, name="evt_t"), _ptr(evt_val, torch.uint8, name="evt_val"),
                                _ptr(evt_slew, torch.float32, name="evt_slew"), int(t_clk), int(t_max),
                                float(tick_s)))


def pa_run(ctx, wave_J, cyc_events, cyc_glitches, evt_glitch=None, evt_state_before=None) -> dict:
    import torch

    Cn, E, _ = _outputs_for(ctx)
    for t, name in ((wave_J, "wave_J"), (cyc_events, "cyc_events"), (cyc_glitches, "cyc_glitches")):
        _need(t, Cn, name, exact=False)
    for t, name in ((evt_glitch, "evt_glitch"), (evt_state_before, "evt_state_before")):
        _need(t, E, name, exact=False)
    tot = pa_totals()
    _check(lib().pa_run(ctx, C.byref(tot), _ptr(wave_J, torch.float64, name="wave_J"),
                        _ptr(cyc_events, torch.uint64, name="cyc_events"),
                        _ptr(cyc_glitches, torch.uint64, name="cyc_glitches"),
                        _ptr(evt_glitch, torch.uint8, name="evt_glitch"),
                        _ptr(evt_state_before, torch.uint8, name="evt_state_before")))
    return tot.as_dict()


def pa_run_noalloc(ctx, wave_J, cyc_events, cyc_glitches, evt_glitch=None, evt_state_before=None) -> dict:
    import torch

    Cn, E, _ = _outputs_for(ctx)
    for t, name in ((wave_J, "wave_J"), (cyc_events, "cyc_events"), (cyc_glitches, "cyc_glitches")):
        _need(t, Cn, name, exact=False)
    for t, name in ((evt_glitch, "evt_glitch"), (evt_state_before, "evt_state_before")):
        _need(t, E, name, exact=False)
    tot = pa_totals()
    _check(lib().pa_run_noalloc(ctx, C.byref(tot), _ptr(wave_J, torch.float64, name="wave_J"),
                                _ptr(cyc_events, torch.uint64, name="cyc_events"),
                                _ptr(cyc_glitches, torch.uint64, name="cyc_glitches"),
                                _ptr(evt_glitch, torch.uint8, name="evt_glitch"),
                                _ptr(evt_state_before, torch.uint8, name="evt_state_before")))
    return tot.as_dict()


def pa_run_gates(ctx, wave_J, cyc_events, cyc_glitches, gate_J) -> dict:
    import torch

    Cn, _, G = _outputs_for(ctx)
    for t, name in ((wave_J, "wave_J"), (cyc_events, "cyc_events"), (cyc_glitches, "cyc_glitches")):
        _need(t, Cn, name, exact=False)
    _need(gate_J, 4 * G, "gate_J", exact=False)
    tot = pa_totals()
    _check(lib().pa_run_gates(ctx, C.byref(tot), _ptr(wave_J, torch.float64, name="wave_J"),
                              _ptr(cyc_events, torch.uint64, name="cyc_events"),
                              _ptr(cyc_glitches, torch.uint64, name="cyc_glitches"),
                              _ptr(gate_J, torch.float64, name="gate_J")))
    return tot.as_dict()


def pa_get_window_stats(ctx) -> dict:
    st = pa_window_stats()
    _check(lib().pa_get_window_stats(ctx, C.byref(st)))
    return st.as_dict()


def pa_get_info(ctx) -> dict:
    info = pa_info()
    _check(lib().pa_get_info(ctx, C.byref(info)))
    return info.as_dict()


def _text_ptr(text):
    """Host address and length of activity text given as bytes, bytearray or a uint8 numpy array."""
    import numpy as np

    if isinstance(text, bytes):
        return C.c_void_p(C.cast(C.c_char_p(text), C.c_void_p).value), len(text), text
    if isinstance(text, bytearray):
        buf = (C.c_char * len(text)).from_buffer(text)
        return C.c_void_p(C.addressof(buf)), len(text), buf
    a = np.ascontiguousarray(text, dtype=np.uint8)
    return C.c_void_p(a.ctypes.data), int(a.size), a


def pa_pack_text(text, n_pins: int, n_threads: int = 0) -> dict:
    """Host CSR of the text's events (numpy arrays): pin_ptr, pin_init, evt_t, evt_val, evt_slew."""
    import numpy as np

    ptr, n, keep = _text_ptr(text)
    ne = C.c_int64(0)
    _check(lib().pa_pack_text(ptr, n, int(n_pins), int(n_threads), 0, C.byref(ne), None, None, None, None, None))
    E = int(ne.value)
    out = dict(pin_ptr=np.empty(n_pins + 1, np.int64), pin_init=np.empty(n_pins, np.uint8),
               evt_t=np.empty(max(E, 1), np.int64), evt_val=np.empty(max(E, 1), np.uint8),
               evt_slew=np.empty(max(E, 1), np.float32))
    _check(lib().pa_pack_text(ptr, n, int(n_pins), int(n_threads), max(E, 1), C.byref(ne),
                              *(C.c_void_p(out[k].ctypes.data) for k in ("pin_ptr", "pin_init", "evt_t", "evt_val",
                                                                          "evt_slew"))))
    del keep
    for k in ("evt_t", "evt_val", "evt_slew"):
        out[k] = out[k][:E]
    return out


def pa_run_text(ctx, text, t_clk: int, t_max: int, tick_s: float, wave_J, cyc_events, cyc_glitches,
                segment_cycles: int = 0, n_threads: int = 0, serial: bool = False):
    """Totals and packing statistics of the text's power analysis (outputs written to the device tensors)."""
    import torch

    if int(t_clk) >= 1 and int(t_max) >= 1:
        Cn = -(-int(t_max) // int(t_clk))
        for t, name in ((wave_J, "wave_J"), (cyc_events, "cyc_events"), (cyc_glitches, "cyc_glitches")):
            _need(t, Cn, name, exact=False)
    ptr, n, keep = _text_ptr(text)
    opts = pa_text_opts(int(segment_cycles), int(n_threads), int(bool(serial)), 0)
    tot, st = pa_totals(), pa_text_stats()
    _check(lib().pa_run_text(ctx, ptr, n, int(t_clk), int(t_max), float(tick_s), C.byref(opts), C.byref(tot),
                             _ptr(wave_J, torch.float64, name="wave_J"),
                             _ptr(cyc_events, torch.uint64, name="cyc_events"),
                             _ptr(cyc_glitches, torch.uint64, name="cyc_glitches"), C.byref(st)))
    del keep
    return tot.as_dict(), st.as_dict()
