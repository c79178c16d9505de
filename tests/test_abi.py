"""CPU checks of the C-ABI library: it loads, exports every entry point that
include/pa.h declares, and its exact cycle division (Granlund-Montgomery
multiply-high) equals plain integer division bit for bit."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pa.h")
LIB = os.path.join(ROOT, "eda_gate_level_amd", "libpa.so")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def libpa():
    if not os.path.exists(LIB):
        from eda_gate_level_amd import build

        build.build()
    return ctypes.CDLL(LIB)


def test_header_declares_the_abi():
    names = declared_functions()
    for n in ("pa_create", "pa_destroy", "pa_load_design", "pa_load_events", "pa_run", "pa_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol(libpa):
    for name in declared_functions():
        assert hasattr(libpa, name), name


def test_binding_names_match_header():
    from eda_gate_level_amd import _pa

    assert sorted(_pa.EXPORTS) == declared_functions()


def test_create_without_gpu_fails_cleanly(libpa):
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    from eda_gate_level_amd import _pa

    with pytest.raises(_pa.PaError) as ei:
        _pa.pa_create(0)
    assert ei.value.code in (_pa.PA_EINVAL, _pa.PA_EHIP)


DIV_TEST = r"""
#include "pa_common.h"
#include <cstdio>
#include <cstdint>
#include <random>
int main() {
  std::mt19937_64 rng(12345);
  const uint32_t ds[] = {1u, 2u, 3u, 5u, 7u, 10u, 997u, 1000u, 4096u, 65535u, 65536u, 100000u, 500000u,
                         1000000u, 999983u, 1u << 31, (1u << 31) + 1u, 4294967291u, 4294967295u};
  long bad = 0, n = 0;
  for (uint32_t d : ds) {
    pa::DivU32 D = pa::make_divu32(d);
    for (uint64_t x = 0; x < 200000; ++x) { uint32_t v = (uint32_t)x; bad += pa::divu32(v, D) != v / d; ++n; }
    for (int k = 0; k < 200000; ++k) { uint32_t v = (uint32_t)rng(); bad += pa::divu32(v, D) != v / d; ++n; }
    for (uint64_t m = 1; m * d <= 0xFFFFFFFFull && m < 5000; ++m) {
      for (int o = -1; o <= 1; ++o) {
        uint64_t v = m * d + o; if (v > 0xFFFFFFFFull) continue;
        bad += pa::divu32((uint32_t)v, D) != (uint32_t)v / d; ++n;
      }
    }
    uint32_t top = 0xFFFFFFFFu; bad += pa::divu32(top, D) != top / d; ++n;
  }
  for (int k = 0; k < 300000; ++k) {
    uint32_t d = (uint32_t)rng() | 1u; if ((k & 1) == 0) d = (uint32_t)(rng() % 2000000) + 1u;
    uint32_t v = (uint32_t)rng();
    pa::DivU32 D = pa::make_divu32(d); bad += pa::divu32(v, D) != v / d; ++n;
  }
  printf("%ld %ld\n", bad, n);
  return bad != 0;
}
"""


def test_cycle_division_is_exact(tmp_path):
    src = tmp_path / "div.cpp"
    src.write_text(DIV_TEST)
    exe = tmp_path / "div"
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    r = subprocess.run([hipcc, "-O2", "-std=c++17", "-x", "hip", "--offload-arch=gfx950", f"-I{ROOT}/include",
                        f"-I{ROOT}/eda_gate_level_amd/csrc", "-o", str(exe), str(src)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    bad, n = map(int, out.stdout.split())
    assert out.returncode == 0 and bad == 0 and n > 1_000_000
