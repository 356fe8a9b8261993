"""Host cost of the dispatch layer (rlx-metal 0.2.14 mps_blas.rs, module doc:
the per-call cost of reaching the GPU library decides whether small products
are worth sending there). tests/host_cost.c times mm_gemm and mm_id up to the
point where they would enqueue (validation, extents, overlap, route decision,
launch-family resolution), stopped there by the resolve-failure hook, so it
runs without a GPU."""
import json
import os
import shutil
import subprocess

import pytest

import gemv_expert_id_amd as mm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CASES = ("gemm_f16_8192_nt", "gemv_f16_1x4096_11008", "skinny_f16_8x4096_11008",
         "id_prefill_bf16_512x8_of_64", "id_decode_bf16_1x8_of_64")


def test_dispatch_host_cost_below_a_microsecond(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    libdir = os.path.dirname(os.path.abspath(mm.LIB_PATH))
    if not os.path.exists(os.path.join(libdir, "libmm.so")):
        pytest.skip("libmm.so not built")
    exe = str(tmp_path / "host_cost")
    subprocess.run([gcc, "-O2", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "host_cost.c"), "-L", libdir, "-lmm",
                    "-Wl,-rpath," + libdir, "-o", exe], check=True)
    out = subprocess.run([exe, "20000", "3"], check=True, capture_output=True, text=True,
                         timeout=120).stdout
    res = json.loads(out)
    print(res)
    for name in CASES:
        # Measured about 0.12-0.15 us per call on the build host; the bound
        # leaves room for slow or loaded CI machines.
        assert 0 < res[name] < 1000.0, (name, res[name])
        assert res[name] >= res["hook"], (name, res)
