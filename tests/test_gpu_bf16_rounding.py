"""The library rounds fp32 to bf16 (every bf16 output of the GEMM epilogues
and the reduce) with gfx950's conversion instruction. This checks that
instruction, through the library's own conversion function, against the
integer round-to-nearest-even on all 2^32 fp32 bit patterns on the GPU: every
non-NaN input must give identical bits and every NaN must stay a NaN (the
`bf16-rounding` mode of the C++ driver, which the build compiles)."""
import os
import subprocess

import pytest

from helpers import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

DRIVER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "mixture_experts_routed_moe_amd", "moe_bench_driver")


def test_bf16_conversion_is_round_to_nearest_even_on_every_input():
    assert os.path.exists(DRIVER), "build the library first (it builds the driver)"
    r = subprocess.run([DRIVER, "bf16-rounding"], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr)
    assert "non-NaN mismatches 0 " in r.stdout, r.stdout
    assert "NaN inputs not NaN 0" in r.stdout, r.stdout
    assert r.returncode == 0
