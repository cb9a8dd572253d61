"""Helpers shared by the GPU parity tests: storage conversion for the oracle,
the graded error metrics and tolerances."""
import numpy as np
import torch

import oracle

# Tolerances of the forward (graded bar): 16-bit outputs against the fp32
# oracle, max |diff| <= 2e-2 and rel-L2 <= 5e-3; the fp32 path rel-L2 <= 1e-4.
MAX_ABS_16 = 2e-2
REL_L2_16 = 5e-3
REL_L2_32 = 1e-4

ORACLE_DT = {torch.float16: oracle.F16, torch.bfloat16: oracle.BF16, torch.float32: oracle.F32,
             torch.float8_e4m3fn: oracle.FP8}


def storage(t):
    """A torch tensor as the oracle's host storage (uint8 / uint16 bits or float32)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    if t.dtype in (torch.float16, torch.bfloat16):
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def to_f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def metrics(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    diff = got - ref
    max_abs = float(np.max(np.abs(diff))) if diff.size else 0.0
    rel = float(np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-30)) if diff.size else 0.0
    return max_abs, rel


def assert_close_16(got, ref, what=""):
    assert not np.any(np.isnan(got)), "%s: NaN in output (unwritten or bad value)" % what
    max_abs, rel = metrics(got, ref)
    assert max_abs <= MAX_ABS_16 and rel <= REL_L2_16, \
        "%s: max|d|=%.3e rel-L2=%.3e" % (what, max_abs, rel)
    return max_abs, rel


def round_like(x_f32, dtype):
    """Round an fp32 numpy array to `dtype` with torch (RNE) and back to f64."""
    return torch.from_numpy(np.asarray(x_f32, np.float32)).to(dtype).double().numpy()


def gpu_available():
    return torch.cuda.is_available()
