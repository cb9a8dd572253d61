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


def cover_tokens(ids, E, block_m, full_upto=512, group_rows=32, seed=0):
    """Tokens whose rows touch every (expert, row block, 32-row group) cell of
    the dispatch at `block_m` -- every active expert, every scheduled row
    block, every row group of a block (so both passes of a block that takes
    two) -- plus the first and last token. All tokens when T <= full_upto.

    ids: int32 [T, K] (negative = masked). Greedy set cover over the cells
    (ties broken by a seeded shuffle of the tokens); the rows come from the
    oracle's dispatch, so the choice does not depend on the GPU tables."""
    ids = np.asarray(ids, np.int32)
    T, K = ids.shape
    if T <= full_upto:
        return np.arange(T, dtype=np.int32)
    tab = oracle.dispatch(ids, None, E, block_m)
    sizes, offs = tab["group_sizes"], tab["group_offsets"]
    n = tab["n_valid"]
    expert_of_row = np.repeat(np.arange(E), sizes)
    local = np.arange(n) - offs[expert_of_row]
    groups_per_block = (block_m + group_rows - 1) // group_rows
    cell_of_row = (expert_of_row.astype(np.int64) * (T * K // block_m + 2) + local // block_m) \
        * groups_per_block + (local % block_m) // group_rows
    _, cell_of_row = np.unique(cell_of_row, return_inverse=True)
    n_cells = int(cell_of_row.max()) + 1 if n else 0
    pos = tab["token_topk_to_pos"]                         # [T, K]
    tok_cells = np.where(pos >= 0, cell_of_row[np.maximum(pos, 0)], n_cells)
    covered = np.zeros(n_cells + 1, bool)
    covered[n_cells] = True                                # the masked-slot sentinel
    chosen = [0, T - 1]
    for t in chosen:
        covered[tok_cells[t]] = True
    order = np.random.default_rng(seed).permutation(T)
    cand = tok_cells[order]
    while not covered.all():
        gain = (~covered[cand]).sum(axis=1)
        j = int(np.argmax(gain))
        chosen.append(int(order[j]))
        covered[cand[j]] = True
    return np.array(sorted(set(chosen)), np.int32)
