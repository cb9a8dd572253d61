"""moe_dispatch on the GPU against the oracle: every table bit-exact."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as S
from helpers import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

DEV = "cuda:0"
BMS = [16, 32, 64, 128, 256]


def _mr():
    import mixture_experts_routed_moe_amd as mr
    return mr


def _compare(ids, w, E, BM):
    mr = _mr()
    ids_d = torch.from_numpy(ids).to(DEV)
    w_d = None if w is None else torch.from_numpy(w).to(DEV)
    t = mr.moe_dispatch(ids_d, w_d, E, block_m=BM)
    torch.cuda.synchronize()
    ref = oracle.dispatch(np.where(ids >= E, -1, ids), w, E, BM)
    n = ref["n_valid"]
    for k in ("group_sizes", "group_offsets", "group_padded_offsets", "block_expert"):
        assert np.array_equal(t.tensor(k).cpu().numpy(), ref[k]), k
    assert np.array_equal(t.token_topk_to_pos.cpu().numpy(), ref["token_topk_to_pos"].reshape(-1))
    for k in ("sorted_pair", "sorted_token"):
        assert np.array_equal(t.tensor(k)[:n].cpu().numpy(), ref[k][:n]), k
    got_w = t.sorted_weight[:n].cpu().numpy().view(np.uint32)
    assert np.array_equal(got_w, ref["sorted_weight"][:n].view(np.uint32))
    wt = np.ones(ids.size, np.float32) if w is None else w.reshape(-1)
    assert np.array_equal(t.topk_weights.cpu().numpy().view(np.uint32), wt.view(np.uint32))
    # the scheduling list: every block that holds rows, ascending
    sizes, pad = ref["group_sizes"], ref["group_padded_offsets"]
    active = [pad[e] // BM + j for e in range(E) for j in range(-(-int(sizes[e]) // BM))]
    cnt = int(t.active_count.item())
    assert cnt == len(active)
    assert t.active_blocks[:cnt].cpu().tolist() == active
    return t


def _random(T, K, E, mask, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, E, size=(T, K)).astype(np.int32)
    if mask:
        ids[rng.random((T, K)) < mask] = -1
    return ids, rng.random((T, K)).astype(np.float32)


@pytest.mark.parametrize("BM", BMS)
@pytest.mark.parametrize("T,K,E,mask", [(1, 1, 1, 0.0), (5, 2, 3, 0.0), (37, 8, 16, 0.2),
                                         (300, 8, 256, 0.05), (2000, 6, 1000, 0.1),
                                         (129, 8, 1024, 0.0), (40, 4, 5, 1.0),
                                         (128, 8, 64, 0.1), (205, 5, 40, 0.0)])
def test_dispatch_random(T, K, E, mask, BM):
    ids, w = _random(T, K, E, mask, seed=T * 3 + K + E)
    _compare(ids, w, E, BM)


@pytest.mark.parametrize("ci", range(5))
def test_dispatch_workloads(ci):
    cfg = S.CONFIGS[ci]
    d = S.make_moe_inputs(cfg, weights=False)
    ids, w = d["topk_ids"].numpy(), d["topk_weights"].numpy()
    for BM in BMS:
        _compare(ids, w, cfg["E"], BM)


def test_dispatch_many_chunks_single_hot_expert():
    ids = np.full((16384, 8), 7, np.int32)
    ids[::5, 3] = 200
    _compare(ids, None, 256, 128)


def test_dispatch_flags_ids_out_of_range():
    ids, w = _random(64, 4, 8, 0.0, seed=1)
    ids[3, 1] = 8
    ids[10, 0] = 1000
    t = _compare(ids, w, 8, 32)
    assert int(t.status.item()) == 1
    ids2, w2 = _random(64, 4, 8, 0.0, seed=2)
    t2 = _compare(ids2, w2, 8, 32)
    assert int(t2.status.item()) == 0


def test_dispatch_is_repeatable():
    mr = _mr()
    ids, w = _random(4096, 8, 256, 0.0, seed=3)
    ids_d, w_d = torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV)
    t1 = mr.moe_dispatch(ids_d, w_d, 256, block_m=32)
    a = t1.buffer.clone()
    t2 = mr.moe_dispatch(ids_d, w_d, 256, block_m=32, tables=t1)
    assert t2 is t1
    P = 4096 * 8
    for k in ("sorted_pair", "token_topk_to_pos", "block_expert"):
        v = t1.tensor(k)
        off = v.data_ptr() - t1.buffer.data_ptr()
        assert torch.equal(a[off:off + 4 * v.numel()], t1.buffer[off:off + 4 * v.numel()]), k
    assert P == t1.T * t1.K
