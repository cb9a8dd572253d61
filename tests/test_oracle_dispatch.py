"""Pins for the oracle's expert-sorted dispatch (CPU only).

Against:
  * the worked examples printed on the tilelang-baseline MoE walkthrough,
    section 'forward' (tests/golden/dispatch_toy.json);
  * an independent brute force written from the definitions of the
    walkthrough's 'forward' section: numpy's stable argsort for the
    permutation, the padded offsets as an exclusive prefix sum of each
    group's span (its count plus one, rounded up to a whole number of
    blocks), and the block -> expert table as a sorted search of each block's
    first row among the padded starts (the last expert starting at or before
    it);
  * invariants that hold at any size.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synthetic

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "dispatch_toy.json")


def brute_force_tables(ids, w, E, BM):
    T, K = ids.shape
    flat = ids.reshape(-1)
    P = flat.size
    valid = np.nonzero(flat >= 0)[0]
    order = valid[np.argsort(flat[valid], kind="stable")]
    counts = np.bincount(flat[valid], minlength=E)[:E]
    cum = np.cumsum(counts)
    offsets = cum - counts
    span = -(-(counts.astype(np.int64) + 1) // BM) * BM      # whole blocks, >= 1 per expert
    padded = np.concatenate([[0], np.cumsum(span)[:-1]])
    n_blocks = -(-P // BM) + E
    blk = np.searchsorted(padded, np.arange(n_blocks) * BM, side="right") - 1
    pos = np.full(P, -1, np.int64)
    pos[order] = np.arange(order.size)
    return dict(group_sizes=counts, group_offsets=offsets, group_padded_offsets=padded,
                block_expert=blk, sorted_pair=order, sorted_token=order // K,
                sorted_weight=w.reshape(-1)[order], token_topk_to_pos=pos.reshape(T, K),
                n_valid=order.size)


def _compare(got, ref):
    n = ref["n_valid"]
    assert got["n_valid"] == n
    for k in ("group_sizes", "group_offsets", "group_padded_offsets", "block_expert",
              "token_topk_to_pos"):
        assert np.array_equal(np.asarray(got[k]), np.asarray(ref[k])), k
    for k in ("sorted_pair", "sorted_token"):
        assert np.array_equal(got[k][:n], ref[k]), k
    assert np.array_equal(got["sorted_weight"][:n].view(np.uint32),
                          ref["sorted_weight"].astype(np.float32).view(np.uint32))


def _random_case(T, K, E, mask_frac, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, E, size=(T, K)).astype(np.int32)
    if mask_frac:
        ids[rng.random((T, K)) < mask_frac] = -1
    w = rng.random((T, K)).astype(np.float32)
    return ids, w


def test_golden_offsets_from_cumsum():
    case = json.load(open(GOLDEN))["cases"][0]
    ids = np.repeat(np.arange(len(case["counts"]), dtype=np.int32), case["counts"]).reshape(-1, 1)
    got = oracle.dispatch(ids, None, E=len(case["counts"]), BM=128)
    assert np.cumsum(got["group_sizes"]).tolist() == case["cumsum"]
    assert got["group_offsets"].tolist() == case["group_offsets"]


def test_golden_block_lookup():
    case = json.load(open(GOLDEN))["cases"][1]
    ids = np.repeat(np.arange(len(case["counts"]), dtype=np.int32), case["counts"]).reshape(-1, 1)
    got = oracle.dispatch(ids, None, E=len(case["counts"]), BM=case["block_m"])
    assert got["group_padded_offsets"].tolist() == case["group_padded_offsets"]
    assert got["block_expert"][case["bx"]] == case["expert"]


@pytest.mark.parametrize("BM", [1, 16, 32, 64, 128, 256])
@pytest.mark.parametrize("T,K,E,mask", [(1, 1, 1, 0.0), (5, 2, 3, 0.0), (37, 8, 16, 0.2),
                                         (64, 2, 8, 0.0), (200, 8, 64, 0.05), (33, 4, 5, 1.0)])
def test_dispatch_matches_brute_force(T, K, E, mask, BM):
    ids, w = _random_case(T, K, E, mask, seed=T * 131 + K * 7 + E)
    _compare(oracle.dispatch(ids, w, E, BM), brute_force_tables(ids, w, E, BM))


def test_dispatch_exact_multiple_gets_extra_block():
    # 128 rows for expert 0 at BM = 128: the +1 rule gives it two blocks.
    ids = np.zeros((128, 1), np.int32)
    got = oracle.dispatch(ids, None, E=2, BM=128)
    assert got["group_padded_offsets"].tolist() == [0, 256]
    assert got["block_expert"].tolist() == [0, 0, 1]


def test_dispatch_rejects_out_of_range_ids():
    ids = np.array([[0, 3]], np.int32)
    with pytest.raises(ValueError):
        oracle.dispatch(ids, None, E=3, BM=16)


def check_invariants(ids, tables, E, BM):
    T, K = ids.shape
    sizes = tables["group_sizes"]
    n = tables["n_valid"]
    valid = ids >= 0
    assert sizes.sum() == n == valid.sum()
    st = tables["sorted_token"][:n]
    assert np.array_equal(np.bincount(st, minlength=T), valid.sum(axis=1))
    pos = tables["token_topk_to_pos"]
    assert np.array_equal(np.sort(pos[valid]), np.arange(n))
    assert np.all(pos[~valid] == -1)
    sp = tables["sorted_pair"][:n]
    off = tables["group_offsets"]
    for e in range(E):
        seg = sp[off[e]:off[e] + sizes[e]]
        assert np.all(np.diff(seg) > 0)
        assert np.all(ids.reshape(-1)[seg] == e)
    pad = tables["group_padded_offsets"].astype(np.int64)
    assert np.all(pad % BM == 0)
    gaps = np.diff(np.append(pad, math.ceil(T * K / BM) * BM + E * BM))
    assert np.all(gaps >= sizes + 1)
    blk = tables["block_expert"]
    assert np.all(np.diff(blk) >= 0)
    for e in range(E):
        first = pad[e] // BM
        nblk = -(-(sizes[e] + 1) // BM)
        assert np.all(blk[first:first + nblk] == e)


@pytest.mark.parametrize("ci", [0, 1, 2, 4])
def test_dispatch_invariants_on_workloads(ci):
    cfg = synthetic.CONFIGS[ci]
    d = synthetic.make_moe_inputs(cfg, weights=False)
    ids = d["topk_ids"].numpy()
    w = d["topk_weights"].numpy()
    for BM in (16, 32, 64, 128, 256):
        tables = oracle.dispatch(ids, w, cfg["E"], BM)
        check_invariants(ids, tables, cfg["E"], BM)
        if ci != 4 or BM == 128:
            _compare(tables, brute_force_tables(ids, w, cfg["E"], BM))


def test_dispatch_masked_slots_invariants():
    ids, w = _random_case(300, 8, 32, 0.3, seed=9)
    check_invariants(ids, oracle.dispatch(ids, w, 32, 64), 32, 64)
