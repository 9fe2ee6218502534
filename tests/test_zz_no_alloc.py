"""csa2_topk_noalloc (the Top-K whose scratch is the library's static device
array) against csa2_topk (caller workspace) through the C ABI: two calls in a
row on the same GPU, the second smaller than the first, each bit-exact with
the workspace entry point (ids and scores).  The first call needs three
reduction levels (two of them through the scratch array), the second one
level less, so the second reads scratch that still holds the first call's
winners wherever it does not overwrite them."""

import sys

import numpy as np
import pytest
import torch

from sparse_attention_decode_csa2_amd import csa2

DEV = "cuda"


def _note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _chunk_level_bytes(B, M, K):
    """The chunked reduction's level buffers, as the header states them."""
    total, m = 0, M
    while True:
        ch = -(-m // 16384)
        if ch <= 1:
            return total
        total += B * ch * K * 8
        m = ch * K


def _scores(B, M, seed):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    # integer-valued scores with many ties (the indexer's scores are integers)
    return torch.randint(-2000, 2000, (B, M), generator=g, dtype=torch.int32).to(torch.float32).to(DEV)


@pytest.mark.gpu
def test_noalloc_topk_matches_workspace_topk_on_two_calls():
    cases = [(2, 16384 * 33 + 77, 2048, 11), (3, 40000, 300, 12)]
    for B, M, K, seed in cases:
        need = _chunk_level_bytes(B, M, K)
        _note(f"noalloc topk: B={B} M={M} K={K} scratch bytes={need}")
        assert 0 < need <= 32 << 20
        sc = _scores(B, M, seed)
        ref_i, ref_s = csa2.csa2_topk(sc, K)
        out_i = torch.full((B, K), -7, dtype=torch.int32, device=DEV)
        out_s = torch.full((B, K), 7.0, dtype=torch.float32, device=DEV)
        got_i, got_s = csa2.csa2_topk_noalloc(sc, K, out_idx=out_i, out_score=out_s)
        torch.cuda.synchronize()
        assert got_i.data_ptr() == out_i.data_ptr()
        assert np.array_equal(got_i.cpu().numpy(), ref_i.cpu().numpy())
        assert np.array_equal(got_s.cpu().numpy().view(np.uint32), ref_s.cpu().numpy().view(np.uint32))


@pytest.mark.gpu
def test_noalloc_topk_with_ids_and_valid_counts():
    B, M, K = 4, 16384 * 3 + 5, 512
    _note(f"noalloc topk with ids: B={B} M={M} K={K}")
    sc = _scores(B, M, 13)
    g = torch.Generator(device="cpu")
    g.manual_seed(14)
    ids = torch.randperm(10 * M, generator=g)[: B * M].view(B, M).to(torch.int32)
    ids[:, ::97] = -1
    ids = ids.to(DEV)
    nv = torch.tensor([M, M - 1, 20000, 0], dtype=torch.int32, device=DEV)
    ref_i, ref_s = csa2.csa2_topk(sc, K, ids=ids, n_valid=nv)
    got_i, got_s = csa2.csa2_topk_noalloc(sc, K, ids=ids, n_valid=nv)
    torch.cuda.synchronize()
    assert np.array_equal(got_i.cpu().numpy(), ref_i.cpu().numpy())
    assert np.array_equal(got_s.cpu().numpy().view(np.uint32), ref_s.cpu().numpy().view(np.uint32))
