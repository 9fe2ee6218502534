"""a1 csa2_index_full / a2 csa2_index_pool on the GPU against the oracle.
Integer-valued inputs: scores bit-exact.  Fractional head weights: fp32
rounding only."""

import numpy as np
import pytest
import torch

from gpu_util import DEV, W, csa2, note, np_bits, oracle

pytestmark = pytest.mark.gpu


def _keys(wl, B):
    return torch.stack([W.index_keys(wl, b, DEV) for b in range(B)])


@pytest.mark.parametrize("wi", [0, 1])
def test_full_mode_workload_exact(wi):
    wl = W.WORKLOADS[wi]
    note(f"index_full: {wl.name} B={wl.B} N={wl.N}")
    k = _keys(wl, wl.B)
    q = W.index_query(wl, DEV)
    sc = csa2.csa2_index_full(q, k).cpu().numpy()
    ref = oracle.index_full(np_bits(q), None, np_bits(k), None)
    assert np.array_equal(sc, ref.astype(np.float32))
    assert np.array_equal(sc.astype(np.float64), ref)


@pytest.mark.parametrize("H_I,D_I", [(1, 32), (4, 64), (8, 128), (16, 256), (5, 128), (16, 64)])
def test_full_mode_shapes_ragged_nvalid(H_I, D_I):
    note(f"index_full: H_I={H_I} D_I={D_I} ragged")
    wl = W.WORKLOADS[1].scaled(B=3, N=1000, H_I=H_I, D_I=D_I)
    k = _keys(wl, 3)
    q = W.index_query(wl, DEV)
    nv = torch.tensor([1000, 517, 0], dtype=torch.int32, device=DEV)
    sc = csa2.csa2_index_full(q, k, n_valid=nv).cpu().numpy()
    ref = oracle.index_full(np_bits(q), None, np_bits(k), nv.cpu().numpy())
    assert np.array_equal(sc.astype(np.float64), ref)
    # integer head weights stay exact; n_valid beyond N_cap clamps
    w = torch.randint(0, 4, (3, H_I), device=DEV).float()
    nv2 = torch.tensor([5000, -3, 999], dtype=torch.int32, device=DEV)
    sc = csa2.csa2_index_full(q, k, w=w, n_valid=nv2).cpu().numpy()
    ref = oracle.index_full(np_bits(q), w.cpu().numpy(), np_bits(k), nv2.cpu().numpy())
    assert np.array_equal(sc.astype(np.float64), ref)


def test_full_mode_fractional_weights():
    note("index_full: fractional head weights")
    wl = W.WORKLOADS[1].scaled(B=2, N=4096)
    k = _keys(wl, 2)
    q = W.index_query(wl, DEV)
    w = torch.rand(2, 8, device=DEV) * 2 - 0.5
    sc = csa2.csa2_index_full(q, k, w=w).cpu().numpy().astype(np.float64)
    ref = oracle.index_full(np_bits(q), w.cpu().numpy().astype(np.float64), np_bits(k), None)
    assert np.allclose(sc, ref, rtol=1e-6, atol=1e-3)


def test_full_mode_1m_sampled():
    wl = W.WORKLOADS[4]
    note(f"index_full: {wl.name} B=8 N=262144 (rows 0 and 7 checked whole)")
    k = _keys(wl, wl.B)
    q = W.index_query(wl, DEV)
    sc = csa2.csa2_index_full(q, k)
    torch.cuda.synchronize()
    for b in (0, 7):
        ref = oracle.index_full(np_bits(q[b:b + 1]), None, np_bits(k[b:b + 1]), None)
        assert np.array_equal(sc[b:b + 1].cpu().numpy().astype(np.float64), ref), b


def test_pool_mode_workload_exact():
    wl = W.WORKLOADS[2].scaled(B=4)
    note(f"index_pool: {wl.name} B=4 N=262144 pool 2048x8")
    k = _keys(wl, 4)
    q = W.index_query(wl, DEV)
    blk, nb = W.pool_blocks(wl, DEV)
    sc, pos = csa2.csa2_index_pool(q, k, blk, nb, block=8)
    rs, rp = oracle.index_pool(np_bits(q), None, np_bits(k), None, blk.cpu().numpy(), nb.cpu().numpy(), 8)
    assert np.array_equal(pos.cpu().numpy(), rp)
    assert np.array_equal(sc.cpu().numpy().astype(np.float64), rs)


@pytest.mark.parametrize("D_I,blocks", [(64, (8, 1, 3)), (128, (4, 8, 12)), (32, (16, 5))])
def test_pool_mode_edges(D_I, blocks):
    """Blocks holding whole wave-wide loads (contiguous loads, one lookup per
    load; 12 does not divide a 16-key tile) and blocks that do not (a lookup
    per key), with empty slots, negative ids and ids past n_valid."""
    note(f"index_pool: D_I={D_I} blocks={blocks}: empty slots, negative ids, ids past n_valid")
    wl = W.WORKLOADS[1].scaled(B=3, N=300, H_I=4, D_I=D_I)
    k = _keys(wl, 3)
    q = W.index_query(wl, DEV)
    for block in blocks:
        P_max = 40
        nbk = 300 // block
        rng = np.random.default_rng(block)
        blk = rng.integers(-2, nbk + 5, size=(3, P_max)).astype(np.int32)
        nb = np.array([40, 17, 0], dtype=np.int32)
        nv = np.array([300, 123, 300], dtype=np.int32)
        bt, nbt, nvt = (torch.from_numpy(a).to(DEV) for a in (blk, nb, nv))
        sc, pos = csa2.csa2_index_pool(q, k, bt, nbt, block=block, n_valid=nvt)
        rs, rp = oracle.index_pool(np_bits(q), None, np_bits(k), nv, blk, nb, block)
        assert np.array_equal(pos.cpu().numpy(), rp), block
        assert np.array_equal(sc.cpu().numpy().astype(np.float64), rs), block


@pytest.mark.parametrize("D_I,P_max", [(256, 41), (128, 33), (64, 7), (128, 2048)])
def test_pool_mode_8_position_blocks(D_I, P_max):
    """The pool's 8-position blocks (the streaming pool kernel, eight tiles per
    wave): an odd P_max leaves the last tile half empty, and waves whose tiles
    run past it; empty slots, negative ids and ids past n_valid."""
    N = 8 * 3000
    note(f"index_pool: 8-position blocks D_I={D_I} P_max={P_max}")
    wl = W.WORKLOADS[1].scaled(B=3, N=N, H_I=8, D_I=D_I)
    k = _keys(wl, 3)
    q = W.index_query(wl, DEV)
    rng = np.random.default_rng(P_max + D_I)
    blk = rng.integers(-2, N // 8 + 5, size=(3, P_max)).astype(np.int32)
    nb = np.array([P_max, P_max // 2 + 1, 0], dtype=np.int32)
    nv = np.array([N, 12345, N], dtype=np.int32)
    bt, nbt, nvt = (torch.from_numpy(a).to(DEV) for a in (blk, nb, nv))
    sc, pos = csa2.csa2_index_pool(q, k, bt, nbt, block=8, n_valid=nvt)
    rs, rp = oracle.index_pool(np_bits(q), None, np_bits(k), nv, blk, nb, 8)
    assert np.array_equal(pos.cpu().numpy(), rp)
    assert np.array_equal(sc.cpu().numpy().astype(np.float64), rs)
