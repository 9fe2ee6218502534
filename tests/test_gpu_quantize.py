"""a0 csa2_quantize_fp4 on the GPU against the oracle: bit-exact codes and scales."""

import numpy as np
import pytest
import torch

from gpu_util import DEV, W, csa2, note, np_bits, oracle

pytestmark = pytest.mark.gpu


def _run(x, d_r=0, cap=None, row0=0, rope=None, layout="record"):
    R, d_c = x.shape
    cap = R + row0 if cap is None else cap
    codes, scales, rope_dst = csa2.alloc_cache(1, cap, d_c, d_r, DEV, layout)
    codes, scales, rope_dst = codes[0], scales[0], rope_dst[0]
    codes.fill_(0xAB)
    scales.fill_(0xCD)
    if d_r:
        rope_dst.zero_()
    csa2.csa2_quantize_fp4(x, codes, scales, row0, rope, rope_dst if d_r else None)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy(), (rope_dst.cpu() if d_r else None)


def _bits_tensor(bits_u16):
    return torch.from_numpy(bits_u16.astype(np.uint16).view(np.int16)).view(torch.bfloat16).to(DEV)


def test_every_bf16_amax_gives_the_oracle_scale():
    note("quantize: every positive finite bf16 as a group amax")
    amax = np.arange(0x0001, 0x7F80, dtype=np.uint16)          # 32639 positive finite patterns
    G = amax.size
    rng = np.random.default_rng(0)
    a = oracle.bf16_bits_to_f64(amax)
    frac = rng.uniform(-1, 1, size=(G, 15))
    rest = torch.from_numpy(a[:, None] * frac).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    grp = np.concatenate([amax[:, None], rest], axis=1)
    pad = (-G) % 32
    grp = np.concatenate([grp, np.zeros((pad, 16), dtype=np.uint16)])
    x = grp.reshape(-1, 512)
    codes, scales, _ = _run(_bits_tensor(x))
    wc, ws = oracle.quantize_fp4(x)
    assert np.array_equal(scales, ws)
    assert np.array_equal(codes, wc)


def test_every_bf16_pattern_as_an_element():
    note("quantize: every finite bf16 pattern as an element")
    pats = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    pats = pats[(pats & 0x7F80) != 0x7F80]                     # drop inf / NaN
    rng = np.random.default_rng(1)
    pats = rng.permutation(pats)
    pad = (-pats.size) % 512
    x = np.concatenate([pats, np.zeros(pad, dtype=np.uint16)]).reshape(-1, 512)
    codes, scales, _ = _run(_bits_tensor(x))
    wc, ws = oracle.quantize_fp4(x)
    assert np.array_equal(scales, ws) and np.array_equal(codes, wc)
    # groups drawn from a narrow band so that ties and saturation are frequent
    e = rng.integers(118, 136, size=(2048, 32, 1))
    m = rng.integers(0, 128, size=(2048, 32, 16))
    s = rng.integers(0, 2, size=(2048, 32, 16))
    x = ((s << 15) | ((e + rng.integers(-3, 1, size=(2048, 32, 16))) << 7) | m).astype(np.uint16)
    x = x.reshape(2048, 512)
    codes, scales, _ = _run(_bits_tensor(x))
    wc, ws = oracle.quantize_fp4(x)
    assert np.array_equal(scales, ws) and np.array_equal(codes, wc)


def test_golden_groups_on_gpu():
    note("quantize: hand-derived golden groups")
    import oracle_pins
    recs = oracle_pins._records("quantize_groups.txt")
    rows = [[float(v) for v in recs[i][1:]] for i in range(0, len(recs), 3)]
    x = oracle.f64_to_bf16_bits_exact(np.array(rows)).reshape(1, -1)
    x = np.concatenate([x, np.zeros((1, (-x.shape[1]) % 32), dtype=np.uint16)], axis=1)
    codes, scales, _ = _run(_bits_tensor(x))
    wc, ws = oracle.quantize_fp4(x)
    assert np.array_equal(scales, ws) and np.array_equal(codes, wc)


@pytest.mark.parametrize("layout", ["record", "separate"])
@pytest.mark.parametrize("d_c,d_r,R,row0,cap", [(512, 64, 8192, 262144 - 8192, 262144), (512, 64, 1, 5, 9),
                                                (512, 0, 777, 100, 1000), (128, 0, 1024, 0, 1024),
                                                (32, 8, 33, 1, 40), (2048, 16, 65, 0, 65), (128, 64, 50, 3, 60)])
def test_append_rows_and_leave_the_rest(d_c, d_r, R, row0, cap, layout):
    note(f"quantize: append d_c={d_c} d_r={d_r} R={R} row0={row0} cap={cap} layout={layout}")
    wl = W.WORKLOADS[4].scaled(prefill_rows=R, d_c=d_c, d_r=d_r)
    x = W.prefill_chunk(wl, DEV)
    rope = W.prefill_rope(wl, DEV) if d_r else None
    codes, scales, rope_dst = _run(x, d_r=d_r, cap=cap, row0=row0, rope=rope, layout=layout)
    wc, ws = oracle.quantize_fp4(np_bits(x))
    assert np.array_equal(codes[row0:row0 + R], wc)
    assert np.array_equal(scales[row0:row0 + R], ws)
    assert np.all(codes[:row0] == 0xAB) and np.all(codes[row0 + R:] == 0xAB)
    assert np.all(scales[:row0] == 0xCD) and np.all(scales[row0 + R:] == 0xCD)
    if d_r:
        assert torch.equal(rope_dst[row0:row0 + R], rope.cpu())


def test_zero_rows_is_a_noop():
    note("quantize: zero rows")
    x = torch.zeros(0, 512, dtype=torch.bfloat16, device=DEV)
    codes, scales, _ = _run(x, cap=4, row0=4)
    assert np.all(codes == 0xAB)


def test_workload_latents():
    note("quantize: workload latent rows (all decode workloads)")
    for wl in W.WORKLOADS[:4]:
        x = W.latent_rows(wl, 0, 4096, DEV)
        codes, scales, _ = _run(x)
        wc, ws = oracle.quantize_fp4(np_bits(x))
        assert np.array_equal(codes, wc) and np.array_equal(scales, ws), wl.name
