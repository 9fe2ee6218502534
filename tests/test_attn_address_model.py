"""CPU model of every global address the sparse-attention launches form.

The model restates, in NumPy, the index arithmetic of the launch plan (heads
per workgroup, slices per query, the XCD-ordered grid), of both attention
kernels (16 heads per workgroup; 32 heads with score and value waves) and of
the split combine, and checks each offset against the extent of the buffer it
addresses: the queries, the index lists, the cache rows (codes, scales, RoPE
part; 32-bit row offsets inside one sequence), the outputs, the LSE and the
workspace, and the window rows and row scales of the 32-head kernel's window
variant.  It also checks that every (query, slice, head group) unit is owned
by exactly one workgroup and every output element written exactly once.

The model's slice count is pinned to the library's own plan through
csa2_sparse_attn_workspace_bytes (which is B * H * slices * (d_c + 2) * 4
bytes when a query is split), so the plan the model enumerates is the one the
library launches.  Pure host code: nothing is launched.
"""

import itertools

import numpy as np
import pytest

from sparse_attention_decode_csa2_amd import csa2

TILE, IDS, IDS_PAD = 64, 512, 640


def heads_per_wg(B, H, d_c):
    return 32 if (d_c == 512 and H > 16 and B * ((H + 31) // 32) >= 64) else 16


def plan(B, H, K, d_c):
    hpw = heads_per_wg(B, H, d_c)
    n_hg = -(-H // hpw)
    tiles = -(-K // TILE)
    base = B * n_hg
    s = 1 if base >= 256 else 256 // base
    s = max(s, -(-tiles // (IDS // TILE)))
    s = max(1, min(s, tiles))
    tps = -(-tiles // s)
    s = -(-tiles // tps)
    return hpw, n_hg, s, tps * TILE


def grid_units(B, H, K, d_c):
    """Workgroup -> (active, b, split, head group) for the attention grid."""
    hpw, n_hg, s, ps = plan(B, H, K, d_c)
    spread = B < 8
    groups = (B * s + 7) // 8 if spread else (B + 7) // 8 * s
    bx = np.arange(groups * 8 * n_hg, dtype=np.int64)
    xcd, slot = bx & 7, bx >> 3
    if spread:
        unit = (slot // n_hg) * 8 + xcd
        active = unit < B * s
        b, split = unit // s, unit % s
    else:
        per_q = s * n_hg
        b = (slot // per_q) * 8 + xcd
        active = b < B
        split = (slot % per_q) // n_hg
    hg = slot % n_hg
    return hpw, n_hg, s, ps, active, b[active], split[active], hg[active]


def combine_rows(B, H):
    """Combine block -> output row (b * H + h) for a split query."""
    spread = B < 8
    if spread:
        return np.arange(B * H, dtype=np.int64)
    bx = np.arange((B + 7) // 8 * 8 * H, dtype=np.int64)
    xcd, slot = bx & 7, bx >> 3
    b = (slot // H) * 8 + xcd
    ok = b < B
    return (b * H + slot % H)[ok]


def pv_chunk(dc, w, m):
    return 8 * (w >> 1) + (w & 1) + 2 * m if dc >= 512 else w


def epilogue_channels_16(dc):
    """Channels the 16-head kernel's epilogue writes per (head slot): wave w,
    d-block d, lane column n."""
    ndb = dc // 4 // 16
    return sorted(32 * pv_chunk(dc, w, d >> 1) + 16 * (d & 1) + n
                  for w in range(4) for d in range(ndb) for n in range(16))


def epilogue_heads_16():
    """Head slots (4 g + i) of the 16-head epilogue: lane group g, element i."""
    return sorted(4 * g + i for g in range(4) for i in range(4))


def epilogue_role():
    """(head slot, channel) pairs the value waves of the 32-head kernel write:
    value wave r, lane (hl, kh), accumulator k, element i."""
    out = []
    for r in range(4):
        for lane in range(64):
            hl, kh = lane & 31, lane >> 5
            for i in range(16):
                hh = 8 * (i >> 2) + 4 * kh + (i & 3)
                for k in range(4):
                    out.append((hh, 128 * r + 32 * k + hl))
    return out


def max_gather_tile_16(n_tiles):
    """Largest tile the 16-head kernel's look-ahead gathers read ids for:
    tiles 0 and 1 first, then t + 2 and t + 3 for t = 0, 2, ... while
    t + 2 <= n_tiles."""
    if n_tiles == 0:
        return -1
    m = 1
    t = 0
    while t + 2 <= n_tiles:
        m = max(m, t + 3)
        t += 2
    return m


def check(B, H, K, d_c, d_r, qps=1, N_cap=1000):
    """Every check for one launch configuration; returns the plan."""
    D = d_c + d_r
    hpw, n_hg, s, ps, active, b, split, hg = grid_units(B, H, K, d_c)
    # ---- each (b, split, hg) unit exactly once
    key = (b * s + split) * n_hg + hg
    assert np.array_equal(np.sort(key), np.arange(B * s * n_hg)), "units not covered exactly once"
    assert (b >= 0).all() and (b < B).all()
    e_begin = split * ps
    e_end = np.minimum(K, e_begin + ps)
    assert (e_end > e_begin).all(), "an empty slice"
    assert (e_end - e_begin <= IDS).all(), "a slice holds more ids than the staging array"
    n_tiles = -(-(e_end - e_begin) // TILE)
    # ---- index list reads: idx[b * K + clamp(e)] with e the staged positions
    if hpw == 16:
        e = e_begin[:, None] + np.arange(IDS)[None, :]
    else:
        e = e_begin[:, None] + np.arange(512)[None, :]
    j = np.minimum(e, np.maximum(e_end[:, None] - 1, 0))
    off = b[:, None] * K + j
    assert off.min() >= 0 and off.max() < B * K, "idx read out of bounds"
    assert (j >= e_begin[:, None]).all() and (j < e_end[:, None]).all(), "id read outside the slice"
    # ---- staged-id reads of the gathers
    if hpw == 16:
        mt = max(max_gather_tile_16(int(t)) for t in np.unique(n_tiles))
        assert mt * TILE + 63 < IDS_PAD, "look-ahead gather past the staged ids"
    # (the 32-head kernel clamps its gather tile to IDS_PAD / TILE - 1)
    # ---- query reads: rows b * H + h (h < H) of D bf16 values, 16-byte pieces
    h0 = hg * hpw
    heads = h0[:, None] + np.arange(hpw)[None, :]
    rows = np.where(heads < H, b[:, None] * H + heads, b[:, None] * H)
    assert rows.min() >= 0 and rows.max() < B * H, "query row out of bounds"
    if hpw == 16:
        qoffs = [128 * (t >> 2) + 32 * g + 8 * (t & 3) for t in range(d_c // 32) for g in range(4)]
        qoffs += [d_c + 16 * g + 8 * t for t in range(d_r // 32) for g in range(4)]
    else:
        KSL, KS = d_c // 32, (d_c + d_r) // 32
        qoffs = []
        for sub in range(8):
            for m in range(KS * 4 // 8):
                p = sub + 8 * m
                t, gg = p >> 2, p & 3
                qoffs.append(128 * (t >> 2) + 32 * gg + 8 * (t & 3) if t < KSL else d_c + 16 * gg + 8 * (t - KSL))
    assert min(qoffs) >= 0 and max(qoffs) + 8 <= D, "query piece outside its row"
    # ---- cache rows: sequence b // qps; row id < N_cap (ids are clamped), and
    # the in-row offsets of one lane stay inside the row widths
    seq = b // qps
    assert seq.max() < B // qps, "query reads a sequence past the cache"
    ncw = d_c // 128
    if hpw == 16:
        code_end = max(16 * g + 64 * i + 16 for g in range(4) for i in range(ncw))
        scale_end = max(2 * g + 8 * i + 2 for g in range(4) for i in range(ncw))
        rope_end = max(32 * g + 16 * t + 16 for g in range(4) for t in range(d_r // 32)) if d_r else 0
    else:
        code_end = max(16 * g + 64 * i + 16 for g in range(4) for i in range(4))
        scale_end = max(2 * g + 8 * i + 2 for g in range(4) for i in range(4))
        rope_end = max(32 * g + 16 * t + 16 for g in range(4) for t in range(d_r // 32)) if d_r else 0
    assert code_end <= d_c // 2 and scale_end <= d_c // 16 and rope_end <= 2 * d_r, "gather past the row"
    # 32-bit row offsets: the host refuses N_cap * stride > 2^32, so the last
    # row's last byte stays below 2^32
    for stride, end in ((d_c // 2, code_end), (d_c // 16, scale_end), (2 * d_r, rope_end)):
        if stride:
            ncap_max = (1 << 32) // stride
            assert (ncap_max - 1) * stride + end <= (1 << 32)
    # ---- outputs
    if hpw == 16:
        ch = epilogue_channels_16(d_c)
        assert ch == list(range(d_c)), "16-head epilogue channels not a permutation"
        hs = epilogue_heads_16()
        assert hs == list(range(16))
        written = heads[:, hs][heads[:, hs] < H]
    else:
        pairs = epilogue_role()
        assert len(pairs) == len(set(pairs)) == 32 * 512, "32-head epilogue writes a cell twice"
        written = heads[heads < H]
    if s == 1:
        out_rows = (b[:, None] * H + (heads * (heads < H)))[heads < H]
        assert np.array_equal(np.sort(out_rows), np.arange(B * H)), "an output row written twice or never"
        ws_bytes = 0
    else:
        slot_o = ((b[:, None] * H + heads) * s + split[:, None])[heads < H]
        assert np.array_equal(np.sort(slot_o), np.arange(B * H * s)), "a partial written twice or never"
        assert slot_o.max() * d_c + d_c <= B * H * s * d_c
        assert 2 * slot_o.max() + 2 <= B * H * s * 2
        ws_bytes = B * H * s * (d_c + 2) * 4
        crow = combine_rows(B, H)
        assert np.array_equal(np.sort(crow), np.arange(B * H)), "combine rows not covered exactly once"
        assert (crow * s * d_c + (s - 1) * d_c + 4 * (d_c // 4) <= B * H * s * d_c).all()
        assert (crow * s * 2 + 2 * (s - 1) + 2 <= B * H * s * 2).all()
    assert written.max() < H
    return hpw, n_hg, s, ps, ws_bytes


@pytest.fixture(scope="module")
def lib():
    return csa2.load()


def _pin_plan(lib, B, H, K, d_c, ws_bytes):
    assert lib.csa2_sparse_attn_workspace_bytes(B, H, d_c, K) == ws_bytes, (B, H, K, d_c)


def test_every_batch_at_the_decode_shape(lib):
    """B = 1 .. 256 at 64 heads, K = 512, both latent sizes: the shapes of the
    decode workloads, including 8 <= B < 64 (split slices, one query per
    XCD)."""
    for B in range(1, 257):
        for d_c, d_r in ((512, 64), (128, 0)):
            _, _, _, _, ws = check(B, 64, 512, d_c, d_r)
            _pin_plan(lib, B, 64, 512, d_c, ws)


@pytest.mark.parametrize("d_c,d_r", [(512, 64), (512, 0), (128, 0), (128, 64)])
def test_heads_and_list_lengths(lib, d_c, d_r):
    Bs = list(range(1, 17)) + [31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256]
    Hs = [1, 8, 15, 16, 17, 31, 32, 33, 64, 100, 128]
    Ks = [1, 63, 64, 65, 511, 512, 513, 1000, 2048]
    for B, H, K in itertools.product(Bs, Hs, Ks):
        _, _, _, _, ws = check(B, H, K, d_c, d_r)
        _pin_plan(lib, B, H, K, d_c, ws)


def test_prefill_queries_per_sequence(lib):
    """A prefill chunk: S sequences x T queries, query b reading sequence
    b // T."""
    for S, T in ((1, 8192), (2, 8), (3, 5), (1, 1), (4, 64)):
        for K in (1, 512, 700):
            _, _, _, _, ws = check(S * T, 64, K, 512, 64, qps=T)
            _pin_plan(lib, S * T, 64, K, 512, ws)


def check_window(B, H, K, W_cap, d_r, n_win):
    """The window reads of the 32-head kernel's window variant: only slice 0
    of a query reads them; row scales sigma[b * W_cap + j] for j < nw; tile t,
    wave w, lane (n, g) reads row 64 t + 16 w + n (row 0 when that is past
    nw) at bytes 32 g + 128 i + {0, 16} (16 each, i < 4) of its 512-byte code
    row, and bytes 32 g + 16 t' (t' < d_r / 32) of its RoPE row, and its scale."""
    hpw, n_hg, s, ps, active, b, split, hg = grid_units(B, H, K, 512)
    assert hpw == 32
    code_end = max(32 * g + 128 * i + o + 16 for g in range(4) for i in range(4) for o in (0, 16))
    rope_end = max(32 * g + 16 * t + 16 for g in range(4) for t in range(d_r // 32)) if d_r else 0
    assert code_end <= 512 and rope_end <= 2 * d_r, "window lane reads past its row"
    nw = np.where(split == 0, np.minimum(np.maximum(n_win[b], 0), W_cap), 0)
    assert (nw <= W_cap).all()
    # row scales read by threads tid < nw (512 threads per workgroup)
    assert (nw <= 512).all()
    last_sig = b * W_cap + nw - 1
    assert (last_sig[nw > 0] < B * W_cap).all(), "row scale past the window"
    n_wt = -(-nw // TILE)
    rows = np.arange(4 * TILE).reshape(4, TILE)          # tile t: rows 64 t .. 64 t + 63
    for u in np.nonzero(n_wt > 0)[0]:
        r = rows[:n_wt[u]].ravel()
        rr = b[u] * W_cap + np.where(r < nw[u], r, 0)
        assert rr.min() >= 0 and rr.max() < B * W_cap, "window row out of bounds"
    return n_wt


@pytest.mark.parametrize("d_r", [64, 0])
def test_window_variant_reads(lib, d_r):
    """Every batch the 32-head kernel serves at 64 heads (and a partial head
    group), windows of 0 .. 256 rows and n_win past W_cap or negative; the
    workspace of the one-call entry is pinned to the library's."""
    rng = np.random.default_rng(d_r)
    for B, H in ((32, 64), (33, 64), (63, 64), (128, 64), (129, 64), (256, 64), (200, 40), (300, 128)):
        for K in (1, 512, 1000):
            for W_cap in (1, 64, 65, 128, 256):
                n_win = rng.integers(-3, W_cap + 4, size=B)
                n_win[0] = W_cap
                check_window(B, H, K, W_cap, d_r, n_win)
                _, _, _, _, ws = check(B, H, K, 512, d_r)
                assert lib.csa2_sparse_swa_attn_workspace_bytes(B, H, 512, K) == ws
    # batches the 32-head kernel does not serve: the sparse kernels' workspace,
    # then B x H floats of LSE for the merge
    for B, H in ((1, 64), (8, 64), (31, 64), (200, 16)):
        _, _, _, _, ws = check(B, H, 512, 512, d_r)
        assert lib.csa2_sparse_swa_attn_workspace_bytes(B, H, 512, 512) == -(-ws // 16) * 16 + B * H * 4


# ---------------------------------------------------------------- persistent kernel
STREAM_WG = 256


def streamed(B, H, K, d_c):
    """The persistent 32-head kernel serves unsplit queries of 2..8 tiles
    when the (query, 32-head) units outnumber its 256 workgroups."""
    hpw, n_hg, s, _ = plan(B, H, K, d_c)
    n_units = (B + 7) // 8 * 8 * n_hg
    return hpw == 32 and s == 1 and TILE < K <= IDS and n_units > STREAM_WG, n_hg, n_units


def stream_units(B, n_hp, n_units, G=STREAM_WG):
    """Workgroup x -> its units (b, head group) in order: v = x + k G while
    the query of v is a real one (the padding of the batch to eight comes
    last in every workgroup's sequence; found by the same bisection)."""
    owned = []
    for x in range(G):
        def ub(k):
            v = x + k * G
            return ((v >> 3) // n_hp) * 8 + (v & 7)
        cnt = (n_units - 1 - x) // G + 1 if n_units > x else 0
        lo, hi = 0, cnt
        while lo < hi:
            mid = (lo + hi) // 2
            if ub(mid) < B:
                lo = mid + 1
            else:
                hi = mid
        bs = [ub(k) for k in range(cnt)]
        assert all(b < B for b in bs[:lo]) and all(b >= B for b in bs[lo:]), "padding units not last"
        assert all(bs[k] <= bs[k + 1] for k in range(cnt - 1))
        units = []
        for k in range(lo):
            v = x + k * G
            assert v & 7 == x & 7, "a unit left its XCD"
            units.append((ub(k), (v >> 3) % n_hp))
        owned.append(units)
    return owned


def stream_protocol(n_my, T):
    """Replays the barrier intervals of one persistent workgroup with n_my
    units of T tiles, both roles, and checks every LDS access of the value
    buffers (tiles, score rows, the converted query), the head scales and the
    double-buffered ids against what it must find: a read sees the last write
    of an earlier interval with the expected contents, and no interval has a
    write that another role (or the other half of a role) also touches."""
    X = lambda k: 0 if T & 1 else k & 1
    ev = {}            # interval -> list of (role, op, resource, tag)

    def put(i, role, op, res, tag):
        ev.setdefault(i, []).append((role, op, res, tag))

    # every thread stages unit 0's ids before the first barrier
    put(0, "all", "w", "idx0", ("ids", 0))
    # score waves
    i = 1
    for kk in range(min(2, T)):
        put(i, "S", "r", "idx0", ("ids", 0))
    for s in range(n_my * T):
        k, j = divmod(s, T)
        if j == 0:
            i += 1
            put(i, "S", "r", f"v{X(k) ^ 1}", ("query", k))
            put(i, "S", "r", "fs", ("query", k))
        put(i, "S", "w", f"v{X(k) ^ (j & 1)}", ("tile", k, j))
        nk, nj = (k, j + 2) if j + 2 < T else (k + 1, j + 2 - T)
        if nk < n_my:
            put(i, "S", "r", f"idx{nk & 1}", ("ids", nk))
        i += 1
    s_barriers = i
    # value waves
    i = 1
    for k in range(n_my):
        if k > 0:
            put(i, "V", "r", f"v{X(k)}", ("tile", k - 1, T - 1))
        put(i, "V", "w", f"v{X(k) ^ 1}", ("query", k))
        put(i, "V", "w", "fs", ("query", k))
        if k + 1 < n_my:
            put(i, "V", "w", f"idx{(k + 1) & 1}", ("ids", k + 1))
        i += 1
        for jt in range(T):
            if jt > 0:
                put(i, "V", "r", f"v{X(k) ^ ((jt - 1) & 1)}", ("tile", k, jt - 1))
            i += 1
    assert i == s_barriers, "the two roles pass different numbers of barriers"
    put(i, "V", "r", f"v{X(n_my)}", ("tile", n_my - 1, T - 1))
    state = {}
    for it in sorted(ev):
        acc = ev[it]
        for role, op, res, tag in acc:
            if op == "r":
                assert state.get(res) == tag, (n_my, T, it, role, res, tag, state.get(res))
        for role, op, res, tag in acc:
            if op == "w":
                others = [a for a in acc if a[2] == res and a[0] != role]
                assert not others, ("race", n_my, T, it, res, acc)
        for role, op, res, tag in acc:
            if op == "w":
                state[res] = tag


def test_stream_kernel_units_and_lds_protocol(lib):
    """The persistent 32-head kernel: every (query, head group) unit owned by
    exactly one workgroup, on the XCD of the one-unit-per-workgroup grid;
    the LDS hand-over between units for every unit count and tile count it
    can meet; and its reads are those of the 32-head kernel (checked above
    through `check`) for the shapes it serves."""
    for n_my in range(1, 9):
        for T in range(2, 9):
            stream_protocol(n_my, T)
    stream_protocol(64, 8)
    stream_protocol(33, 3)
    cases = [(8192, 64, 512), (8192, 64, 100), (257, 64, 512), (300, 40, 512), (129, 64, 128),
             (2048, 128, 512), (1000, 100, 65), (4096, 64, 700), (128, 64, 512), (64, 64, 512)]
    n_streamed = 0
    for B, H, K in cases:
        ok, n_hp, n_units = streamed(B, H, K, 512)
        _, _, _, _, ws = check(B, H, K, 512, 64, qps=B if B > 256 else 1)
        _pin_plan(lib, B, H, K, 512, ws)
        if not ok:
            continue
        n_streamed += 1
        owned = stream_units(B, n_hp, n_units)
        flat = [u for us in owned for u in us]
        assert len(flat) == len(set(flat)) == B * n_hp, (B, H, K)
        assert all(0 <= b < B and 0 <= hg < n_hp for b, hg in flat)
    assert n_streamed >= 6
