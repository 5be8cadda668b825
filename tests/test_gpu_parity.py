"""GPU parity: every C-ABI call against the CPU oracle on the same seeded inputs.

Bars: selected index sets and nsel bit-exact; indexer scores bit-exact (fixed fp32
order); attention outputs within rel = max|g-r|/max|r| <= 2e-3 for fp32 inputs and 1e-2
for bf16 inputs; RoPE within a few fp32 ulps (fp32) or one bf16 ulp (bf16), untouched dims
bit-exact.  Pages: chen3feng, "colibri-analysis 06: MLA attention and KV cache" (sec. 2.1,
2.2, 2.3); aiknowledge.cn, "Ch.7 sec. 03 ... faithful DSA" (sec. 2).
"""
import math

import numpy as np
import pytest

import oracle
from mla_latent_kv_dsa_amd import synth
from tests.helpers import dev, dev_bf16, host, log, rel_err

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import mla_latent_kv_dsa_amd as mla  # noqa: E402

TOL_F32, TOL_BF16 = 2e-3, 1e-2


def _kv(lc, rc, ic=None, seq_len=None, max_seq_len=0, block_table=None, block_size=0, seq_stride=0, bf16=True,
        tiled=False):
    """tiled: hand the indexer pool over in the 64-row tiled layout (same rows)."""
    to = dev_bf16 if bf16 else dev
    if ic is not None and tiled:
        ic = synth.tile_index_keys(ic)
    return mla.KvCache(to(lc), to(rc), dev(ic) if ic is not None else None,
                       seq_len=dev(np.asarray(seq_len, np.int32)) if seq_len is not None else None,
                       max_seq_len=max_seq_len,
                       block_table=dev(block_table) if block_table is not None else None,
                       block_size=block_size, seq_stride=seq_stride,
                       ic_layout=mla.MLA_IC_TILE64 if tiled else mla.MLA_IC_ROWS)


# ------------------------------------------------------------------------------ RoPE
@pytest.mark.parametrize("bf16", [False, True])
def test_rope_query_tails_and_shared_key(bf16):
    rng = np.random.default_rng(100)
    n, H, nope, rope = 37, 64, 192, 64
    x = rng.standard_normal((n, H, nope + rope)).astype(np.float32)
    pos = rng.integers(0, 131072, n).astype(np.int32)
    pos[0] = 0
    pos[1] = 131071
    xin = synth.bf16_bits_to_f32(synth.to_bf16_bits(x)) if bf16 else x
    log(f"rope q tails bf16={bf16} n={n}")
    t = dev_bf16(synth.to_bf16_bits(x)) if bf16 else dev(x)
    mla.mla_rope_interleave(t, dev(pos), nope, rope)
    got = host(t)
    ref = oracle.rope_interleave(xin, pos, nope, rope)
    assert np.array_equal(got[..., :nope], xin[..., :nope])
    err = np.abs(got - ref)
    if bf16:
        assert np.all(err <= 2.0 ** -8 * np.abs(ref) + 2e-6 * np.abs(xin).max())
    else:
        assert err.max() <= 2e-6 * np.abs(xin).max()
    # the shared key Rc: one head, offset 0, rows of a cache
    rc = rng.standard_normal((300, 1, rope)).astype(np.float32)
    pr = np.arange(300, dtype=np.int32) * 400
    rin = synth.bf16_bits_to_f32(synth.to_bf16_bits(rc)) if bf16 else rc
    t = dev_bf16(synth.to_bf16_bits(rc)) if bf16 else dev(rc)
    mla.mla_rope_interleave(t, dev(pr), 0, rope)
    ref = oracle.rope_interleave(rin, pr, 0, rope)
    err = np.abs(host(t) - ref)
    if bf16:
        assert np.all(err <= 2.0 ** -8 * np.abs(ref) + 2e-6 * np.abs(rin).max())
    else:
        assert err.max() <= 2e-6 * np.abs(rin).max()


def test_rope_strided_view_and_odd_geometry():
    rng = np.random.default_rng(101)
    x = rng.standard_normal((9, 3, 40)).astype(np.float32)
    pos = rng.integers(0, 5000, 9).astype(np.int32)
    full = dev(x)
    view = full[:, :, :]                     # strides (120, 40, 1)
    mla.mla_rope_interleave(view, dev(pos), 10, 22)
    ref = oracle.rope_interleave(x, pos, 10, 22)
    got = host(full)
    assert np.array_equal(got[..., :10], x[..., :10]) and np.array_equal(got[..., 32:], x[..., 32:])
    assert np.abs(got - ref).max() <= 2e-6 * np.abs(x).max()


# ------------------------------------------------------------------------------ indexer
def _index_case(B, seq_len, t_max, n_ih, hd, paged, seed, bs=64, hole=False, tiled=False):
    """Random indexer problem.  Returns q, w, the view, and per sequence the logical key rows
    plus a mask of keys that have a row (a block-table hole leaves a gap of -1 entries)."""
    rng = np.random.default_rng(seed)
    if paged:
        nb = [(s + bs - 1) // bs for s in seq_len]
        perm = rng.permutation(sum(nb)).astype(np.int32)
        max_blocks = (t_max + bs - 1) // bs
        bt = np.full((B, max_blocks), -1, np.int32)
        o = 0
        for b in range(B):
            bt[b, : nb[b]] = perm[o: o + nb[b]]
            o += nb[b]
        if hole and nb[0] > 2:
            bt[0, nb[0] // 2] = -1
        rows = sum(nb) * bs
        ic = rng.standard_normal((rows, hd)).astype(np.float32)
        logical, masks = [], []
        for b in range(B):
            t = np.arange(seq_len[b])
            blk = bt[b, t // bs].astype(np.int64)
            m = blk >= 0
            r = np.where(m, blk * bs + t % bs, 0)
            logical.append(ic[r])
            masks.append(m)
        kvd = dict(block_table=bt, block_size=bs)
    else:
        stride = (t_max + 63) // 64 * 64 if tiled else t_max
        ic = rng.standard_normal((B * stride, hd)).astype(np.float32)
        logical = [ic[b * stride: b * stride + seq_len[b]] for b in range(B)]
        masks = [np.ones(seq_len[b], bool) for b in range(B)]
        kvd = dict(seq_stride=stride)
    q = rng.standard_normal((B, n_ih, hd)).astype(np.float32)
    w = rng.standard_normal((B, n_ih)).astype(np.float32)
    lc = np.zeros((ic.shape[0], 8), np.uint16)
    rc = np.zeros((ic.shape[0], 8), np.uint16)
    kv = _kv(lc, rc, ic, seq_len, t_max, tiled=tiled, **kvd)
    return q, w, kv, logical, masks


def _index_check(q, w, kv, logical, masks, seq_len, t_max):
    s = host(mla.dsa_index_scores(dev(q), dev(w), kv, t_max))
    for b in range(len(seq_len)):
        ref = oracle.index_scores(q[b], w[b], logical[b])
        ref = np.where(masks[b], ref, np.float32(-np.inf)).astype(np.float32)
        assert np.array_equal(s[b, : seq_len[b]].view(np.uint32), ref.view(np.uint32)), b
        assert np.all(np.isneginf(s[b, seq_len[b]:]))


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("n_ih,hd", [(32, 128), (5, 64), (1, 4)])
def test_index_scores_bit_exact(paged, n_ih, hd):
    B, t_max = 3, 1100
    seq_len = [1100, 777, 1]
    log(f"index paged={paged} n_ih={n_ih} hd={hd}")
    q, w, kv, logical, masks = _index_case(B, seq_len, t_max, n_ih, hd, paged, 200 + n_ih + paged)
    _index_check(q, w, kv, logical, masks, seq_len, t_max)


@pytest.mark.parametrize("paged,bs,hole", [(False, 0, False), (True, 64, True), (True, 128, False)])
@pytest.mark.parametrize("n_ih,hd", [(32, 128), (7, 128), (5, 64)])
def test_index_scores_tiled_layout(paged, bs, hole, n_ih, hd):
    """The 64-row tiled indexer pool gives the same bits as rows (matrix-core, lane-per-key and
    generic kernels; contiguous and paged with a hole)."""
    B, t_max = 3, 1100
    seq_len = [1100, 777, 1]
    log(f"index tiled paged={paged} bs={bs} n_ih={n_ih} hd={hd}")
    q, w, kv, logical, masks = _index_case(B, seq_len, t_max, n_ih, hd, paged, 230 + n_ih + bs, bs=bs or 64,
                                           hole=hole, tiled=True)
    _index_check(q, w, kv, logical, masks, seq_len, t_max)


@pytest.mark.parametrize("bs,hole", [(16, False), (16, True), (128, True), (64, True), (1, False)])
def test_index_scores_block_sizes(bs, hole):
    """Every addressing mode of the matrix-core indexer: block sizes that keep a 64-key tile
    in one block (one table entry per tile) and ones that do not (one per key), with a -1
    hole inside a sequence, a ragged tail and several tiles per wave."""
    B, t_max = 2, 70000
    seq_len = [70000, 4097]
    log(f"index bs={bs} hole={hole}")
    q, w, kv, logical, masks = _index_case(B, seq_len, t_max, 32, 128, True, 260 + bs, bs=bs, hole=hole)
    _index_check(q, w, kv, logical, masks, seq_len, t_max)


def test_index_scores_full_context_131072():
    d = synth.decode(3, 131072, dsa=True, bf16=True)
    log("index full T=131072")
    kv = _kv(d.lc, d.rc, d.ic, [d.T], d.T, seq_stride=d.T)
    s = host(mla.dsa_index_scores(dev(d.q_idx), dev(d.w_idx), kv, d.T))[0]
    ref = oracle.index_scores(d.q_idx[0], d.w_idx[0], d.ic)
    assert np.array_equal(s.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("tiled", [False, True])
def test_index_scores_subnormal_products_bit_exact(tiled):
    """Products and partial sums in the subnormal range and near FLT_MIN, with mixed magnitudes and
    signs: heads scaled by 2^-70 .. 1 and key rows by 2^-70 .. 1, so per-head dot products land
    anywhere from 2^-140 (subnormal) to O(1).  The scores must equal the fixed-order fmaf oracle bit
    for bit (a flush of subnormal products or sums to zero would change them), and so must the
    selection that ranks them."""
    rng = np.random.default_rng(240 + tiled)
    T, n_ih, hd, k = 9000, 32, 128, 8000     # k so large that the threshold sits among subnormal scores
    q = rng.standard_normal((1, n_ih, hd)).astype(np.float32)
    q *= np.float32(2.0) ** rng.choice([-70, -64, -40, -3, 0], n_ih).astype(np.float32)[None, :, None]
    ic = rng.standard_normal((T, hd)).astype(np.float32)
    ic *= np.float32(2.0) ** rng.choice([-70, -56, -20, 0, -126, -130, -134], T).astype(np.float32)[:, None]
    ic[::7, ::3] = np.float32(2.0 ** -126) * rng.choice([-1, 1], ic[::7, ::3].shape).astype(np.float32)
    w = (rng.standard_normal((1, n_ih)) * np.float32(2.0) ** rng.choice([-6, 0], (1, n_ih))).astype(np.float32)
    ref = oracle.index_scores(q[0], w[0], ic)
    tiny = np.finfo(np.float32).tiny
    assert ((ref != 0) & (np.abs(ref) < tiny)).sum() > 1000, "the case must produce subnormal scores"
    assert ((ic != 0) & (np.abs(ic) < tiny)).sum() > 1000, "and subnormal key inputs"
    log(f"index subnormal tiled={tiled}")
    Tp = (T + 63) // 64 * 64             # the tiled pool holds whole 64-row tiles
    icp = np.zeros((Tp, hd), np.float32)
    icp[:T] = ic
    zero = np.zeros((Tp, 8), np.uint16)
    kv = _kv(zero, zero, icp, [T], T, seq_stride=Tp, tiled=tiled)
    s = host(mla.dsa_index_scores(dev(q), dev(w), kv, T))[0]
    assert np.array_equal(s.view(np.uint32), ref.view(np.uint32))
    sel, nsel = _select_check(q, w, kv, T, k, [T])
    rs, rn = oracle.topk(ref, T, k)
    assert int(nsel[0]) == rn and np.array_equal(sel[0], rs)


def test_index_empty_and_zero_length():
    q, w, kv, logical, _ = _index_case(2, [0, 5], 64, 32, 128, False, 250)
    s = host(mla.dsa_index_scores(dev(q), dev(w), kv, 64))
    assert np.all(np.isneginf(s[0])) and np.all(np.isneginf(s[1, 5:]))
    assert np.array_equal(s[1, :5], oracle.index_scores(q[1], w[1], logical[1]))


# ------------------------------------------------------------------------------ fused index + select
def _select_check(q, w, kv, t_max, k, seq_len, logical=None, masks=None):
    """dsa_index_select == dsa_index_scores + dsa_topk_select (bit for bit), and the oracle."""
    qd, wd = dev(q), dev(w)
    sc, sel, nsel = mla.dsa_index_select(qd, wd, kv, t_max, k)
    ref_sc = mla.dsa_index_scores(qd, wd, kv, t_max)
    n_valid = dev(np.minimum(np.asarray(seq_len, np.int32), t_max))
    ref_sel, ref_nsel = mla.dsa_topk_select(ref_sc, n_valid, k)
    assert np.array_equal(host(sc).view(np.uint32), host(ref_sc).view(np.uint32))
    assert np.array_equal(host(nsel), host(ref_nsel))
    assert np.array_equal(host(sel), host(ref_sel))
    rs, rn = oracle.topk_batch(host(ref_sc), np.minimum(np.asarray(seq_len, np.int32), t_max), k)
    assert np.array_equal(host(sel), rs) and np.array_equal(host(nsel), rn)
    return host(sel), host(nsel)


@pytest.mark.parametrize("tiled", [False, True])
def test_index_select_full_context_131072(tiled):
    d = synth.decode(3, 131072, dsa=True, bf16=True)
    log(f"index+select T=131072 k=2048 tiled={tiled}")
    kv = _kv(d.lc, d.rc, d.ic, [d.T], d.T, seq_stride=d.T, tiled=tiled)
    _select_check(d.q_idx, d.w_idx, kv, d.T, 2048, [d.T])


@pytest.mark.parametrize("paged,bs", [(False, 0), (True, 64), (True, 16)])
def test_index_select_batched_rows(paged, bs):
    """Rows longer and shorter than k, an empty row, a ragged tail, block-table holes."""
    B, t_max, k = 5, 9000, 777
    seq_len = [9000, 8191, 700, 0, 777]
    log(f"index+select batched paged={paged} bs={bs}")
    q, w, kv, logical, masks = _index_case(B, seq_len, t_max, 32, 128, paged, 270 + bs, bs=bs or 64, hole=paged)
    _select_check(q, w, kv, t_max, k, seq_len)


def test_index_select_generic_indexer_shape():
    B, t_max, k = 2, 5000, 300
    seq_len = [5000, 4321]
    log("index+select n_ih=5 hd=64")
    q, w, kv, logical, masks = _index_case(B, seq_len, t_max, 5, 64, False, 280)
    _select_check(q, w, kv, t_max, k, seq_len)


def test_index_select_ties_and_all_equal():
    """Duplicated key rows tie exactly (lower position wins); all-zero keys tie everywhere
    (the candidate list overflows the LDS-resident path)."""
    rng = np.random.default_rng(290)
    T, k = 20000, 2048
    base = rng.standard_normal((T // 8, 128)).astype(np.float32)
    ic = np.repeat(base, 8, axis=0)
    q = rng.standard_normal((1, 32, 128)).astype(np.float32)
    w = rng.standard_normal((1, 32)).astype(np.float32)
    z = np.zeros((T, 8), np.uint16)
    log("index+select ties")
    kv = _kv(z, z, ic, [T], T, seq_stride=T)
    _select_check(q, w, kv, T, k, [T])
    kv0 = _kv(z, z, np.zeros_like(ic), [T], T, seq_stride=T)
    sel, nsel = _select_check(q, w, kv0, T, k, [T])
    assert np.array_equal(sel[0], np.arange(k))


def _ixm_parts(B, T, tiled):
    """Workgroups per row of the matrix-core indexer and the keys each one scores (the kernel's
    grid: tiles of 64 keys, 4 waves per workgroup, wave (p, w) takes tiles 4 p + w + 4 bx j)."""
    ntiles = (T + 63) // 64
    if tiled:
        bx = min(256, (ntiles + 7) // 8)
    else:
        bx = min(max(768 // B, 1), (ntiles + 3) // 4)
    bx = max(bx, 1)
    parts = []
    for p in range(bx):
        tiles = [t for w in range(4) for t in range(4 * p + w, ntiles, 4 * bx)]
        parts.append(np.concatenate([np.arange(64 * t, min(64 * t + 64, T)) for t in tiles]))
    return parts


@pytest.mark.parametrize("tiled", [False, True])
def test_index_select_deep_histogram_parts(tiled):
    """Scores spread over ~480 quarter-octave bins (about one key per bin) with k = T / 8: every
    indexer workgroup has more than 16 nonzero bins above the threshold, so the filter's first
    read of the lists stops above the threshold bin and it must add the rest of the lists
    (checked here on the CPU first)."""
    rng = np.random.default_rng(292)
    B, T, k = 2, 32768, 4096
    seq = [T, 20001]
    ic = rng.standard_normal((B * T, 128)).astype(np.float32)
    ic[:, 0] = np.exp2(rng.uniform(0.0, 120.0, B * T)).astype(np.float32)
    q = rng.standard_normal((B, 32, 128)).astype(np.float32)
    q[:, 0, :] = 0.0
    q[:, 0, 0] = 1.0                       # head 0 scores max(Ic[t, 0], 0) exactly
    w = np.zeros((B, 32), np.float32)
    w[:, 0] = 1.0
    score0 = np.maximum(ic[:T, 0], 0.0)
    key = score0.view(np.uint32) | np.uint32(0x80000000)   # positive scores: order key
    bins = (key >> 21).astype(np.int64)
    tb = np.sort(bins)[::-1][k - 1]
    floor = max(np.unique(bins[pk])[::-1][15] for pk in _ixm_parts(B, T, tiled) if np.unique(bins[pk]).size > 16)
    assert floor > tb, (floor, tb)
    z = np.zeros((B * T, 8), np.uint16)
    log(f"index+select deep histogram lists tiled={tiled}")
    kv = _kv(z, z, ic, seq, T, seq_stride=T, tiled=tiled)
    _select_check(q, w, kv, T, k, seq)


def test_index_select_ties_across_filter_workgroups():
    """T = 131072, k = 2048, scores spread over 64 octaves, with the k-th score given to 61 keys
    spread over the row (one per filter workgroup): the first 29 of them in position order are
    kept."""
    rng = np.random.default_rng(340)
    T, k = 131072, 2048
    vals = np.exp2(np.arange(T) * (64.0 / T) - 20.0).astype(np.float32)
    vals = vals[rng.permutation(T)]
    order = np.argsort(-vals, kind="stable")
    v = vals[order[2019]]                                  # 2019 keys above it
    low = np.nonzero(vals < v)[0]
    spread = low[np.linspace(0, low.size - 1, 60).astype(np.int64)]
    vals[spread] = v                                       # 61 keys equal to the k-th
    ic = rng.standard_normal((T, 128)).astype(np.float32)
    ic[:, 0] = vals
    q = np.zeros((1, 32, 128), np.float32)
    q[0, 0, 0] = 1.0                                       # head 0 scores Ic[t, 0] exactly
    w = np.zeros((1, 32), np.float32)
    w[0, 0] = 1.0
    z = np.zeros((T, 8), np.uint16)
    log("index+select ties across filter workgroups")
    kv = _kv(z, z, ic, [T], T, seq_stride=T, tiled=True)
    sel, nsel = _select_check(q, w, kv, T, k, [T])
    eq = np.sort(np.nonzero(vals == v)[0])
    assert np.isin(eq[:29], sel[0]).all() and not np.isin(eq[29:], sel[0]).any()


def _cand_case(seed, B, T, window=None, repeat=1, equal=False):
    """Tiled indexer pool at full context (256 indexer workgroups per row).
    window: (start, length, factor) scales a block of key rows so the top keys crowd into a few
    parts; repeat: every row repeated so that equal scores come in groups; equal: all rows equal."""
    rng = np.random.default_rng(seed)
    ic = rng.standard_normal((B * T // repeat, 128)).astype(np.float32)
    if repeat > 1:
        ic = np.repeat(ic, repeat, axis=0)
    if equal:
        ic[:] = ic[0]
    if window is not None:
        s0, ln, f = window
        for b in range(B):
            ic[b * T + s0: b * T + s0 + ln] *= np.float32(f)
    q = rng.standard_normal((B, 32, 128)).astype(np.float32)
    w = rng.standard_normal((B, 32)).astype(np.float32)
    return q, w, ic


@pytest.mark.parametrize("case", ["random", "window", "wide_window", "repeats", "all_equal"])
def test_index_select_score_patterns(case):
    """The selection behind the tiled matrix-core indexer at T = 131072 (k = 2048) on score patterns
    that load its passes differently: random scores, the top keys crowded into a 4096- or 12288-key
    window (a few indexer workgroups hold them all), every score repeated 16 times (equal keys at
    the threshold) and all scores equal.  Bit-exact against the stand-alone top-k and the oracle's
    sort."""
    B, T, k = 1, 131072, 2048
    kw = {"random": {}, "window": dict(window=(40000, 4096, 3.0)), "wide_window": dict(window=(70000, 12288, 2.0)),
          "repeats": dict(repeat=16), "all_equal": dict(equal=True)}[case]
    q, w, ic = _cand_case(300 + len(case), B, T, **kw)
    z = np.zeros((B * T, 8), np.uint16)
    log(f"index+select score pattern: {case}")
    kv = _kv(z, z, ic, [T], T, seq_stride=T, tiled=True)
    sel, nsel = _select_check(q, w, kv, T, k, [T])
    if case == "all_equal":
        assert np.array_equal(sel[0], np.arange(k))


def test_index_select_batched_full_context_window():
    """Three rows of different lengths at full context (workgroups past a row's end write empty
    lists; a row just over k and one under it), the top keys crowded into a window."""
    B, T, k = 3, 131072, 2048
    q, w, ic = _cand_case(330, B, T, window=(100000, 2048, 2.5))
    seq = [T, 2100, 1500]
    z = np.zeros((B * T, 8), np.uint16)
    log("index+select batched full context")
    kv = _kv(z, z, ic, seq, T, seq_stride=T, tiled=True)
    _select_check(q, w, kv, T, k, seq)


def test_index_select_row_past_131072_keys():
    """A row of 200,000 keys (past 131072, so the resolve holds eight bitmask words per thread)
    and a second, shorter row in the same call: scores and selection bit-exact against the oracle."""
    T, k = 200000, 2048
    rng = np.random.default_rng(77)
    ic = rng.standard_normal((2 * T, 128), dtype=np.float32)
    qi = rng.standard_normal((2, 32, 128), dtype=np.float32)
    wi = rng.standard_normal((2, 32), dtype=np.float32)
    seq_len = [T, 150001]
    log("index+select T=200000 k=2048 (eight words per resolve thread)")
    lc = torch.empty((2 * T, 512), dtype=torch.bfloat16, device="cuda")   # not read by the selection
    rc = torch.empty((2 * T, 64), dtype=torch.bfloat16, device="cuda")
    kv = mla.KvCache(lc, rc, dev(ic), seq_len=dev(np.asarray(seq_len, np.int32)), max_seq_len=T, seq_stride=T)
    sc, sel, nsel = mla.dsa_index_select(dev(qi), dev(wi), kv, T, k)
    sc, sel, nsel = host(sc), host(sel), host(nsel)
    for b in range(2):
        n = seq_len[b]
        ref_s = oracle.index_scores(qi[b], wi[b], ic[b * T:b * T + n])
        assert np.array_equal(sc[b, :n].view(np.uint32), ref_s.view(np.uint32)), b
        assert np.all(np.isneginf(sc[b, n:])), b
        ref_sel, ref_n = oracle.topk(ref_s, n, k)
        assert int(nsel[b]) == ref_n == k and np.array_equal(sel[b], ref_sel), b


def test_index_select_long_row_general_path():
    T, k = 300000, 2048
    rng = np.random.default_rng(291)
    ic = rng.standard_normal((T, 128)).astype(np.float32)
    q = rng.standard_normal((1, 32, 128)).astype(np.float32)
    w = rng.standard_normal((1, 32)).astype(np.float32)
    z = np.zeros((T, 8), np.uint16)
    log("index+select T=300000 (general top-k)")
    kv = _kv(z, z, ic, [T - 5], T, seq_stride=T)
    _select_check(q, w, kv, T, k, [T - 5])


# ------------------------------------------------------------------------------ top-k
def _topk_check(scores, n_valid, k):
    sel, nsel = mla.dsa_topk_select(dev(scores), dev(np.asarray(n_valid, np.int32)), k)
    rs, rn = oracle.topk_batch(scores, np.asarray(n_valid, np.int32), k)
    assert np.array_equal(host(nsel), rn)
    assert np.array_equal(host(sel), rs)


@pytest.mark.parametrize("seed", [300, 301])
def test_topk_bit_exact_with_ties(seed):
    rng = np.random.default_rng(seed)
    B, T = 5, 9000
    s = (np.round(rng.standard_normal((B, T)) * 4) / 4).astype(np.float32)   # heavy ties
    s[0, ::7] = -0.0
    s[1, ::5] = 0.0
    s[2] = 1.5                                                                # all equal
    n_valid = [9000, 8191, 4000, 2048, 0]
    log(f"topk ties seed={seed}")
    for k in (1, 7, 2048, 3000):
        _topk_check(s, n_valid, k)


def test_topk_random_full_context():
    rng = np.random.default_rng(302)
    T = 131072
    s = rng.standard_normal((2, T)).astype(np.float32)
    log("topk T=131072")
    _topk_check(s, [T, 100001], 2048)


def test_topk_special_values():
    s = np.array([[np.inf, -np.inf, 3.0, -0.0, 0.0, 1e-38, -1e-38, 3.0, 2.0, -5.0]], np.float32)
    for k in range(1, 11):
        _topk_check(s, [10], k)


# ------------------------------------------------------------------------------ decode
def _decode_ref(d, b, keys, sm, absorbed=True):
    f = oracle.absorbed_decode if absorbed else oracle.nonabsorbed_decode
    cv = synth.bf16_bits_to_f32 if d.bf16 else (lambda a: a)
    lc = cv(d.lc[b * d.T:(b + 1) * d.T])
    rc = cv(d.rc[b * d.T:(b + 1) * d.T])
    return f(cv(d.q_nope[b]), cv(d.q_rope[b]), cv(d.kv_b), lc, rc, keys, d.v, sm)


def _run_decode(d, seq_len, sel=None, nsel=None, paged=None):
    to = dev_bf16 if d.bf16 else dev
    kv = _kv(d.lc, d.rc, None, seq_len, d.T, seq_stride=d.T, bf16=d.bf16)
    sm = 1.0 / math.sqrt(d.nope + d.rope)
    out = mla.mla_absorbed_decode(to(d.q_nope), to(d.q_rope), to(d.kv_b), kv, sm,
                                  sel=dev(sel) if sel is not None else None,
                                  nsel=dev(nsel) if nsel is not None else None)
    return host(out), sm


def test_decode_tiny_fp32_layer_absorbed_equals_nonabsorbed():
    t = synth.tiny_layer(1)
    lc, rc, q = oracle.tiny_layer(t.x, t.q_a, t.q_b, t.kv_a, t.H, t.nope, t.rope, t.L)
    lc32, rc32, q32 = lc.astype(np.float32), rc.astype(np.float32), q.astype(np.float32)
    sm = 1.0 / math.sqrt(t.nope + t.rope)
    log("decode tiny fp32")
    kv = mla.KvCache(dev(lc32), dev(rc32), seq_len=dev(np.array([t.T], np.int32)), max_seq_len=t.T, seq_stride=t.T)
    out = host(mla.mla_absorbed_decode(dev(q32[None, :, : t.nope].copy()), dev(q32[None, :, t.nope:].copy()),
                                       dev(t.kv_b), kv, sm))[0]
    keys = np.arange(t.T)
    ref_a = oracle.absorbed_decode(q32[:, : t.nope], q32[:, t.nope:], t.kv_b, lc32, rc32, keys, t.v, sm)
    ref_n = oracle.nonabsorbed_decode(q32[:, : t.nope], q32[:, t.nope:], t.kv_b, lc32, rc32, keys, t.v, sm)
    assert rel_err(out, ref_a) <= TOL_F32
    assert rel_err(out, ref_n) <= TOL_F32
    # the layer output after o_proj, from the GPU attention and from the oracle
    assert rel_err(oracle.o_proj(t.o_w, out), oracle.o_proj(t.o_w, ref_a)) <= TOL_F32


@pytest.mark.parametrize("T,B", [(300, 1), (1000, 2)])
def test_decode_dense_glm_bf16(T, B):
    d = synth.decode(2 + T, T, B=B)
    seq_len = [T] + [T - 333 * i for i in range(1, B)]
    log(f"decode dense bf16 T={T} B={B}")
    out, sm = _run_decode(d, seq_len)
    for b in range(B):
        ref = _decode_ref(d, b, np.arange(seq_len[b]), sm)
        assert rel_err(out[b], ref) <= TOL_BF16, b


def test_decode_selected_keys_and_keep_all_equals_dense():
    T, k = 700, 256
    d = synth.decode(20, T, B=2)
    rng = np.random.default_rng(21)
    sel = np.full((2, k), -1, np.int32)
    s0 = np.sort(rng.choice(T, k, replace=False)).astype(np.int32)
    s1 = np.sort(rng.choice(400, 100, replace=False)).astype(np.int32)
    sel[0], sel[1, :100] = s0, s1
    nsel = np.array([k, 100], np.int32)
    log("decode selected keys")
    out, sm = _run_decode(d, [T, 400], sel, nsel)
    assert rel_err(out[0], _decode_ref(d, 0, s0, sm)) <= TOL_BF16
    assert rel_err(out[1], _decode_ref(d, 1, s1, sm)) <= TOL_BF16
    # keeping every causal key reproduces the dense path bit for bit
    all_sel = np.tile(np.arange(T, dtype=np.int32), (2, 1))
    dense, _ = _run_decode(d, [T, T])
    kept, _ = _run_decode(d, [T, T], all_sel, np.array([T, T], np.int32))
    assert np.array_equal(dense, kept)


@pytest.mark.parametrize("bf16,B", [(True, 2), (False, 2), (True, 6)])
def test_decode_split_steps_equal_fused(bf16, B):
    """mla_decode_absorb followed by mla_decode_attend on one workspace gives the fused call's
    output bit for bit (matrix-core path for bf16 GLM shapes, with the batch kernels at B = 6;
    generic kernels for fp32)."""
    T, k = 900, 300
    d = synth.decode(40, T, B=B, bf16=bf16)
    rng = np.random.default_rng(41)
    sel = np.full((B, k), -1, np.int32)
    nsel = np.array([k, 77] + [int(rng.integers(1, k + 1)) for _ in range(B - 2)], np.int32)
    sel[0] = np.sort(rng.choice(T, k, replace=False))
    sel[1, :77] = np.sort(rng.choice(600, 77, replace=False))
    for b in range(2, B):
        sel[b, : nsel[b]] = np.sort(rng.choice(600, nsel[b], replace=False))
    to = dev_bf16 if bf16 else dev
    kv = _kv(d.lc, d.rc, None, [T] + [600] * (B - 1), T, seq_stride=T, bf16=bf16)
    sm = 1.0 / math.sqrt(d.nope + d.rope)
    qn, qr, kvb = to(d.q_nope), to(d.q_rope), to(d.kv_b)
    sl, ns = dev(sel), dev(nsel)
    log(f"decode split steps bf16={bf16} B={B}")
    fused = host(mla.mla_absorbed_decode(qn, qr, kvb, kv, sm, sel=sl, nsel=ns))
    need = mla.mla_decode_workspace_bytes(d.H, d.nope, d.rope, d.v, d.L, B, k)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    mla.mla_decode_absorb(qn, kvb, ws, qk_rope=d.rope)
    split = host(mla.mla_decode_attend(qr, kvb, kv, d.nope, sm, ws, sel=sl, nsel=ns))
    assert np.array_equal(fused, split)
    assert rel_err(split[1], _decode_ref(d, 1, sel[1, :77], sm)) <= (TOL_BF16 if bf16 else TOL_F32)


def test_decode_paged_equals_contiguous():
    T = 640
    d = synth.decode(30, T, B=2)
    bs = 64
    rng = np.random.default_rng(31)
    nb = T // bs
    perm = rng.permutation(2 * nb).astype(np.int32)
    bt = perm.reshape(2, nb)
    rows = 2 * nb * bs
    lc_p = np.zeros((rows, d.L), np.uint16)
    rc_p = np.zeros((rows, d.rope), np.uint16)
    for b in range(2):
        for j in range(nb):
            lc_p[bt[b, j] * bs:(bt[b, j] + 1) * bs] = d.lc[b * T + j * bs: b * T + (j + 1) * bs]
            rc_p[bt[b, j] * bs:(bt[b, j] + 1) * bs] = d.rc[b * T + j * bs: b * T + (j + 1) * bs]
    sm = 1.0 / math.sqrt(d.nope + d.rope)
    log("decode paged vs contiguous")
    kvp = _kv(lc_p, rc_p, None, [T, 500], T, block_table=bt, block_size=bs)
    outp = host(mla.mla_absorbed_decode(dev_bf16(d.q_nope), dev_bf16(d.q_rope), dev_bf16(d.kv_b), kvp, sm))
    outc, _ = _run_decode(d, [T, 500])
    assert np.array_equal(outp, outc)
    assert rel_err(outc[1], _decode_ref(d, 1, np.arange(500), sm)) <= TOL_BF16


def test_decode_empty_sequence_gives_zeros():
    d = synth.decode(40, 64, B=2)
    out, _ = _run_decode(d, [64, 0])
    assert np.all(out[1] == 0) and np.all(np.isfinite(out[0]))


def test_decode_repeat_runs_bit_identical():
    d = synth.decode(41, 2048)
    a, _ = _run_decode(d, [2048])
    b, _ = _run_decode(d, [2048])
    assert np.array_equal(a, b)


# ------------------------------------------------------------------------------ tiny layer (config 1)
def test_tiny_layer_gpu_rope_absorbed_and_nonabsorbed():
    """The tiny fp32 layer with the GPU doing the rotations: the raw kv_a and q_b tails (plain float64
    matmuls of the layer's weights, rounded to fp32) are rotated by mla_rope_interleave at each
    token's position (Rc) and at T - 1 (the query); the absorbed decode and the non-absorbed prefill
    (S = 1) of the rotated query then both match the oracle's tiny layer, whose RoPE is its own."""
    t = synth.tiny_layer(1)
    lc, rc, q = oracle.tiny_layer(t.x, t.q_a, t.q_b, t.kv_a, t.H, t.nope, t.rope, t.L)
    sm = 1.0 / math.sqrt(t.nope + t.rope)
    ref = oracle.absorbed_decode(q[:, : t.nope].astype(np.float32), q[:, t.nope:].astype(np.float32), t.kv_b,
                                 lc.astype(np.float32), rc.astype(np.float32), np.arange(t.T), t.v, sm)
    comp = t.x.astype(np.float64) @ t.kv_a.astype(np.float64).T
    qa = t.q_a.astype(np.float64) @ t.x[-1].astype(np.float64)
    qa = qa / np.sqrt((qa ** 2).mean() + 1e-6)
    qf = (t.q_b.astype(np.float64) @ qa).reshape(t.H, t.nope + t.rope).astype(np.float32)
    log("tiny layer: GPU RoPE, absorbed and non-absorbed")
    rc_d = dev(np.ascontiguousarray(comp[:, t.L:].astype(np.float32)).reshape(t.T, 1, t.rope))
    mla.mla_rope_interleave(rc_d, dev(np.arange(t.T, dtype=np.int32)), 0, t.rope)
    q_d = dev(qf[None])
    mla.mla_rope_interleave(q_d, dev(np.array([t.T - 1], np.int32)), t.nope, t.rope)
    assert np.abs(host(rc_d).reshape(t.T, t.rope) - rc).max() <= 2e-6 * np.abs(rc).max()
    kv = mla.KvCache(dev(lc.astype(np.float32)), rc_d.reshape(t.T, t.rope), max_seq_len=t.T, seq_stride=t.T,
                     seq_len=dev(np.array([t.T], np.int32)))
    q_h = q_d[0]
    out_a = host(mla.mla_absorbed_decode(q_h[None, :, : t.nope].contiguous(), q_h[None, :, t.nope:].contiguous(),
                                         dev(t.kv_b), kv, sm))[0]
    out_n = host(mla.mla_prefill_nonabsorbed(q_d, dev(t.kv_b), kv, t.nope, t.T - 1, sm))[0]
    assert rel_err(out_a, ref) <= TOL_F32
    assert rel_err(out_n, ref) <= TOL_F32


# ------------------------------------------------------------------------------ prefill
def test_prefill_tiny_fp32_last_row_equals_decode():
    t = synth.tiny_layer(1)
    lc, rc, q = oracle.tiny_layer(t.x, t.q_a, t.q_b, t.kv_a, t.H, t.nope, t.rope, t.L)
    lc32, rc32, q32 = lc.astype(np.float32), rc.astype(np.float32), q.astype(np.float32)
    sm = 1.0 / math.sqrt(t.nope + t.rope)
    log("prefill tiny fp32 S=1")
    kv = mla.KvCache(dev(lc32), dev(rc32), max_seq_len=t.T, seq_stride=t.T)
    out = host(mla.mla_prefill_nonabsorbed(dev(q32[None]), dev(t.kv_b), kv, t.nope, t.T - 1, sm))[0]
    ref = oracle.absorbed_decode(q32[:, : t.nope], q32[:, t.nope:], t.kv_b, lc32, rc32, np.arange(t.T), t.v, sm)
    assert rel_err(out, ref) <= TOL_F32


@pytest.mark.parametrize("S,pos_base,out_bf16", [(130, 0, False), (77, 50, True)])
def test_prefill_small_glm_heads(S, pos_base, out_bf16):
    p = synth.prefill(60 + S, S, pos_base, H_=4)
    sm = 1.0 / math.sqrt(p.nope + p.rope)
    log(f"prefill S={S} pos_base={pos_base}")
    kv = _kv(p.lc, p.rc, None, None, pos_base + S, seq_stride=pos_base + S)
    out = mla.mla_prefill_nonabsorbed(dev_bf16(p.q), dev_bf16(p.kv_b), kv, p.nope, pos_base, sm,
                                      out_dtype=torch.bfloat16 if out_bf16 else torch.float32)
    out = host(out)
    cv = synth.bf16_bits_to_f32
    rows = np.unique(np.r_[0, S - 1, np.linspace(0, S - 1, 9).astype(int)])
    ref = oracle.prefill_rows(cv(p.q), cv(p.kv_b), cv(p.lc), cv(p.rc), pos_base, p.nope, p.v, sm, rows)
    assert rel_err(out[rows], ref) <= TOL_BF16


def _prefill_glm_check(S, pos_base, seed, out_bf16, rows, heads, bs=0):
    """64-head GLM geometry (the matrix-core path): rows x heads of the output against the oracle."""
    p = synth.prefill(seed, S, pos_base)
    T = pos_base + S
    sm = 1.0 / math.sqrt(p.nope + p.rope)
    if bs:
        rng = np.random.default_rng(seed + 1)
        lc_p, bt = _paged_copy([p.lc], bs, rng)
        rc_p, _ = _paged_copy([p.rc], bs, np.random.default_rng(seed + 1))
        kv = _kv(lc_p, rc_p, None, None, T, block_table=bt, block_size=bs)
    else:
        kv = _kv(p.lc, p.rc, None, None, T, seq_stride=T)
    out = mla.mla_prefill_nonabsorbed(dev_bf16(p.q), dev_bf16(p.kv_b), kv, p.nope, pos_base, sm,
                                      out_dtype=torch.bfloat16 if out_bf16 else torch.float32)
    out = host(out)
    cv = synth.bf16_bits_to_f32
    R = p.nope + p.v
    kvb_h = np.concatenate([p.kv_b[h * R:(h + 1) * R] for h in heads])
    ref = oracle.prefill_rows(cv(p.q)[:, heads], cv(kvb_h), cv(p.lc), cv(p.rc), pos_base, p.nope, p.v, sm, rows)
    got = out[rows][:, heads]
    assert np.isfinite(got).all()
    assert rel_err(got, ref) <= TOL_BF16
    return out


@pytest.mark.parametrize("S,pos_base,out_bf16,bs", [(300, 0, False, 0), (200, 333, True, 0), (256, 64, False, 64),
                                                    (280, 40, False, 32), (300, 36, True, 16)])
def test_prefill_glm_64_heads(S, pos_base, out_bf16, bs):
    """Ragged query blocks and token tiles, a pos_base offset, bf16 output, a paged cache."""
    log(f"prefill 64 heads S={S} pos_base={pos_base} bf16={out_bf16} bs={bs}")
    rows = np.unique(np.r_[0, 1, S - 1, np.linspace(0, S - 1, 7).astype(int)])
    _prefill_glm_check(S, pos_base, 110 + S, out_bf16, rows, [0, 5, 31, 63], bs=bs)


def test_prefill_full_4096_sampled_rows():
    """S = T = 4096 (the benchmark configuration): 64 evenly spaced query rows, including 0 and
    S - 1, on all 64 heads, against the oracle."""
    S = 4096
    log("prefill S=T=4096, 64 rows x 64 heads")
    rows = np.unique(np.linspace(0, S - 1, 64).round().astype(int))
    assert rows.size == 64 and rows[0] == 0 and rows[-1] == S - 1
    _prefill_glm_check(S, 0, 4, False, rows, list(range(64)))


@pytest.mark.parametrize("T", [1, 777, 4096])
def test_prefill_single_query_equals_absorbed_decode(T):
    """colibri-analysis 06, sec. 2.3: the two attention paths compute the same function.  One
    prefill query at pos_base = T - 1 on the matrix-core kernels (64 heads, GLM shapes) equals the
    oracle's absorbed decode of that query over keys 0..T-1."""
    p = synth.prefill(170 + T, 1, T - 1)
    sm = 1.0 / math.sqrt(p.nope + p.rope)
    log(f"prefill S=1 pos_base={T - 1} vs absorbed decode")
    kv = _kv(p.lc, p.rc, None, None, T, seq_stride=T)
    out = host(mla.mla_prefill_nonabsorbed(dev_bf16(p.q), dev_bf16(p.kv_b), kv, p.nope, T - 1, sm))[0]
    cv = synth.bf16_bits_to_f32
    q = cv(p.q)[0]
    ref = oracle.absorbed_decode(q[:, : p.nope], q[:, p.nope:], cv(p.kv_b), cv(p.lc), cv(p.rc), np.arange(T),
                                 p.v, sm)
    assert rel_err(out, ref) <= TOL_BF16


@pytest.mark.parametrize("H_,S,pos_base,bs,holes", [(64, 200, 56, 64, (0, 2)), (64, 150, 106, 16, (0, 5, 6)),
                                                    (4, 90, 38, 16, (0, 3))])
def test_prefill_paged_hole(H_, S, pos_base, bs, holes):
    """Keys in a block-table hole (entry -1) have no row and are not attended, as in the decode: on
    the matrix-core kernels (64 heads; block size 64 looks a tile up once, 16 once per key) and on
    the generic ones (4 heads).  Block 0 is a hole, so the first queries start with no attended
    key (their output is 0 while they see holes only).  Reference: the oracle's non-absorbed
    attention over the keys that have a row."""
    T = pos_base + S
    assert T % bs == 0
    p = synth.prefill(190 + S + bs, S, pos_base, H_=H_)
    sm = 1.0 / math.sqrt(p.nope + p.rope)
    lc_p, bt = _paged_copy([p.lc], bs, np.random.default_rng(191 + S))
    rc_p, _ = _paged_copy([p.rc], bs, np.random.default_rng(191 + S))
    bt = bt.copy()
    bt[0, list(holes)] = -1
    log(f"prefill paged hole H={H_} S={S} pos_base={pos_base} bs={bs} holes={holes}")
    kv = _kv(lc_p, rc_p, None, None, T, block_table=bt, block_size=bs)
    out = host(mla.mla_prefill_nonabsorbed(dev_bf16(p.q), dev_bf16(p.kv_b), kv, p.nope, pos_base, sm))
    assert np.isfinite(out).all()
    valid = np.ones(T, bool)
    for j in holes:
        valid[j * bs:(j + 1) * bs] = False
    cv = synth.bf16_bits_to_f32
    q, lc, rc, kvb = cv(p.q), cv(p.lc), cv(p.rc), cv(p.kv_b)
    rows = np.unique(np.r_[0, 1, S - 1, np.linspace(0, S - 1, 8).astype(int)])
    empty = 0
    for i in rows:
        keys = np.nonzero(valid[: pos_base + i + 1])[0]
        if keys.size == 0:
            assert np.all(out[i] == 0), i
            empty += 1
            continue
        ref = oracle.nonabsorbed_decode(q[i][:, : p.nope], q[i][:, p.nope:], kvb, lc, rc, keys, p.v, sm)
        assert rel_err(out[i], ref) <= TOL_BF16, i
    assert empty == (1 if pos_base < bs else 0) * int(np.sum(rows + pos_base < bs))


# ------------------------------------------------------------------------------ end to end
def test_dsa_decode_step_end_to_end_small():
    """index -> top-k -> absorbed decode over the selected keys, at a size with T > k."""
    T, k = 5000, 512
    d = synth.decode(70, T, dsa=True)
    log("end-to-end DSA decode T=5000 k=512")
    kv = _kv(d.lc, d.rc, d.ic, [T], T, seq_stride=T)
    scores = mla.dsa_index_scores(dev(d.q_idx), dev(d.w_idx), kv, T)
    sel, nsel = mla.dsa_topk_select(scores, dev(np.array([T], np.int32)), k)
    sm = 1.0 / math.sqrt(d.nope + d.rope)
    out = host(mla.mla_absorbed_decode(dev_bf16(d.q_nope), dev_bf16(d.q_rope), dev_bf16(d.kv_b), kv, sm,
                                       sel=sel, nsel=nsel))
    ref_s = oracle.index_scores(d.q_idx[0], d.w_idx[0], d.ic)
    ref_sel, ref_n = oracle.topk(ref_s, T, k)
    assert int(host(nsel)[0]) == ref_n == k
    assert np.array_equal(host(sel)[0], ref_sel)
    assert rel_err(out[0], _decode_ref(d, 0, ref_sel, sm)) <= TOL_BF16


def _paged_copy(rows_by_seq, bs, rng):
    """Scatter per-sequence row arrays [B][T, w] into a pool of bs-row blocks in a random
    physical order; returns (pool, block_table [B, T/bs])."""
    B, T = len(rows_by_seq), rows_by_seq[0].shape[0]
    nb = T // bs
    perm = rng.permutation(B * nb).astype(np.int32)
    bt = perm.reshape(B, nb)
    pool = np.zeros((B * nb * bs, rows_by_seq[0].shape[1]), rows_by_seq[0].dtype)
    for b in range(B):
        for j in range(nb):
            pool[bt[b, j] * bs:(bt[b, j] + 1) * bs] = rows_by_seq[b][j * bs:(j + 1) * bs]
    return pool, bt


def _dsa_step_check(d, kv, seq_len, t_max, k, theta=10000.0, oracle_rows=()):
    """mla_dsa_decode == mla_rope_interleave (at seq_len - 1, on a copy) + dsa_index_select +
    mla_absorbed_decode, bit for bit; q_rope is left unrotated; rows in oracle_rows are also
    checked against the oracle (selection and attention)."""
    to = dev_bf16 if d.bf16 else dev
    qn, qr, kvb = to(d.q_nope), to(d.q_rope), to(d.kv_b)
    qi, wi = dev(d.q_idx), dev(d.w_idx)
    qr0 = qr.clone()
    sm = 1.0 / math.sqrt(d.nope + d.rope)
    out, sc, sel, nsel = mla.mla_dsa_decode(qn, qr, qi, wi, kvb, kv, t_max, k, sm, theta=theta)
    assert torch.equal(qr, qr0)
    qr2 = qr.clone()
    pos = dev(np.maximum(np.minimum(np.asarray(seq_len, np.int32), t_max) - 1, 0).astype(np.int32))
    mla.mla_rope_interleave(qr2, pos, 0, d.rope, theta=theta)
    sc2, sel2, nsel2 = mla.dsa_index_select(qi, wi, kv, t_max, k)
    out2 = mla.mla_absorbed_decode(qn, qr2, kvb, kv, sm, sel=sel2, nsel=nsel2)
    assert np.array_equal(host(sc).view(np.uint32), host(sc2).view(np.uint32))
    assert np.array_equal(host(sel), host(sel2)) and np.array_equal(host(nsel), host(nsel2))
    assert np.array_equal(host(out), host(out2))
    cv = synth.bf16_bits_to_f32 if d.bf16 else (lambda a: a)
    for b in oracle_rows:
        n = min(seq_len[b], t_max)
        ref_s = oracle.index_scores(d.q_idx[b], d.w_idx[b], d.ic[b * d.T:b * d.T + n])
        ref_sel, ref_n = oracle.topk(ref_s, n, k)
        ref_sel = ref_sel[:ref_n]
        assert int(host(nsel)[b]) == ref_n and np.array_equal(host(sel)[b, :ref_n], ref_sel)
        q_rot = oracle.rope_interleave(cv(d.q_rope[b])[None], np.array([n - 1], np.int32), 0, d.rope, theta)[0]
        ref = oracle.absorbed_decode(cv(d.q_nope[b]), q_rot, cv(d.kv_b), cv(d.lc[b * d.T:(b + 1) * d.T]),
                                     cv(d.rc[b * d.T:(b + 1) * d.T]), ref_sel, d.v, sm)
        assert rel_err(host(out)[b], ref) <= (TOL_BF16 if d.bf16 else TOL_F32), b
    return host(out), host(sel), host(nsel)


@pytest.mark.parametrize("tiled", [False, True])
def test_dsa_decode_call_full_context_131072(tiled):
    T, k = 131072, 2048
    d = synth.decode(3, T, dsa=True)
    log(f"mla_dsa_decode T=131072 k=2048 tiled={tiled}")
    kv = _kv(d.lc, d.rc, d.ic, [T], T, seq_stride=T, tiled=tiled)
    _dsa_step_check(d, kv, [T], T, k, oracle_rows=(0,))


def test_dsa_decode_call_batched_and_short_rows():
    """Rows above and below k (a short row keeps every key: the dense decode), a ragged
    tail, and t_max beyond the longest row."""
    T, k = 6000, 1024
    seq_len = [6000, 700, 4097]
    d = synth.decode(95, T, B=3, dsa=True)
    log("mla_dsa_decode batched")
    kv = _kv(d.lc, d.rc, d.ic, seq_len, T, seq_stride=T)
    out, sel, nsel = _dsa_step_check(d, kv, seq_len, T, k, theta=50000.0, oracle_rows=(0, 1, 2))
    assert int(nsel[1]) == 700 and np.array_equal(sel[1, :700], np.arange(700))


def test_dsa_decode_call_paged():
    T, k, bs = 4096, 512, 64
    seq_len = [4096, 3000]
    d = synth.decode(96, T, B=2, dsa=True)
    rng = np.random.default_rng(97)
    split = lambda a: [a[b * T:(b + 1) * T] for b in range(2)]
    lc_p, bt = _paged_copy(split(d.lc), bs, rng)
    rc_p, _ = _paged_copy(split(d.rc), bs, np.random.default_rng(97))
    ic_p, _ = _paged_copy(split(d.ic), bs, np.random.default_rng(97))
    log("mla_dsa_decode paged")
    kv = _kv(lc_p, rc_p, ic_p, seq_len, T, block_table=bt, block_size=bs)
    _dsa_step_check(d, kv, seq_len, T, k, oracle_rows=(1,))


def test_dsa_decode_call_batched_paged_full_size():
    """The batched paged step at full size, as the benchmark launches it: 32 sequences of
    8k..131k tokens in 64-token blocks in a random physical order, the indexer pool tiled,
    k = 2048.  The fused call equals the composed calls bit for bit on every row; the
    shortest, the longest and the first sequence also meet the oracle."""
    pb = synth.paged_batch(5, meta_only=True)
    T, k, bs = pb.max_blocks * pb.block_size, synth.TOPK, pb.block_size
    log(f"mla_dsa_decode batched paged B={pb.B} sum_len={int(pb.seq_len.sum())} T={T} k={k}")
    d = synth.paged_values_torch(pb, 1005, torch.device("cuda:0"))
    qn, qr, qi, wi, kvb = d["q_nope"], d["q_rope"], d["q_idx"], d["w_idx"], d["kv_b"]
    kv = mla.KvCache(d["lc"], d["rc"], synth.tile_index_keys(d["ic"]), seq_len=dev(pb.seq_len), max_seq_len=T,
                     block_table=dev(pb.block_table), block_size=bs, ic_layout=mla.MLA_IC_TILE64)
    sm = 1.0 / math.sqrt(pb.nope + pb.rope)
    qr0 = qr.clone()
    out, sc, sel, nsel = mla.mla_dsa_decode(qn, qr, qi, wi, kvb, kv, T, k, sm)
    assert torch.equal(qr, qr0)
    qr2 = qr.clone()
    mla.mla_rope_interleave(qr2, dev(pb.seq_len - 1), 0, pb.rope)
    sc2, sel2, nsel2 = mla.dsa_index_select(qi, wi, kv, T, k)
    out2 = mla.mla_absorbed_decode(qn, qr2, kvb, kv, sm, sel=sel2, nsel=nsel2)
    assert torch.equal(sc.view(torch.int32), sc2.view(torch.int32))
    assert torch.equal(sel, sel2) and torch.equal(nsel, nsel2) and torch.equal(out, out2)
    assert bool((nsel == k).all())
    sc_h, sel_h, out_h = host(sc), host(sel), host(out)
    for b in sorted({int(np.argmin(pb.seq_len)), int(np.argmax(pb.seq_len)), 0}):
        n = int(pb.seq_len[b])
        log(f"  oracle row {b} len {n}")
        r = dev(pb.rows(b, np.arange(n)))
        ref_s = oracle.index_scores(host(qi[b]), host(wi[b]), host(d["ic"].index_select(0, r)))
        assert np.array_equal(sc_h[b, :n].view(np.uint32), ref_s.view(np.uint32)), b
        assert np.all(np.isneginf(sc_h[b, n:])), b
        ref_sel, ref_n = oracle.topk(ref_s, n, k)
        assert ref_n == k and np.array_equal(sel_h[b], ref_sel[:k]), b
        q_rot = oracle.rope_interleave(host(qr0[b])[None], np.array([n - 1], np.int32), 0, pb.rope)[0]
        ref = oracle.absorbed_decode(host(qn[b]), q_rot, host(kvb), host(d["lc"].index_select(0, r)),
                                     host(d["rc"].index_select(0, r)), ref_sel[:k], pb.v, sm)
        assert rel_err(out_h[b], ref) <= TOL_BF16, b


def test_dsa_decode_call_fp32_generic_path():
    T, k = 1500, 256
    d = synth.decode(98, T, B=2, dsa=True, bf16=False)
    seq_len = [1500, 200]
    log("mla_dsa_decode fp32")
    kv = _kv(d.lc, d.rc, d.ic, seq_len, T, seq_stride=T, bf16=False)
    _dsa_step_check(d, kv, seq_len, T, k, oracle_rows=(0, 1))


def test_topk_all_equal_full_context():
    # every score in one threshold bin: all 131072 positions become candidates
    T = 131072
    s = np.full((1, T), 0.75, np.float32)
    log("topk all equal T=131072")
    _topk_check(s, [T], 2048)
    s[0, 5000:5100] = 0.7500001
    _topk_check(s, [T], 2048)


def test_decode_generic_and_matrix_core_paths_agree():
    """The same GLM-shape values through the matrix-core kernels (bf16) and the generic kernels
    (the same values widened to fp32) both meet the oracle; a query pointer 2 bytes off is
    rejected with MLA_ERR_UNSUPPORTED, never routed to other kernels."""
    T = 900
    d = synth.decode(80, T, B=2)
    sm = 1.0 / math.sqrt(d.nope + d.rope)
    kv = _kv(d.lc, d.rc, None, [T, 611], T, seq_stride=T)
    qn = dev_bf16(d.q_nope)
    buf = torch.empty(qn.numel() + 1, dtype=torch.bfloat16, device=qn.device)
    qn_mis = buf[1:].view(qn.shape)
    qn_mis.copy_(qn)
    log("decode generic vs matrix-core")
    fast = host(mla.mla_absorbed_decode(qn, dev_bf16(d.q_rope), dev_bf16(d.kv_b), kv, sm))
    with pytest.raises(mla.MlaError) as e:
        mla.mla_absorbed_decode(qn_mis, dev_bf16(d.q_rope), dev_bf16(d.kv_b), kv, sm)
    assert e.value.status == mla.MLA_ERR_UNSUPPORTED
    f32 = lambda bits: dev(synth.bf16_bits_to_f32(bits))
    kv32 = _kv(synth.bf16_bits_to_f32(d.lc), synth.bf16_bits_to_f32(d.rc), None, [T, 611], T, seq_stride=T,
               bf16=False)
    slow = host(mla.mla_absorbed_decode(f32(d.q_nope), f32(d.q_rope), f32(d.kv_b), kv32, sm))
    for b, n in enumerate([T, 611]):
        ref = _decode_ref(d, b, np.arange(n), sm)
        assert rel_err(fast[b], ref) <= TOL_BF16
        assert rel_err(slow[b], ref) <= TOL_F32


@pytest.mark.parametrize("B", [4, 5])
def test_decode_batched_long_splits_and_growing_scores(B):
    """More than 256 keys per split (dense, 20000 keys) on both batch paths -- four queries on the
    per-head-group kernel (64 splits of 320 keys), five on the all-heads kernel (52 splits of 448)
    -- and scores that grow along the sequence (latent rows scaled up with the position), so later
    chunks keep raising the running maximum."""
    T = 20000
    d = synth.decode(83, T, B=B)
    lc = synth.bf16_bits_to_f32(d.lc).reshape(B, T, -1)
    lc *= (1.0 + np.arange(T, dtype=np.float32) / 2000.0)[None, :, None]
    d.lc = synth.to_bf16_bits(lc.reshape(B * T, -1))
    seq_len = [T, 19999, 16385, 300, 12345][:B]
    log(f"decode batched long splits B={B}")
    out, sm = _run_decode(d, seq_len)
    for b in (0, 2, 3, B - 1):
        assert rel_err(out[b], _decode_ref(d, b, np.arange(seq_len[b]), sm)) <= TOL_BF16, b


@pytest.mark.parametrize("B", [64, 300])
def test_decode_large_batch_shared_pool(B):
    """Batches large enough that the all-heads kernel splits the keys little or not at all (B = 64:
    four splits of 512 keys; B = 300: one split of 2048, so each query's partial is its whole
    attention), every sequence reading the same 2048 pool rows through its block table; sampled
    rows against the oracle."""
    T, bs = 2048, 64
    pool = synth.decode(86, T)
    qs = synth.decode(87 + B, 1, B=B)
    rng = np.random.default_rng(88 + B)
    seq_len = rng.integers(1, T + 1, B).astype(np.int32)
    seq_len[:3] = [T, T - 1, 65]
    bt = np.tile(np.arange(T // bs, dtype=np.int32), (B, 1))
    kv = _kv(pool.lc, pool.rc, None, seq_len, T, block_table=bt, block_size=bs)
    sm = 1.0 / math.sqrt(pool.nope + pool.rope)
    log(f"decode large batch B={B} over one shared pool")
    out = host(mla.mla_absorbed_decode(dev_bf16(qs.q_nope), dev_bf16(qs.q_rope), dev_bf16(pool.kv_b), kv, sm))
    cv = synth.bf16_bits_to_f32
    lc, rc, kvb = cv(pool.lc), cv(pool.rc), cv(pool.kv_b)
    for b in sorted({0, 1, 2, B // 2, B - 1}):
        ref = oracle.absorbed_decode(cv(qs.q_nope[b]), cv(qs.q_rope[b]), kvb, lc, rc, np.arange(seq_len[b]),
                                     pool.v, sm)
        assert rel_err(out[b], ref) <= TOL_BF16, b


@pytest.mark.parametrize("nope,v", [(128, 128), (256, 192)])
def test_decode_batched_other_head_dims(nope, v):
    """Batches on the matrix-core absorption and all-heads attention with the other supported
    qk_nope sizes, as separate calls and inside the fused step (its absorption runs beside the
    selection); the two equal each other bit for bit and meet the oracle."""
    B, T, k = 5, 1500, 512
    d = synth.decode(84 + nope, T, B=B, nope=nope, v=v, dsa=True)
    seq_len = [T, 1499, 900, 513, 200]
    log(f"decode batched nope={nope} v={v}")
    out, sm = _run_decode(d, seq_len)
    for b in (0, 4):
        assert rel_err(out[b], _decode_ref(d, b, np.arange(seq_len[b]), sm)) <= TOL_BF16, b
    kv = _kv(d.lc, d.rc, d.ic, seq_len, T, seq_stride=T)
    _dsa_step_check(d, kv, seq_len, T, k, oracle_rows=(1, 4))


def test_dsa_decode_call_batch_over_side_limit():
    """40 sequences (more than the selection's side workgroups take: the absorption runs as its
    own launch) of ragged lengths, some shorter than k; fused call == composed calls, rows
    against the oracle."""
    B, T, k = 40, 700, 256
    d = synth.decode(85, T, B=B, dsa=True)
    seq_len = [T - 13 * b for b in range(B)]
    seq_len[7] = 100
    log("mla_dsa_decode B=40")
    kv = _kv(d.lc, d.rc, d.ic, seq_len, T, seq_stride=T)
    out, sel, nsel = _dsa_step_check(d, kv, seq_len, T, k, oracle_rows=(0, 7, 39))
    assert int(nsel[7]) == 100


def test_decode_dense_4096_full_heads():
    """The dense decode configuration at full size: one query over all 4096 cached keys, 64
    heads (sel = NULL, the path `dense_decode_T4096` of the benchmark times), against the
    oracle; the same keys passed as an explicit selection give the same bits."""
    T = 4096
    d = synth.decode(2, T)
    log("decode dense T=4096")
    out, sm = _run_decode(d, [T])
    assert rel_err(out[0], _decode_ref(d, 0, np.arange(T), sm)) <= TOL_BF16
    sel = np.arange(T, dtype=np.int32)[None]
    out_sel, _ = _run_decode(d, [T], sel, np.array([T], np.int32))
    assert np.array_equal(out, out_sel)


def test_decode_batched_selected_large():
    """Many sequences with selections of different sizes (covers multi-tile splits)."""
    B, T, k = 6, 3000, 2048
    d = synth.decode(81, T, B=B)
    rng = np.random.default_rng(82)
    sel = np.full((B, k), -1, np.int32)
    nsel = np.array([2048, 1, 0, 777, 2048, 33], np.int32)
    for b in range(B):
        sel[b, : nsel[b]] = np.sort(rng.choice(T, nsel[b], replace=False))
    log("decode batched selected")
    out, sm = _run_decode(d, [T] * B, sel, nsel)
    for b in range(B):
        if nsel[b] == 0:
            assert np.all(out[b] == 0)
            continue
        assert rel_err(out[b], _decode_ref(d, b, sel[b, : nsel[b]], sm)) <= TOL_BF16, b
