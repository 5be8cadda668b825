"""GPU parity of attention over S queries of one sequence (multi-query absorbed decode with the
g_absorb rule) and of DSA in prefill (per-query selection, sparse attention on either path).

Pages: chen3feng, "colibri-analysis 06: MLA attention and KV cache", sec. 2 (query i of S at position
pos_base + i over Tk = pos_base + S keys), sec. 2.2 (the indexer and top-k whenever the context
exceeds k, prefill included) and sec. 2.3 (g_absorb: absorbed when S <= 4 by default; both paths
compute the same function).  Bars: scores bit-exact, sel / nsel bit-exact, attention within 1e-2 (bf16)
or 2e-3 (fp32) of the oracle.
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
cv = synth.bf16_bits_to_f32


def _paged(rows, bs, seed):
    """rows [T, w] scattered into a pool of bs-row blocks in a seeded random order (+ block table [1, nb])."""
    T = rows.shape[0]
    nb = (T + bs - 1) // bs
    perm = np.random.default_rng(seed).permutation(nb).astype(np.int32)
    pool = np.zeros((nb * bs, rows.shape[1]), rows.dtype)
    for j in range(nb):
        n = min(bs, T - j * bs)
        pool[perm[j] * bs: perm[j] * bs + n] = rows[j * bs: j * bs + n]
    return pool, perm[None]


def _kv(p, bs=0):
    T = p.lc.shape[0]
    to = dev_bf16 if p.bf16 else dev
    if bs:
        lc, bt = _paged(p.lc, bs, 700 + bs)
        rc, _ = _paged(p.rc, bs, 700 + bs)
        return mla.KvCache(to(lc), to(rc), max_seq_len=T, block_table=dev(bt), block_size=bs)
    return mla.KvCache(to(p.lc), to(p.rc), max_seq_len=T, seq_stride=T)


def _ref_rows(p, rows, keys_of, sm):
    """Oracle: the absorbed decode of query i over keys_of(i) (absorbed == non-absorbed is pinned)."""
    f = cv if p.bf16 else (lambda a: a)
    q = f(p.q)
    out = []
    for i in rows:
        out.append(oracle.absorbed_decode(q[i, :, : p.nope], q[i, :, p.nope:], f(p.kv_b), f(p.lc), f(p.rc),
                                          keys_of(i), p.v, sm))
    return np.stack(out)


@pytest.mark.parametrize("S", [1, 2, 3, 4])
@pytest.mark.parametrize("bs", [0, 16])
def test_multi_query_decode_both_paths(S, bs):
    """S <= 4 draft queries at the end of a 3000-token sequence: the default rule absorbs; forcing the
    non-absorbed path gives the same function; both match the oracle query by query."""
    T = 3000
    p = synth.prefill(720 + S, S, T - S)
    sm = 1.0 / math.sqrt(p.nope + p.rope)
    kv = _kv(p, bs)
    assert mla.mla_attention_absorbs(S, -1)
    log(f"multi-query decode S={S} bs={bs}")
    q = dev_bf16(p.q)
    a = host(mla.mla_attention(q, dev_bf16(p.kv_b), kv, p.nope, T - S, sm, g_absorb=-1))
    n = host(mla.mla_attention(q, dev_bf16(p.kv_b), kv, p.nope, T - S, sm, g_absorb=0))
    ref = _ref_rows(p, range(S), lambda i: np.arange(T - S + i + 1), sm)
    assert rel_err(a, ref) <= TOL_BF16
    assert rel_err(n, ref) <= TOL_BF16


def test_multi_query_decode_fp32_generic_geometry():
    """The tiny geometry in fp32 (generic kernels) on both paths, S = 3 at pos_base 61."""
    S, pb = 3, 61
    p = synth.prefill(730, S, pb, H_=4, nope=16, rope=8, v=16, L=32, bf16=False, w_std=0.3)
    sm = 1.0 / math.sqrt(p.nope + p.rope)
    kv = _kv(p)
    log("multi-query decode fp32 tiny")
    ref = _ref_rows(p, range(S), lambda i: np.arange(pb + i + 1), sm)
    for g in (-1, 0):
        out = host(mla.mla_attention(dev(p.q), dev(p.kv_b), kv, p.nope, pb, sm, g_absorb=g))
        assert rel_err(out, ref) <= TOL_F32, g


def _rand_sel(S, pb, k, seed, extra=True):
    """Per-query selections of at most k causal keys (sorted), with some entries past the query's
    position or negative (skipped by the call) and one empty row."""
    rng = np.random.default_rng(seed)
    sel = np.full((S, k), -1, np.int32)
    nsel = np.zeros(S, np.int32)
    keys = []
    for i in range(S):
        n_c = pb + i + 1
        m = min(k, n_c) if i % 5 else min(k // 3, n_c)
        ks = np.sort(rng.choice(n_c, m, replace=False)).astype(np.int32)
        row = ks.copy()
        if extra and m < k:
            row = np.r_[row, pb + i + 1 + rng.integers(0, 50)].astype(np.int32)   # a future key: skipped
        sel[i, : row.size] = row
        nsel[i] = row.size
        keys.append(ks)
    sel[S // 2], nsel[S // 2], keys[S // 2] = -1, 0, np.zeros(0, np.int32)
    return sel, nsel, keys


@pytest.mark.parametrize("S,pb,k,bs", [(4, 900, 256, 0), (300, 40, 128, 0), (200, 333, 256, 64), (130, 60, 64, 32)])
def test_sparse_attention_both_paths(S, pb, k, bs):
    """Given per-query selections (ragged, some entries in the future, one empty row), the absorbed and
    the non-absorbed paths (key bitmap on the matrix-core prefill) both match the oracle over exactly
    each query's causal selected keys; the empty row gives zeros."""
    p = synth.prefill(740 + S, S, pb)
    sm = 1.0 / math.sqrt(p.nope + p.rope)
    kv = _kv(p, bs)
    sel, nsel, keys = _rand_sel(S, pb, k, 741 + S)
    q, kvb = dev_bf16(p.q), dev_bf16(p.kv_b)
    rows = np.unique(np.r_[0, S // 2, S - 1, np.linspace(0, S - 1, 6).astype(int)])
    rows_ne = [r for r in rows if r != S // 2]
    ref = _ref_rows(p, rows_ne, lambda i: keys[i], sm)
    for g in (1, 0):
        log(f"sparse attention S={S} pb={pb} k={k} bs={bs} g_absorb={g}")
        out = host(mla.mla_attention(q, kvb, kv, p.nope, pb, sm, g_absorb=g, sel=dev(sel), nsel=dev(nsel)))
        assert np.all(out[S // 2] == 0), g
        assert np.isfinite(out).all()
        assert rel_err(out[rows_ne], ref) <= TOL_BF16, g


def test_sparse_attention_fp32_generic_geometry():
    S, pb, k = 40, 30, 16
    p = synth.prefill(750, S, pb, H_=4, nope=16, rope=8, v=16, L=32, bf16=False, w_std=0.3)
    sm = 1.0 / math.sqrt(p.nope + p.rope)
    kv = _kv(p)
    sel, nsel, keys = _rand_sel(S, pb, k, 751)
    rows = [r for r in range(S) if r != S // 2]
    ref = _ref_rows(p, rows, lambda i: keys[i], sm)
    log("sparse attention fp32 tiny")
    for g in (1, 0):
        out = host(mla.mla_attention(dev(p.q), dev(p.kv_b), kv, p.nope, pb, sm, g_absorb=g, sel=dev(sel),
                                     nsel=dev(nsel)))
        assert np.all(out[S // 2] == 0)
        assert rel_err(out[rows], ref) <= TOL_F32, g


def _ic_case(seed, T, hd=128, n_ih=32, S=1):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((T, hd)).astype(np.float32), rng.standard_normal((S, n_ih, hd)).astype(np.float32),
            rng.standard_normal((S, n_ih)).astype(np.float32))


@pytest.mark.parametrize("S,pb,k,tiled", [(300, 700, 256, False), (64, 4000, 2048, True), (257, 0, 64, False)])
def test_prefill_select_per_query(S, pb, k, tiled):
    """dsa_prefill_select: row i scores keys 0 .. pb + i (bit for bit, -inf after) and keeps their top-k
    exactly as the oracle's sort does; rows with pb + i + 1 <= k keep every causal key."""
    T = pb + S
    Tp = (T + 63) // 64 * 64
    ic, qi, wi = _ic_case(760 + S, Tp, S=S)
    z = np.zeros((Tp, 8), np.uint16)
    kv = mla.KvCache(dev_bf16(z), dev_bf16(z), dev(synth.tile_index_keys(ic) if tiled else ic), max_seq_len=T,
                     seq_stride=Tp, ic_layout=mla.MLA_IC_TILE64 if tiled else mla.MLA_IC_ROWS)
    log(f"prefill select S={S} pb={pb} k={k} tiled={tiled}")
    sc, sel, nsel = (host(x) for x in mla.dsa_prefill_select(dev(qi), dev(wi), kv, pb, k))
    for i in np.unique(np.r_[0, 1, S - 1, np.linspace(0, S - 1, 12).astype(int)]):
        n = pb + i + 1
        ref = oracle.index_scores(qi[i], wi[i], ic[:n])
        assert np.array_equal(sc[i, :n].view(np.uint32), ref.view(np.uint32)), i
        assert np.all(np.isneginf(sc[i, n:])), i
        rs, rn = oracle.topk(ref, n, k)
        assert int(nsel[i]) == rn and np.array_equal(sel[i], rs), i


@pytest.mark.parametrize("layout", ["rows", "tiled", "paged64", "paged16", "paged64_tiled"])
def test_prefill_select_every_row_all_layouts(layout):
    """The multi-query indexer (queries of the sequence in groups of two per workgroup, a ragged last
    group of one) in every addressing mode: every row's scores bit for bit against the oracle over its
    causal keys (-inf after), and every row's selection."""
    S, pb, k = 67, 130, 64
    T = pb + S
    rng = np.random.default_rng(790 + len(layout))
    tiled = layout.endswith("tiled")
    if layout.startswith("paged"):
        bs = 64 if layout.startswith("paged64") else 16
        nblk = (T + bs - 1) // bs + 2
        perm = rng.permutation(nblk).astype(np.int32)
        bt = perm[None, : (T + bs - 1) // bs].copy()
        ic_pool = rng.standard_normal((nblk * bs, 128)).astype(np.float32)
        t = np.arange(T)
        ic = ic_pool[bt[0, t // bs].astype(np.int64) * bs + t % bs]
        pool = synth.tile_index_keys(ic_pool) if tiled else ic_pool
        z = np.zeros((nblk * bs, 8), np.uint16)
        kv = mla.KvCache(dev_bf16(z), dev_bf16(z), dev(pool), max_seq_len=T, block_table=dev(bt), block_size=bs,
                         ic_layout=mla.MLA_IC_TILE64 if tiled else mla.MLA_IC_ROWS)
    else:
        Tp = (T + 63) // 64 * 64
        ic = rng.standard_normal((Tp, 128)).astype(np.float32)
        z = np.zeros((Tp, 8), np.uint16)
        kv = mla.KvCache(dev_bf16(z), dev_bf16(z), dev(synth.tile_index_keys(ic) if tiled else ic), max_seq_len=T,
                         seq_stride=Tp, ic_layout=mla.MLA_IC_TILE64 if tiled else mla.MLA_IC_ROWS)
    qi = rng.standard_normal((S, 32, 128)).astype(np.float32)
    wi = rng.standard_normal((S, 32)).astype(np.float32)
    log(f"prefill select every row layout={layout}")
    sc, sel, nsel = (host(x) for x in mla.dsa_prefill_select(dev(qi), dev(wi), kv, pb, k))
    for i in range(S):
        n = pb + i + 1
        ref = oracle.index_scores(qi[i], wi[i], ic[:n])
        assert np.array_equal(sc[i, :n].view(np.uint32), ref.view(np.uint32)), i
        assert np.all(np.isneginf(sc[i, n:])), i
        rs, rn = oracle.topk(ref, n, k)
        assert int(nsel[i]) == rn and np.array_equal(sel[i], rs), i


def test_dsa_prefill_full_4096():
    """DSA in prefill at S = T = 4096, k = 2048: per-query selection, then sparse attention on both
    paths; 64 evenly spaced rows on all heads against the oracle over each row's selected keys."""
    S, k = 4096, 2048
    p = synth.prefill(4, S, 0)
    ic, qi, wi = _ic_case(770, S, S=S)
    sm = 1.0 / math.sqrt(p.nope + p.rope)
    kv = mla.KvCache(dev_bf16(p.lc), dev_bf16(p.rc), dev(ic), max_seq_len=S, seq_stride=S)
    log("DSA prefill S=T=4096: select")
    _, sel, nsel = mla.dsa_prefill_select(dev(qi), dev(wi), kv, 0, k)
    sel_h, nsel_h = host(sel), host(nsel)
    rows = np.unique(np.linspace(0, S - 1, 64).round().astype(int))
    for i in rows[::8]:   # the selection itself, spot-checked
        rs, rn = oracle.topk(oracle.index_scores(qi[i], wi[i], ic[: i + 1]), i + 1, k)
        assert int(nsel_h[i]) == rn and np.array_equal(sel_h[i], rs), i
    ref = _ref_rows(p, rows, lambda i: sel_h[i, : nsel_h[i]], sm)
    q, kvb = dev_bf16(p.q), dev_bf16(p.kv_b)
    for g in (0, 1):
        log(f"DSA prefill S=T=4096: attention g_absorb={g}")
        out = host(mla.mla_attention(q, kvb, kv, p.nope, 0, sm, g_absorb=g, sel=sel, nsel=nsel))
        assert rel_err(out[rows], ref) <= TOL_BF16, g
