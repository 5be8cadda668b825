"""GPU parity of the cache-write side and of the DSA-shared layer.

Pages: chen3feng, "colibri-analysis 06: MLA attention and KV cache", sec. 2.1 (KV path: RMSNorm of the
kv_a latent into Lc, RoPE of the shared key into Rc) and sec. 2.2 (indexer key: LayerNorm + RoPE into
Ic; shared layers reuse the full layer's selection).  Bars: written rows against the oracle's float64
rows within one bf16 ulp plus 2e-6 of the row scale (bf16 pools) or 2e-6 / 2e-5 relative (fp32 Lc, Rc / Ic); rows the call does not
address stay bit-identical; the rotated key equals mla_rope_interleave bit for bit; attention outputs
within 2e-3 (fp32) / 1e-2 (bf16) of the oracle.
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


def _to_dev(a, bf16):
    return dev_bf16(synth.to_bf16_bits(a)) if bf16 else dev(np.ascontiguousarray(a, np.float32))


def _in_vals(a, bf16):
    """The values the kernel sees for an input array (bf16-rounded when the input dtype is bf16)."""
    return synth.bf16_bits_to_f32(synth.to_bf16_bits(a)) if bf16 else np.asarray(a, np.float32)


@pytest.mark.parametrize("in_bf16,kv_bf16,tiled,per", [(False, False, False, 100), (False, True, True, 100),
                                                       (True, True, False, 100), (True, False, True, 100),
                                                       (True, True, True, 97)])
def test_cache_write_paged_rows_against_oracle(in_bf16, kv_bf16, tiled, per):
    """per: tokens per sequence (97: a token count that leaves the last workgroup part-filled)."""
    rng = np.random.default_rng(600 + 2 * in_bf16 + kv_bf16 + per)
    B, L, rope, hd = 3, 512, 64, 128
    bs = 64 if tiled else 16                        # a tiled indexer pool holds whole 64-row tiles per block
    max_blocks = 512 // bs
    n_blocks = B * max_blocks
    rows = n_blocks * bs
    perm = rng.permutation(n_blocks).astype(np.int32)
    bt = perm.reshape(B, max_blocks).copy()
    bt[1, 5] = -1                                   # a hole: tokens there are not written
    seq = np.repeat(np.arange(B, dtype=np.int32), per)
    allowed = [np.arange(max_blocks * bs)] * B
    allowed[1] = np.setdiff1d(allowed[1], np.arange(5 * bs, 6 * bs))
    pos = np.concatenate([np.sort(rng.choice(a, per, replace=False)) for a in allowed]).astype(np.int32)
    pos[150] = 5 * bs + 3                          # lands in the hole of sequence 1
    n = seq.size
    comp = (rng.standard_normal((n, L + rope)) * 2.0 + 0.3).astype(np.float32)
    ik = (rng.standard_normal((n, hd)) * 1.5 - 0.7).astype(np.float32)
    gain = rng.uniform(0.5, 1.5, L).astype(np.float32)
    gm, bt_ = rng.uniform(0.5, 1.5, hd).astype(np.float32), (rng.standard_normal(hd) * 0.1).astype(np.float32)
    ix_off, ix_rd = hd - 64, 64
    # sentinel pools
    kdt = torch.bfloat16 if kv_bf16 else torch.float32
    lc = torch.full((rows, L), 7.0, dtype=kdt, device="cuda")
    rc = torch.full((rows, rope), 7.0, dtype=kdt, device="cuda")
    ic = torch.full((rows, hd), 7.0, dtype=torch.float32, device="cuda")
    kv = mla.KvCache(lc, rc, ic, max_seq_len=max_blocks * bs, block_table=dev(bt), block_size=bs,
                     ic_layout=mla.MLA_IC_TILE64 if tiled else mla.MLA_IC_ROWS)
    log(f"cache write in_bf16={in_bf16} kv_bf16={kv_bf16} tiled={tiled} per={per}")
    mla.mla_cache_write(_to_dev(comp, in_bf16), dev(seq), dev(pos), kv, B, ik=_to_dev(ik, in_bf16), kv_gain=dev(gain),
                        ix_gamma=dev(gm), ix_beta=dev(bt_), ix_rope_off=ix_off, ix_rope_dim=ix_rd)
    r_lc, r_rc, r_ic = oracle.cache_write(_in_vals(comp, in_bf16), _in_vals(ik, in_bf16), seq, pos, L, rope, rows=rows,
                                          kv_gain=gain, gamma=gm, beta=bt_, ix_off=ix_off, ix_rdim=ix_rd,
                                          block_table=bt, block_size=bs)
    g_lc, g_rc = host(lc), host(rc)
    g_ic = host(ic)
    if tiled:   # back to rows: element d of row r sits in the 64-row tile of r
        g_ic = g_ic.reshape(rows // 64, hd // 4, 64, 4).transpose(0, 2, 1, 3).reshape(rows, hd)
    written = ~np.isnan(r_lc[:, 0])
    assert written.sum() == n - 1
    assert np.all(g_lc[~written] == 7.0) and np.all(g_rc[~written] == 7.0) and np.all(g_ic[~written] == 7.0)
    for g, r in ((g_lc, r_lc), (g_rc, r_rc)):
        g, r = g[written], r[written]
        if kv_bf16:   # one bf16 rounding of the fp32 result (whose own error is ~1e-7 of the inputs)
            assert np.all(np.abs(g - r) <= 2.0 ** -8 * np.abs(r) + 2e-6 * np.abs(r).max())
        else:
            assert np.abs(g - r).max() <= 2e-6 * np.abs(r).max()
    assert np.abs(g_ic[written] - r_ic[written]).max() <= 2e-5 * np.abs(r_ic[written]).max()
    if in_bf16 == kv_bf16:   # the rotated key equals mla_rope_interleave on the same tail, bit for bit
        tail = _to_dev(comp[:, L:], in_bf16).reshape(n, 1, rope).contiguous()
        mla.mla_rope_interleave(tail, dev(pos), 0, rope)
        rows_w = (bt[seq, pos // bs].astype(np.int64) * bs + pos % bs)
        ok = bt[seq, pos // bs] >= 0
        a = host(tail).reshape(n, rope)[ok]
        b = g_rc[rows_w[ok]]
        assert np.array_equal(a.view(np.uint32) if not kv_bf16 else a, b.view(np.uint32) if not kv_bf16 else b)


@pytest.mark.parametrize("ix_off,ix_rd,with_ik,in_bf16", [(0, 64, True, True), (0, 128, True, False),
                                                           (32, 96, True, True), (0, 0, False, True)])
def test_cache_write_rotated_slice_placements(ix_off, ix_rd, with_ik, in_bf16):
    """The 512/64/128 geometry with the indexer's rotated slice in the lower half of the key (its
    pairs then share lanes with the Rc pairs), over the whole key, straddling the middle, and
    without an indexer key; contiguous pools, bf16 latent and rope rows, fp32 indexer rows."""
    rng = np.random.default_rng(640 + ix_off + ix_rd + with_ik)
    L, rope, hd, rows = 512, 64, 128, 300
    n = 257
    seq = np.zeros(n, np.int32)
    pos = np.sort(rng.choice(rows, n, replace=False)).astype(np.int32)
    comp = (rng.standard_normal((n, L + rope)) * 1.5 - 0.2).astype(np.float32)
    ik = (rng.standard_normal((n, hd)) * 0.8 + 0.4).astype(np.float32) if with_ik else None
    gain = rng.uniform(0.5, 1.5, L).astype(np.float32)
    lc = torch.full((rows, L), 7.0, dtype=torch.bfloat16, device="cuda")
    rc = torch.full((rows, rope), 7.0, dtype=torch.bfloat16, device="cuda")
    ic = torch.full((rows, hd), 7.0, dtype=torch.float32, device="cuda") if with_ik else None
    kv = mla.KvCache(lc, rc, ic, max_seq_len=rows, seq_stride=rows)
    log(f"cache write slice off={ix_off} dim={ix_rd} ik={with_ik} in_bf16={in_bf16}")
    mla.mla_cache_write(_to_dev(comp, in_bf16), dev(seq), dev(pos), kv, 1,
                        ik=_to_dev(ik, in_bf16) if with_ik else None, kv_gain=dev(gain), ix_rope_off=ix_off,
                        ix_rope_dim=ix_rd, theta=500000.0)
    r_lc, r_rc, r_ic = oracle.cache_write(_in_vals(comp, in_bf16), _in_vals(ik, in_bf16) if with_ik else None, seq,
                                          pos, L, rope, rows=rows, kv_gain=gain, ix_off=ix_off, ix_rdim=ix_rd,
                                          theta=500000.0, seq_stride=rows)
    written = np.zeros(rows, bool)
    written[pos] = True
    g_lc, g_rc = host(lc), host(rc)
    assert np.all(g_lc[~written] == 7.0) and np.all(g_rc[~written] == 7.0)
    for g, r in ((g_lc, r_lc), (g_rc, r_rc)):
        g, r = g[written], r[written]
        assert np.all(np.abs(g - r) <= 2.0 ** -8 * np.abs(r) + 2e-6 * np.abs(r).max())
    if with_ik:
        g_ic = host(ic)
        assert np.all(g_ic[~written] == 7.0)
        assert np.abs(g_ic[written] - r_ic[written]).max() <= 2e-5 * np.abs(r_ic[written]).max()


def test_tiny_layer_cache_written_on_gpu():
    """The tiny fp32 layer end to end with the GPU filling the cache: the kv_a outputs (plain float64
    matmuls rounded to fp32) go through mla_cache_write (RMSNorm eps 1e-6, unit gain, RoPE at
    positions 0..T-1), the query tail through mla_rope_interleave at T-1; the absorbed decode then
    matches the oracle's tiny layer."""
    t = synth.tiny_layer(1)
    lc, rc, q = oracle.tiny_layer(t.x, t.q_a, t.q_b, t.kv_a, t.H, t.nope, t.rope, t.L)
    sm = 1.0 / math.sqrt(t.nope + t.rope)
    ref = oracle.absorbed_decode(q[:, : t.nope].astype(np.float32), q[:, t.nope:].astype(np.float32), t.kv_b,
                                 lc.astype(np.float32), rc.astype(np.float32), np.arange(t.T), t.v, sm)
    comp = (t.x.astype(np.float64) @ t.kv_a.astype(np.float64).T).astype(np.float32)
    qa = t.q_a.astype(np.float64) @ t.x[-1].astype(np.float64)
    qa = qa / np.sqrt((qa ** 2).mean() + 1e-6)
    qf = (t.q_b.astype(np.float64) @ qa).reshape(t.H, t.nope + t.rope).astype(np.float32)
    log("tiny layer: cache written on the GPU")
    lc_d = torch.zeros((t.T, t.L), dtype=torch.float32, device="cuda")
    rc_d = torch.zeros((t.T, t.rope), dtype=torch.float32, device="cuda")
    kv = mla.KvCache(lc_d, rc_d, max_seq_len=t.T, seq_stride=t.T, seq_len=dev(np.array([t.T], np.int32)))
    mla.mla_cache_write(dev(comp), dev(np.zeros(t.T, np.int32)), dev(np.arange(t.T, dtype=np.int32)), kv, 1)
    assert np.abs(host(lc_d) - lc).max() <= 2e-6 * np.abs(lc).max()
    assert np.abs(host(rc_d) - rc).max() <= 2e-6 * np.abs(rc).max()
    q_d = dev(qf[None])
    mla.mla_rope_interleave(q_d, dev(np.array([t.T - 1], np.int32)), t.nope, t.rope)
    qh = q_d[0]
    out = host(mla.mla_absorbed_decode(qh[None, :, : t.nope].contiguous(), qh[None, :, t.nope:].contiguous(),
                                       dev(t.kv_b), kv, sm))[0]
    assert rel_err(out, ref) <= TOL_F32


def test_shared_layer_reuses_the_full_layers_selection():
    """A full DSA layer selects keys (mla_dsa_decode); a shared layer with its own cache, queries and
    kv_b reuses that selection: mla_dsa_decode_shared equals RoPE + mla_absorbed_decode over the same
    keys bit for bit, and the oracle's absorbed decode of the shared layer over those keys."""
    B, T, k = 2, 5000, 512
    seq_len = [T, 3001]
    full = synth.decode(610, T, B=B, dsa=True)
    shared = synth.decode(611, T, B=B)
    sm = 1.0 / math.sqrt(full.nope + full.rope)
    sl = dev(np.asarray(seq_len, np.int32))
    kv_full = mla.KvCache(dev_bf16(full.lc), dev_bf16(full.rc), dev(full.ic), seq_len=sl, max_seq_len=T, seq_stride=T)
    log("full layer: mla_dsa_decode")
    _, _, sel, nsel = mla.mla_dsa_decode(dev_bf16(full.q_nope), dev_bf16(full.q_rope), dev(full.q_idx),
                                         dev(full.w_idx), dev_bf16(full.kv_b), kv_full, T, k, sm)
    kv_sh = mla.KvCache(dev_bf16(shared.lc), dev_bf16(shared.rc), seq_len=sl, max_seq_len=T, seq_stride=T)
    log("shared layer: mla_dsa_decode_shared")
    qn, qr, kvb = dev_bf16(shared.q_nope), dev_bf16(shared.q_rope), dev_bf16(shared.kv_b)
    out = host(mla.mla_dsa_decode_shared(qn, qr, kvb, kv_sh, sel, nsel, sm))
    qr_rot = qr.clone()
    mla.mla_rope_interleave(qr_rot, dev(np.asarray(seq_len, np.int32) - 1), 0, shared.rope)
    ref_gpu = host(mla.mla_absorbed_decode(qn, qr_rot, kvb, kv_sh, sm, sel=sel, nsel=nsel))
    assert np.array_equal(out.view(np.uint32), ref_gpu.view(np.uint32))
    s_h, n_h = host(sel), host(nsel)
    cv = synth.bf16_bits_to_f32
    for b in range(B):
        keys = s_h[b, : n_h[b]]
        q_rot = oracle.rope_interleave(cv(shared.q_rope[b])[None], np.array([seq_len[b] - 1]), 0, shared.rope)[0]
        ref = oracle.absorbed_decode(cv(shared.q_nope[b]), q_rot, cv(shared.kv_b), cv(shared.lc[b * T:(b + 1) * T]),
                                     cv(shared.rc[b * T:(b + 1) * T]), keys, shared.v, sm)
        assert rel_err(out[b], ref) <= TOL_BF16, b
