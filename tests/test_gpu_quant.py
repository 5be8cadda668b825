"""GPU parity of the absorbed decode with a quantized kv_b (FP8 E4M3, INT8, MXFP4).

Pages: chen3feng, "colibri-analysis 06: MLA attention and KV cache", sec. 2.3 (the absorbed path reads
kv_b through qt_addrow / qt_matvec_rows over quantized rows) and aiknowledge.cn, "Ch.7 sec. 03 ...",
sec. 3 and 5 (int8 / FP8 / MXFP4 weights, each format gated by a correctness check).  The reference
is the oracle's absorbed decode with kv_b = the oracle's own decoding of the same codes and scales
(rounded to fp32 to enter the attention oracle: at most 2^-24 relative per weight); bar 1e-2 (bf16
queries and cache).  The selection of the quantized step equals the bf16 step's bit for bit.
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

TOL_BF16 = 1e-2
FMTS = [mla.MLA_Q_FP8_E4M3, mla.MLA_Q_INT8, mla.MLA_Q_MXFP4]
cv = synth.bf16_bits_to_f32


def _ref(d, b, keys, kvb, sm, T):
    return oracle.absorbed_decode(cv(d.q_nope[b]), cv(d.q_rope[b]), kvb, cv(d.lc[b * T:(b + 1) * T]),
                                  cv(d.rc[b * T:(b + 1) * T]), keys, d.v, sm)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("B", [1, 2, 5, 33])
def test_quantized_decode_dense_and_selected(fmt, B):
    """B = 1: the absorption job and combine_one decoding W_UV into LDS; B = 2: the split reduction
    and unabsorb_quant; B = 5: the all-heads decode core; B = 33: the stand-alone absorb_q_quant."""
    T = 1500
    d = synth.decode(800 + B, T, B=B)
    N = d.H * (d.nope + d.v)
    codes, scales = synth.quantized_kv_b(810 + fmt, fmt, N, d.L)
    kvb = oracle.dequant_rows(codes, scales, fmt, d.L).astype(np.float32)
    sm = 1.0 / math.sqrt(d.nope + d.rope)
    seq_len = [T - (211 * b) % 1400 for b in range(B)]
    kv = mla.KvCache(dev_bf16(d.lc), dev_bf16(d.rc), seq_len=dev(np.asarray(seq_len, np.int32)), max_seq_len=T,
                     seq_stride=T)
    qn, qr, c_d, s_d = dev_bf16(d.q_nope), dev_bf16(d.q_rope), dev(codes), dev(scales)
    log(f"quantized decode fmt={fmt} B={B} dense")
    out = host(mla.mla_absorbed_decode_q(qn, qr, c_d, s_d, fmt, kv, sm))
    for b in range(B):
        assert rel_err(out[b], _ref(d, b, np.arange(seq_len[b]), kvb, sm, T)) <= TOL_BF16, b
    rng = np.random.default_rng(820 + B)
    k = 512
    sel = np.full((B, k), -1, np.int32)
    nsel = np.zeros(B, np.int32)
    for b in range(B):
        n = min(k, seq_len[b]) if b != 1 else 7
        sel[b, :n] = np.sort(rng.choice(seq_len[b], n, replace=False))
        nsel[b] = n
    log(f"quantized decode fmt={fmt} B={B} selected")
    out = host(mla.mla_absorbed_decode_q(qn, qr, c_d, s_d, fmt, kv, sm, sel=dev(sel), nsel=dev(nsel)))
    for b in range(B):
        assert rel_err(out[b], _ref(d, b, sel[b, : nsel[b]], kvb, sm, T)) <= TOL_BF16, b


@pytest.mark.parametrize("fmt", FMTS)
def test_quantized_dsa_step_full_context(fmt):
    """The whole decode step at T = 131072 with a quantized kv_b: the selection equals the bf16 step's
    bit for bit and the output matches the oracle over the selected keys with the decoded weights."""
    T, k = 131072, 2048
    d = synth.decode(3, T, dsa=True)
    N = d.H * (d.nope + d.v)
    codes, scales = synth.quantized_kv_b(830 + fmt, fmt, N, d.L)
    kvb = oracle.dequant_rows(codes, scales, fmt, d.L).astype(np.float32)
    sm = 1.0 / math.sqrt(d.nope + d.rope)
    kv = mla.KvCache(dev_bf16(d.lc), dev_bf16(d.rc), dev(d.ic), seq_len=dev(np.array([T], np.int32)), max_seq_len=T,
                     seq_stride=T)
    args = (dev_bf16(d.q_nope), dev_bf16(d.q_rope), dev(d.q_idx), dev(d.w_idx))
    log(f"quantized DSA step T=131072 fmt={fmt}")
    out, sc, sel, nsel = (host(x) for x in mla.mla_dsa_decode_q(*args, dev(codes), dev(scales), fmt, kv, T, k, sm))
    _, sc_b, sel_b, nsel_b = (host(x) for x in mla.mla_dsa_decode(*args, dev_bf16(d.kv_b), kv, T, k, sm))
    assert np.array_equal(sc.view(np.uint32), sc_b.view(np.uint32))
    assert np.array_equal(sel, sel_b) and np.array_equal(nsel, nsel_b)
    q_rot = oracle.rope_interleave(cv(d.q_rope[0])[None], np.array([T - 1]), 0, d.rope)[0]
    ref = oracle.absorbed_decode(cv(d.q_nope[0]), q_rot, kvb, cv(d.lc), cv(d.rc), sel[0, : nsel[0]], d.v, sm)
    assert rel_err(out[0], ref) <= TOL_BF16


@pytest.mark.parametrize("fmt", FMTS)
def test_quantized_dsa_step_batch(fmt):
    """The quantized step over three sequences of different lengths (the absorption runs beside the
    selection's resolve workgroups for every row): selection equal to the bf16 step's, output against
    the oracle per row."""
    B, T, k = 3, 6000, 2048
    d = synth.decode(31, T, B=B, dsa=True)
    N = d.H * (d.nope + d.v)
    codes, scales = synth.quantized_kv_b(840 + fmt, fmt, N, d.L)
    kvb = oracle.dequant_rows(codes, scales, fmt, d.L).astype(np.float32)
    sm = 1.0 / math.sqrt(d.nope + d.rope)
    seq_len = np.array([T, 2500, 1300], np.int32)
    kv = mla.KvCache(dev_bf16(d.lc), dev_bf16(d.rc), dev(d.ic), seq_len=dev(seq_len), max_seq_len=T, seq_stride=T)
    args = (dev_bf16(d.q_nope), dev_bf16(d.q_rope), dev(d.q_idx), dev(d.w_idx))
    log(f"quantized DSA step B=3 fmt={fmt}")
    out, sc, sel, nsel = (host(x) for x in mla.mla_dsa_decode_q(*args, dev(codes), dev(scales), fmt, kv, T, k, sm))
    _, sc_b, sel_b, nsel_b = (host(x) for x in mla.mla_dsa_decode(*args, dev_bf16(d.kv_b), kv, T, k, sm))
    assert np.array_equal(sel, sel_b) and np.array_equal(nsel, nsel_b)
    for b in range(B):
        L = int(seq_len[b])
        q_rot = oracle.rope_interleave(cv(d.q_rope[b])[None], np.array([L - 1]), 0, d.rope)[0]
        ref = oracle.absorbed_decode(cv(d.q_nope[b]), q_rot, kvb, cv(d.lc[b * T:(b + 1) * T]),
                                     cv(d.rc[b * T:(b + 1) * T]), sel[b, : nsel[b]], d.v, sm)
        assert rel_err(out[b], ref) <= TOL_BF16, b
