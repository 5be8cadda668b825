"""Pins for the CPU oracle: each oracle function is checked against something other than
itself -- worked examples fixed by hand (tests/golden), closed forms, invariants the pages
state (absorbed == non-absorbed, keep-all selection == dense), brute force on tiny inputs,
error bounds, and library routines (numpy sort, torch's scaled-dot-product attention).

Pages: chen3feng, "colibri-analysis 06: MLA attention and KV cache" (sec. 1, 2, 2.1, 2.2,
2.3); aiknowledge.cn, "Ch.7 sec. 03: token-exact forward validation and faithful DSA".
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _closed(v):
    if isinstance(v, str):
        return float(eval(v, {"__builtins__": {}}, {"cos": math.cos, "sin": math.sin}))
    return float(v)


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ----------------------------------------------------------------------------- sizes
def test_state_size_arithmetic_matches_pages():
    g = _golden("mla_state_sizes.json")
    naive = g["n_heads"] * (g["k_head"] + g["v_head"])
    mla = g["kv_lora"] + g["qk_rope"]
    assert naive == g["naive_floats_per_token"]
    assert mla == g["mla_floats_per_token"]
    assert round(naive / mla) == g["ratio_rounded"]


# ----------------------------------------------------------------------------- RoPE
def test_rope_worked_examples(oracle):
    g = _golden("rope_worked_examples.json")
    for c in g["cases"]:
        x = np.array(c["x"], np.float64).reshape(1, 1, -1)
        y = oracle.rope_interleave(x, [c["pos"]], 0, c["rope_dim"], c["theta"]).reshape(-1)
        exp = np.array([_closed(v) for v in c["expected"]])
        assert np.max(np.abs(y - exp)) <= 1e-15, c["name"]


def test_rope_position_zero_is_exact_deinterleave_and_nope_untouched(oracle):
    rng = np.random.default_rng(10)
    nope, rope = 16, 8
    x = rng.standard_normal((5, 3, nope + rope))
    y = oracle.rope_interleave(x, np.zeros(5, np.int32), nope, rope)
    assert np.array_equal(y[..., :nope], x[..., :nope])
    assert np.array_equal(y[..., nope: nope + rope // 2], x[..., nope::2])
    assert np.array_equal(y[..., nope + rope // 2:], x[..., nope + 1::2])
    # at other positions the nope dims are still bit-identical
    y2 = oracle.rope_interleave(x, rng.integers(0, 1 << 17, 5).astype(np.int32), nope, rope)
    assert np.array_equal(y2[..., :nope], x[..., :nope])


def test_rope_preserves_pair_norms(oracle):
    rng = np.random.default_rng(11)
    rope = 64
    x = rng.standard_normal((7, 2, rope))
    pos = rng.integers(0, 131072, 7).astype(np.int32)
    y = oracle.rope_interleave(x, pos, 0, rope)
    h = rope // 2
    n_in = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    n_out = y[..., :h] ** 2 + y[..., h:] ** 2
    assert np.max(np.abs(n_in - n_out)) <= 1e-12 * np.max(n_in)


def test_rope_dot_depends_only_on_relative_position(oracle):
    rng = np.random.default_rng(12)
    rope = 64
    q = rng.standard_normal((1, 1, rope))
    k = rng.standard_normal((1, 1, rope))
    for m, n in [(5, 3), (1000, 17), (131071, 129000), (40, 40)]:
        a = np.dot(oracle.rope_interleave(q, [m], 0, rope).ravel(), oracle.rope_interleave(k, [n], 0, rope).ravel())
        b = np.dot(oracle.rope_interleave(q, [m - n], 0, rope).ravel(), oracle.rope_interleave(k, [0], 0, rope).ravel())
        assert abs(a - b) <= 1e-9 * (np.linalg.norm(q) * np.linalg.norm(k))


# ----------------------------------------------------------------------------- indexer
def test_indexer_fixed_order_worked_examples(oracle):
    g = _golden("indexer_fixed_order.json")
    for c in g["cases"]:
        s = oracle.index_scores(np.array(c["q"]), np.array(c["w"]), np.array(c["ic"]))
        assert s.astype(np.float64).tolist() == c["expected"], c["name"]


def test_indexer_integer_inputs_are_exact(oracle):
    # small integers: every partial sum is exact in fp32, so any correct evaluation
    # equals exact integer arithmetic
    rng = np.random.default_rng(20)
    n_ih, hd, T = 5, 7, 300
    q = rng.integers(-3, 4, (n_ih, hd))
    w = rng.integers(-2, 3, n_ih)
    ic = rng.integers(-3, 4, (T, hd))
    dots = ic @ q.T                                   # [T, n_ih] exact int64
    exact = (np.maximum(dots, 0) * w).sum(axis=1)
    got = oracle.index_scores(q, w, ic)
    assert np.array_equal(got.astype(np.int64), exact)


def test_indexer_one_hot_keys_closed_form(oracle):
    rng = np.random.default_rng(21)
    n_ih, hd, T = 32, 128, 256
    q = rng.standard_normal((n_ih, hd)).astype(np.float32)
    w = rng.standard_normal(n_ih).astype(np.float32)
    d_of_t = rng.integers(0, hd, T)
    ic = np.zeros((T, hd), np.float32)
    ic[np.arange(T), d_of_t] = 1.0
    got = oracle.index_scores(q, w, ic).astype(np.float64)
    ref = (w.astype(np.float64)[None, :] * np.maximum(q.T[d_of_t].astype(np.float64), 0)).sum(1)
    bound = n_ih * 2.0 ** -24 * (np.abs(w)[None, :] * np.abs(q.T[d_of_t])).sum(1) * 1.01
    assert np.all(np.abs(got - ref) <= bound + 1e-30)


def test_indexer_one_hot_weight_is_relu_dot(oracle):
    rng = np.random.default_rng(22)
    n_ih, hd, T = 8, 128, 200
    q = rng.standard_normal((n_ih, hd)).astype(np.float32)
    ic = rng.standard_normal((T, hd)).astype(np.float32)
    for h in (0, 5):
        w = np.zeros(n_ih, np.float32)
        w[h] = 1.0
        got = oracle.index_scores(q, w, ic).astype(np.float64)
        ref = np.maximum(ic.astype(np.float64) @ q[h].astype(np.float64), 0)
        gam = hd * 2.0 ** -24 / (1 - hd * 2.0 ** -24)
        bound = gam * (np.abs(ic) @ np.abs(q[h])).astype(np.float64)
        assert np.all(np.abs(got - ref) <= bound)


def test_indexer_fp32_within_forward_error_bound(oracle):
    rng = np.random.default_rng(23)
    n_ih, hd, T = 32, 128, 1024
    q = rng.standard_normal((n_ih, hd)).astype(np.float32)
    w = rng.standard_normal(n_ih).astype(np.float32)
    ic = rng.standard_normal((T, hd)).astype(np.float32)
    s32 = oracle.index_scores(q, w, ic).astype(np.float64)
    s64 = oracle.index_scores_f64(q, w, ic)
    # the fp64 path itself agrees with a library product
    lib = (np.maximum(ic.astype(np.float64) @ q.T.astype(np.float64), 0) @ w.astype(np.float64))
    assert _rel(s64, lib) <= 1e-12
    n = hd + n_ih
    u = 2.0 ** -24
    gam = n * u / (1 - n * u)
    mag = (np.abs(ic).astype(np.float64) @ np.abs(q.T).astype(np.float64)) @ np.abs(w).astype(np.float64)
    assert np.all(np.abs(s32 - s64) <= gam * mag)


def test_indexer_power_of_two_homogeneity_is_bit_exact(oracle):
    rng = np.random.default_rng(24)
    q = rng.standard_normal((32, 128)).astype(np.float32)
    w = rng.standard_normal(32).astype(np.float32)
    ic = rng.standard_normal((300, 128)).astype(np.float32)
    base = oracle.index_scores(q, w, ic)
    assert np.array_equal(oracle.index_scores(q, 2 * w, ic), 2 * base)
    assert np.array_equal(oracle.index_scores(4 * q, w / 4, ic), base)


# ----------------------------------------------------------------------------- top-k
def test_topk_worked_examples(oracle):
    g = _golden("topk_worked_examples.json")
    for c in g["cases"]:
        sel, nsel = oracle.topk(np.array(c["scores"], np.float32), c["n_valid"], c["k"])
        assert nsel == c["nsel"], c["name"]
        assert sel[:nsel].tolist() == c["sel"], c["name"]
        assert np.all(sel[nsel:] == -1)


def _rank_select(s, n_valid, k):
    """Brute force by counting: key t is kept iff fewer than k keys precede it in the
    order (higher score, or equal score at a lower position)."""
    out = []
    for t in range(n_valid):
        better = sum(1 for u in range(n_valid) if s[u] > s[t] or (s[u] == s[t] and u < t))
        if better < k:
            out.append(t)
    return out


def test_topk_exhaustive_brute_force(oracle):
    for T in range(1, 8):
        pats = np.array(list(itertools.product([0.0, 1.0, 2.0], repeat=T)), np.float32)
        for n_valid in {T, max(T - 2, 0)}:
            for k in range(1, T + 2):
                sel, nsel = oracle.topk_batch(pats, np.full(len(pats), n_valid, np.int32), k)
                for i, s in enumerate(pats):
                    ref = _rank_select(s, n_valid, k)
                    assert nsel[i] == len(ref)
                    assert sel[i, : nsel[i]].tolist() == ref


def test_topk_large_random_matches_library_sort(oracle):
    rng = np.random.default_rng(30)
    T, k = 131072, 2048
    s = np.round(rng.standard_normal(T) * 8).astype(np.float32) / 8   # many ties
    s[rng.integers(0, T, 50)] = -0.0
    for n_valid in (T, 100000, 2048, 1500):
        sel, nsel = oracle.topk(s, n_valid, k)
        order = np.lexsort((np.arange(n_valid), -s[:n_valid].astype(np.float64)))
        ref = np.sort(order[: min(k, n_valid)])
        assert nsel == ref.size
        assert np.array_equal(sel[:nsel], ref)


# ----------------------------------------------------------------------------- decode
def _rand_decode(seed, H=4, nope=16, rope=8, v=16, L=32, T=50, wstd=0.3):
    rng = np.random.default_rng(seed)
    return dict(
        q_nope=rng.standard_normal((H, nope)).astype(np.float32),
        q_rope=rng.standard_normal((H, rope)).astype(np.float32),
        kv_b=(rng.standard_normal((H * (nope + v), L)) * wstd).astype(np.float32),
        lc=rng.standard_normal((T, L)).astype(np.float32),
        rc=rng.standard_normal((T, rope)).astype(np.float32),
    ), (H, nope, rope, v, L, T)


@pytest.mark.parametrize("dims", [(4, 16, 8, 16, 32, 50), (8, 24, 16, 20, 40, 130)])
def test_absorbed_equals_nonabsorbed(oracle, dims):
    H, nope, rope, v, L, T = dims
    a, _ = _rand_decode(40, H, nope, rope, v, L, T)
    keys = np.arange(T)
    sc = 1 / math.sqrt(nope + rope)
    o1 = oracle.absorbed_decode(a["q_nope"], a["q_rope"], a["kv_b"], a["lc"], a["rc"], keys, v, sc)
    o2 = oracle.nonabsorbed_decode(a["q_nope"], a["q_rope"], a["kv_b"], a["lc"], a["rc"], keys, v, sc)
    assert _rel(o1, o2) <= 1e-10


def test_decode_matches_torch_sdpa(oracle):
    import torch
    a, (H, nope, rope, v, L, T) = _rand_decode(41, 6, 12, 8, 10, 24, 77)
    keys = np.random.default_rng(1).permutation(T)[:40]
    sc = 0.37
    got = oracle.absorbed_decode(a["q_nope"], a["q_rope"], a["kv_b"], a["lc"], a["rc"], keys, v, sc)
    kvb = torch.from_numpy(a["kv_b"].astype(np.float64)).view(H, nope + v, L)
    lc = torch.from_numpy(a["lc"].astype(np.float64))[keys]
    rc = torch.from_numpy(a["rc"].astype(np.float64))[keys]
    k_nope = torch.einsum("hic,tc->hti", kvb[:, :nope], lc)
    vv = torch.einsum("hjc,tc->htj", kvb[:, nope:], lc)
    k = torch.cat([k_nope, rc.unsqueeze(0).expand(H, -1, -1)], dim=-1)
    q = torch.cat([torch.from_numpy(a["q_nope"]).double(), torch.from_numpy(a["q_rope"]).double()], -1)
    ref = torch.nn.functional.scaled_dot_product_attention(q[:, None, :], k, vv, scale=sc)[:, 0]
    assert _rel(got, ref.numpy()) <= 1e-10


def test_decode_single_key_closed_form(oracle):
    a, (H, nope, rope, v, L, T) = _rand_decode(42)
    got = oracle.absorbed_decode(a["q_nope"], a["q_rope"], a["kv_b"], a["lc"], a["rc"], [17], v, 0.2)
    W = a["kv_b"].astype(np.float64).reshape(H, nope + v, L)
    ref = W[:, nope:] @ a["lc"][17].astype(np.float64)
    assert _rel(got, ref) <= 1e-12


def test_decode_zero_query_is_uniform_average(oracle):
    a, (H, nope, rope, v, L, T) = _rand_decode(43)
    z1 = np.zeros_like(a["q_nope"])
    z2 = np.zeros_like(a["q_rope"])
    keys = np.arange(3, 41)
    got = oracle.absorbed_decode(z1, z2, a["kv_b"], a["lc"], a["rc"], keys, v, 0.5)
    W = a["kv_b"].astype(np.float64).reshape(H, nope + v, L)
    ref = W[:, nope:] @ a["lc"][keys].astype(np.float64).mean(0)
    assert _rel(got, ref) <= 1e-12


def test_decode_dominant_key(oracle):
    a, (H, nope, rope, v, L, T) = _rand_decode(44)
    star = 29
    rc = a["rc"].astype(np.float64)
    gap = rc[star] @ rc[star] - np.max(np.delete(rc @ rc[star], star))
    assert gap > 0
    qr = np.tile(rc[star] * (80.0 / gap), (H, 1)).astype(np.float32)   # score margin >= ~80
    got = oracle.absorbed_decode(np.zeros_like(a["q_nope"]), qr, a["kv_b"], a["lc"], a["rc"], np.arange(T), v, 1.0)
    W = a["kv_b"].astype(np.float64).reshape(H, nope + v, L)
    ref = W[:, nope:] @ a["lc"][star].astype(np.float64)
    assert _rel(got, ref) <= 1e-9


def test_decode_key_order_and_keep_all(oracle):
    a, (H, nope, rope, v, L, T) = _rand_decode(45, T=90)
    dense = np.arange(T)
    perm = np.random.default_rng(2).permutation(T)
    o1 = oracle.absorbed_decode(a["q_nope"], a["q_rope"], a["kv_b"], a["lc"], a["rc"], dense, v, 0.25)
    o2 = oracle.absorbed_decode(a["q_nope"], a["q_rope"], a["kv_b"], a["lc"], a["rc"], perm, v, 0.25)
    assert _rel(o1, o2) <= 1e-13
    # a top-k that keeps every key selects exactly the dense key set
    sel, nsel = oracle.topk(np.random.default_rng(3).standard_normal(T).astype(np.float32), T, 4 * T)
    assert nsel == T and np.array_equal(sel[:nsel], dense)


# ----------------------------------------------------------------------------- prefill
def _rand_prefill(seed, S, pos_base, H=4, nope=16, rope=8, v=16, L=32):
    rng = np.random.default_rng(seed)
    T = pos_base + S
    return dict(q=rng.standard_normal((S, H, nope + rope)).astype(np.float32),
                kv_b=(rng.standard_normal((H * (nope + v), L)) * 0.3).astype(np.float32),
                lc=rng.standard_normal((T, L)).astype(np.float32),
                rc=rng.standard_normal((T, rope)).astype(np.float32)), (H, nope, rope, v, L, T)


def test_prefill_first_row_is_first_value(oracle):
    p, (H, nope, rope, v, L, T) = _rand_prefill(50, 9, 0)
    got = oracle.prefill_rows(p["q"], p["kv_b"], p["lc"], p["rc"], 0, nope, v, 0.3, [0])[0]
    W = p["kv_b"].astype(np.float64).reshape(H, nope + v, L)
    assert _rel(got, W[:, nope:] @ p["lc"][0].astype(np.float64)) <= 1e-12


def test_prefill_last_row_equals_decode(oracle):
    p, (H, nope, rope, v, L, T) = _rand_prefill(51, 1, 63)
    sc = 1 / math.sqrt(nope + rope)
    got = oracle.prefill_rows(p["q"], p["kv_b"], p["lc"], p["rc"], 63, nope, v, sc, [0])[0]
    ref = oracle.absorbed_decode(p["q"][0, :, :nope], p["q"][0, :, nope:], p["kv_b"], p["lc"], p["rc"],
                                 np.arange(T), v, sc)
    assert _rel(got, ref) <= 1e-10


def test_prefill_matches_torch_causal_sdpa(oracle):
    import torch
    S, pb = 20, 7
    p, (H, nope, rope, v, L, T) = _rand_prefill(52, S, pb, H=3, nope=10, rope=6, v=12, L=20)
    sc = 0.29
    got = oracle.prefill_rows(p["q"], p["kv_b"], p["lc"], p["rc"], pb, nope, v, sc, np.arange(S))
    kvb = torch.from_numpy(p["kv_b"].astype(np.float64)).view(H, nope + v, L)
    lc = torch.from_numpy(p["lc"].astype(np.float64))
    rc = torch.from_numpy(p["rc"].astype(np.float64))
    k = torch.cat([torch.einsum("hic,tc->hti", kvb[:, :nope], lc), rc.expand(H, -1, -1)], -1)
    vv = torch.einsum("hjc,tc->htj", kvb[:, nope:], lc)
    q = torch.from_numpy(p["q"].astype(np.float64)).permute(1, 0, 2)
    mask = torch.arange(T)[None, :] <= (pb + torch.arange(S))[:, None]
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, vv, attn_mask=mask, scale=sc)
    assert _rel(got, ref.permute(1, 0, 2).numpy()) <= 1e-10


# ----------------------------------------------------------------------------- tiny layer
def test_tiny_layer_pins(oracle):
    from mla_latent_kv_dsa_amd import synth
    t = synth.tiny_layer(1)
    lc, rc, q = oracle.tiny_layer(t.x, t.q_a, t.q_b, t.kv_a, t.H, t.nope, t.rope, t.L)
    # latent rows are RMS-normalised with unit gain: mean square = ms / (ms + eps)
    comp = t.x.astype(np.float64) @ t.kv_a.astype(np.float64).T
    ms = (comp[:, : t.L] ** 2).mean(1)
    assert np.max(np.abs((lc ** 2).mean(1) - ms / (ms + 1e-6))) <= 1e-12
    # the shared rope key is the rotated tail of the kv_a projection (pair norms kept)
    tail = comp[:, t.L:]
    n_in = tail[:, 0::2] ** 2 + tail[:, 1::2] ** 2
    n_out = rc[:, : t.rope // 2] ** 2 + rc[:, t.rope // 2:] ** 2
    assert np.max(np.abs(n_in - n_out)) <= 1e-12 * n_in.max()
    # the query's nope dims are untouched by RoPE: q_b . RMSNorm(q_a x)
    qa = t.q_a.astype(np.float64) @ t.x[-1].astype(np.float64)
    qa = qa / np.sqrt((qa ** 2).mean() + 1e-6)
    qf = (t.q_b.astype(np.float64) @ qa).reshape(t.H, t.nope + t.rope)
    assert np.max(np.abs(q[:, : t.nope] - qf[:, : t.nope])) <= 1e-12 * np.abs(qf).max()
    sc = 1 / math.sqrt(t.nope + t.rope)
    keys = np.arange(t.T)
    o1 = oracle.absorbed_decode(q[:, : t.nope], q[:, t.nope:], t.kv_b, lc, rc, keys, t.v, sc)
    o2 = oracle.nonabsorbed_decode(q[:, : t.nope], q[:, t.nope:], t.kv_b, lc, rc, keys, t.v, sc)
    assert _rel(o1, o2) <= 1e-10
    y = oracle.o_proj(t.o_w, o1)
    assert _rel(y, t.o_w.astype(np.float64) @ o1.reshape(-1)) <= 1e-12


def test_tiny_layer_rope_positions(oracle):
    """Rc[t] is the kv_a tail rotated at the token's own position t, and the query tail is rotated
    at the last token's position T-1 (colibri-analysis 06, sec. 2.1: the cache row of position pos
    holds the RoPE'd key; the query head tails rotate at the query's position).  Viewed as complex
    numbers, an output pair (y[j], y[half+j]) is the input pair (x[2j], x[2j+1]) multiplied by
    exp(i*pos*theta^(-2j/rope)); every angle is checked against that closed form at its position,
    and the attention logits against the relative-position identity through the separately pinned
    rope function."""
    from mla_latent_kv_dsa_amd import synth
    t = synth.tiny_layer(1)
    lc, rc, q = oracle.tiny_layer(t.x, t.q_a, t.q_b, t.kv_a, t.H, t.nope, t.rope, t.L)
    half = t.rope // 2
    inv = 10000.0 ** (-2.0 * np.arange(half) / t.rope)
    # raw (unrotated) tails from plain float64 matmuls of the layer's weights
    comp = t.x.astype(np.float64) @ t.kv_a.astype(np.float64).T
    k_raw = comp[:, t.L:]
    qa = t.q_a.astype(np.float64) @ t.x[-1].astype(np.float64)
    qa = qa / np.sqrt((qa ** 2).mean() + 1e-6)
    q_raw = (t.q_b.astype(np.float64) @ qa).reshape(t.H, t.nope + t.rope)[:, t.nope:]
    z_in_k = k_raw[:, 0::2] + 1j * k_raw[:, 1::2]
    z_out_k = rc[:, :half] + 1j * rc[:, half:]
    pos = np.arange(t.T, dtype=np.float64)[:, None]
    assert np.max(np.abs(z_out_k - z_in_k * np.exp(1j * pos * inv))) <= 1e-12 * np.abs(z_in_k).max()
    z_in_q = q_raw[:, 0::2] + 1j * q_raw[:, 1::2]
    z_out_q = q[:, t.nope:t.nope + half] + 1j * q[:, t.nope + half:]
    assert np.max(np.abs(z_out_q - z_in_q * np.exp(1j * (t.T - 1) * inv))) <= 1e-12 * np.abs(z_in_q).max()
    # logits q_rot(T-1) . Rc[t] depend on T-1-t only: rotate the raw query by T-1-t and the raw key by 0
    for tt in (0, 17, t.T - 1):
        qr = oracle.rope_interleave(q_raw[None], np.array([t.T - 1 - tt]), 0, t.rope)[0]
        k0 = oracle.rope_interleave(k_raw[tt][None, None], np.array([0]), 0, t.rope)[0, 0]
        lhs = q[:, t.nope:] @ rc[tt]
        assert np.max(np.abs(lhs - qr @ k0)) <= 1e-10 * max(np.abs(lhs).max(), 1e-30)


# ----------------------------------------------------------------------------- cache write
def _cw_case(seed, n=7, L=32, rope=8, hd=24):
    rng = np.random.default_rng(seed)
    comp = (rng.standard_normal((n, L + rope)) * 3.0 + 0.5).astype(np.float32)
    ik = (rng.standard_normal((n, hd)) * 2.0 - 1.5).astype(np.float32)
    pos = rng.integers(0, 5000, n).astype(np.int32)
    return comp, ik, pos


def test_cache_write_latent_is_rms_normalised(oracle):
    """colibri-analysis 06, sec. 2.1: Lc = RMSNorm(first kv_lora values of the kv_a output).  With unit
    gain the mean square of a row is ms / (ms + eps) exactly; a gain vector scales each column."""
    comp, ik, pos = _cw_case(500)
    n, L, rope = comp.shape[0], 32, 8
    eps = 1e-3
    seq = np.zeros(n, np.int32)
    p = np.arange(n, dtype=np.int32)
    lc, rc, _ = oracle.cache_write(comp, None, seq, p, L, rope, rows=n, seq_stride=n, eps_kv=eps)
    ms = (comp[:, :L].astype(np.float64) ** 2).mean(1)
    assert np.max(np.abs((lc ** 2).mean(1) - ms / (ms + eps))) <= 1e-12
    assert np.all(np.sign(lc) == np.sign(comp[:, :L]))
    g = np.random.default_rng(501).uniform(0.5, 2.0, L).astype(np.float32)
    lg, _, _ = oracle.cache_write(comp, None, seq, p, L, rope, rows=n, seq_stride=n, eps_kv=eps, kv_gain=g)
    assert np.max(np.abs(lg - lc * g.astype(np.float64))) <= 1e-12 * np.abs(lg).max()


def test_cache_write_rope_key_rotates_at_token_position(oracle):
    """Rc is the qk_rope tail of the kv_a output rotated at the token's position (sec. 2.1): each
    output pair (y[j], y[half+j]) is the input pair (x[2j], x[2j+1]) times exp(i pos theta_j)."""
    comp, ik, pos = _cw_case(502)
    n, L, rope = comp.shape[0], 32, 8
    seq = np.arange(n, dtype=np.int32) % 3
    _, rc, _ = oracle.cache_write(comp, None, seq, pos, L, rope, rows=3 * 5000, seq_stride=5000)
    rows = seq.astype(np.int64) * 5000 + pos
    half = rope // 2
    inv = 10000.0 ** (-2.0 * np.arange(half) / rope)
    zin = comp[:, L::2].astype(np.float64) + 1j * comp[:, L + 1::2]
    zout = rc[rows, :half] + 1j * rc[rows, half:]
    assert np.max(np.abs(zout - zin * np.exp(1j * pos[:, None] * inv))) <= 1e-12 * np.abs(zin).max()


def test_cache_write_indexer_key_layernorm_and_rope_slice(oracle):
    """sec. 2.2: Ic = RoPE(LayerNorm(ix_wk output), eps 1e-6).  Unrotated, a row has mean 0 and variance
    var / (var + eps); gamma and beta act per column; only dims [off, off + rdim) rotate, by
    exp(i pos theta_j) on the interleaved pairs of that slice."""
    comp, ik, pos = _cw_case(503)
    n, L, rope, hd = comp.shape[0], 32, 8, 24
    seq = np.zeros(n, np.int32)
    p = np.arange(n, dtype=np.int32)
    kw = dict(rows=n, seq_stride=n, eps_ix=1e-2)
    _, _, y = oracle.cache_write(comp, ik, seq, p, L, rope, ix_off=0, ix_rdim=0, **kw)
    var = ik.astype(np.float64).var(1)
    assert np.max(np.abs(y.mean(1))) <= 1e-14
    assert np.max(np.abs(y.var(1) - var / (var + 1e-2))) <= 1e-12
    rng = np.random.default_rng(504)
    gm, bt = rng.uniform(0.5, 2, hd).astype(np.float32), rng.standard_normal(hd).astype(np.float32)
    _, _, yg = oracle.cache_write(comp, ik, seq, p, L, rope, ix_off=0, ix_rdim=0, gamma=gm, beta=bt, **kw)
    assert np.max(np.abs(yg - (y * gm + bt))) <= 1e-12 * np.abs(yg).max()
    off, rd = 10, 12
    _, _, yr = oracle.cache_write(comp, ik, seq, p, L, rope, ix_off=off, ix_rdim=rd, gamma=gm, beta=bt, **kw)
    keep = np.r_[0:off, off + rd:hd]
    assert np.array_equal(yr[:, keep], yg[:, keep])
    h = rd // 2
    inv = 10000.0 ** (-2.0 * np.arange(h) / rd)
    zin = yg[:, off:off + rd:2] + 1j * yg[:, off + 1:off + rd:2]
    zout = yr[:, off:off + h] + 1j * yr[:, off + h:off + rd]
    assert np.max(np.abs(zout - zin * np.exp(1j * p[:, None] * inv))) <= 1e-12 * np.abs(zin).max()


def test_cache_write_paged_rows_worked_example(oracle):
    """Row placement (the cache view: row = block_table[seq][pos / bs] * bs + pos % bs), worked by hand
    for bs = 4 and block table [[2, 0], [1, -1]]: (seq 0, pos 5) -> block 0, row 1; (seq 0, pos 2) ->
    block 2, row 10; (seq 1, pos 3) -> block 1, row 7; (seq 1, pos 6) -> a hole, not written.  Every
    other row keeps its contents; each written row equals the same token written to a contiguous pool."""
    comp, ik, _ = _cw_case(505, n=4)
    L, rope, hd = 32, 8, 24
    seq = np.array([0, 0, 1, 1], np.int32)
    pos = np.array([5, 2, 3, 6], np.int32)
    bt = np.array([[2, 0], [1, -1]], np.int32)
    lc, rc, ic = oracle.cache_write(comp, ik, seq, pos, L, rope, rows=12, block_table=bt, block_size=4,
                                    ix_off=16, ix_rdim=8)
    written = {0: 1, 1: 10, 2: 7}
    assert sorted(np.flatnonzero(~np.isnan(lc[:, 0]))) == sorted(written.values())
    assert sorted(np.flatnonzero(~np.isnan(ic[:, 0]))) == sorted(written.values())
    lc2, rc2, ic2 = oracle.cache_write(comp, ik, seq, pos, L, rope, rows=2 * 8, seq_stride=8, ix_off=16, ix_rdim=8)
    for j, r in written.items():
        c = seq[j] * 8 + pos[j]
        assert np.array_equal(lc[r], lc2[c]) and np.array_equal(rc[r], rc2[c]) and np.array_equal(ic[r], ic2[c])


# ----------------------------------------------------------------------------- quantized kv_b rows
def test_quant_formats_worked_values(oracle):
    """FP8 E4M3, MXFP4 (E2M1 elements with E8M0 block scales) and INT8 rows decode to the values of
    the published format definitions (tests/golden/quant_formats.json, worked by hand)."""
    g = _golden("quant_formats.json")
    codes = np.array([[int(c, 16) for c, _ in g["e4m3"]]], np.uint8)
    got = oracle.dequant_rows(codes, np.array([1.0], np.float32), 1, codes.shape[1])[0]
    assert np.array_equal(got, np.array([v for _, v in g["e4m3"]]))
    assert np.isnan(oracle.dequant_rows(np.array([[0x7F, 0xFF]], np.uint8), np.ones(1, np.float32), 1, 2)).all()
    # E2M1: 32 elements of one block, scale 2^0; element 2k in the low nibble of byte k
    nib = np.array([n for n, _ in g["e2m1"]] + [0] * (32 - len(g["e2m1"])), np.uint8)
    packed = (nib[0::2] | (nib[1::2] << 4)).astype(np.uint8)[None]
    got = oracle.dequant_rows(packed, np.array([[127]], np.uint8), 3, 32)[0]
    assert np.array_equal(got[: len(g["e2m1"])], np.array([v for _, v in g["e2m1"]]))
    for x, v in g["e8m0"]:   # an all-ones-value block (code 2 = 1.0) shows the scale alone
        got = oracle.dequant_rows(np.full((1, 16), 0x22, np.uint8), np.array([[x]], np.uint8), 3, 32)[0]
        assert np.all(got == v), x
    assert np.isnan(oracle.dequant_rows(np.full((1, 16), 0x22, np.uint8), np.array([[255]], np.uint8), 3, 32)).all()
    got = oracle.dequant_rows(np.array([[0x80, 0x7F, 0xFF, 0x01]], np.uint8), np.array([0.25], np.float32), 2, 4)[0]
    assert np.array_equal(got, [-32.0, 31.75, -0.25, 0.25])


def test_quant_e4m3_is_monotone_and_scales_per_row(oracle):
    """Every positive E4M3 code below NaN decodes to a strictly larger value than the one before it
    (the format orders like its integer codes), negatives mirror them, and each row's scale
    multiplies that row only; MXFP4 blocks of 32 take their own scale."""
    pos = np.arange(127, dtype=np.uint8)[None]
    v = oracle.dequant_rows(pos, np.ones(1, np.float32), 1, 127)[0]
    assert np.all(np.diff(v) > 0) and v[0] == 0.0
    neg = oracle.dequant_rows((pos | 0x80).astype(np.uint8), np.ones(1, np.float32), 1, 127)[0]
    assert np.array_equal(neg, -v)
    two = oracle.dequant_rows(np.vstack([pos, pos]), np.array([1.0, 3.0], np.float32), 1, 127)
    assert np.array_equal(two[1], 3.0 * two[0])
    blocks = oracle.dequant_rows(np.full((2, 32), 0x22, np.uint8), np.array([[127, 130], [125, 128]], np.uint8), 3, 64)
    assert np.all(blocks[0, :32] == 1.0) and np.all(blocks[0, 32:] == 8.0)
    assert np.all(blocks[1, :32] == 0.25) and np.all(blocks[1, 32:] == 2.0)
