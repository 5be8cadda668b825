"""CPU oracle for the MLA + DSA path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import this package.  The product (``mla_latent_kv_dsa_amd``) never imports it and
shares no code with it.

The arithmetic lives in ``mla_oracle.c`` (plain C, double precision, plus the fixed-order
fp32 indexer contract); this module compiles it with gcc and wraps it with ctypes.
Each wrapper names the passage it follows:

* chen3feng, "colibri-analysis 06: MLA attention and KV cache" -- sec. 1 (compressed cache),
  sec. 2.1 (interleaved partial RoPE), sec. 2.2 (DSA lightning indexer, top-2048),
  sec. 2.3 (absorbed / non-absorbed attention).
* aiknowledge.cn, "Ch.7 sec. 03: token-exact forward validation and faithful DSA" --
  sec. 2 (the indexer cache Ic is fp32).

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mla_oracle.c")
_LIB = os.path.join(_HERE, "libmla_oracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile ``mla_oracle.c`` into ``libmla_oracle.so`` (gcc, no fast-math, no FMA
    contraction, OpenMP over independent units)."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
               "-fno-fast-math", "-fopenmp", "-Wall", "-Wextra", "-o", _LIB + ".tmp", _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    lib.orc_num_threads.restype = ctypes.c_int
    lib.orc_set_num_threads.argtypes = [ctypes.c_int]
    lib.orc_rope_interleave.argtypes = [P, P, i64, i32, i32, i32, i32, P, f64]
    lib.orc_index_scores_f32.argtypes = [P, P, P, i64, i32, i32, P]
    lib.orc_index_scores_f64.argtypes = [P, P, P, i64, i32, i32, P]
    lib.orc_topk.argtypes = [P, i64, i32, P]
    lib.orc_topk.restype = i32
    lib.orc_topk_batch.argtypes = [P, i32, i64, P, i32, P, P]
    lib.orc_absorbed_decode.argtypes = [P, P, P, P, P, P, i64, i32, i32, i32, i32, i32, f64, P]
    lib.orc_nonabsorbed_decode.argtypes = [P, P, P, P, P, P, i64, i32, i32, i32, i32, i32, f64, P]
    lib.orc_prefill_rows.argtypes = [P, P, P, P, i32, i32, i32, i32, i32, i32, i32, f64, P, i32, P]
    lib.orc_tiny_layer.argtypes = [P, i32, i32, P, i32, P, P, i32, i32, i32, i32, f64, f64, P, P, P]
    lib.orc_o_proj.argtypes = [P, P, i32, i32, P]
    lib.orc_dequant_rows.argtypes = [P, P, i32, i64, i32, P]
    lib.orc_cache_write.argtypes = [P, P, i64, P, P, i32, i32, i32, P, P, P, i32, i32, f64, f64, f64, P, i32, i32,
                                    i64, i64, P, P, P]
    _lib = lib
    return lib


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> the float32 values they encode (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def num_threads() -> int:
    return int(_load().orc_num_threads())


def set_num_threads(n: int) -> None:
    _load().orc_set_num_threads(int(n))


def rope_interleave(x, pos, rope_off: int, rope_dim: int, theta: float = 10000.0) -> np.ndarray:
    """Interleaved partial RoPE in double.  x: [n_tok, n_heads, head_dim]; pos: [n_tok].
    (colibri-analysis 06, sec. 2.1)"""
    x = _f64(x)
    assert x.ndim == 3 and rope_dim % 2 == 0 and rope_off + rope_dim <= x.shape[2]
    pos = _i32(pos)
    assert pos.shape == (x.shape[0],)
    y = np.empty_like(x)
    _load().orc_rope_interleave(_p(x), _p(y), x.shape[0], x.shape[1], x.shape[2], rope_off,
                                rope_dim, _p(pos), float(theta))
    return y


def index_scores(q, w, ic) -> np.ndarray:
    """Fixed-order fp32 indexer scores for one query.  q: [n_ih, hd], w: [n_ih],
    ic: [T, hd] -> [T] float32.  (colibri-analysis 06, sec. 2.2)"""
    q, w, ic = _f32(q), _f32(w), _f32(ic)
    n_ih, hd = q.shape
    assert w.shape == (n_ih,) and ic.ndim == 2 and ic.shape[1] == hd
    out = np.empty(ic.shape[0], dtype=np.float32)
    _load().orc_index_scores_f32(_p(q), _p(w), _p(ic), ic.shape[0], n_ih, hd, _p(out))
    return out


def index_scores_f64(q, w, ic) -> np.ndarray:
    q, w, ic = _f32(q), _f32(w), _f32(ic)
    n_ih, hd = q.shape
    out = np.empty(ic.shape[0], dtype=np.float64)
    _load().orc_index_scores_f64(_p(q), _p(w), _p(ic), ic.shape[0], n_ih, hd, _p(out))
    return out


def topk(scores, n_valid: int, k: int):
    """Top-k positions of scores[:n_valid] (score desc, position asc), returned ascending.
    Returns (sel[k] with -1 padding, nsel).  (colibri-analysis 06, sec. 2.2)"""
    s = _f32(scores)
    sel = np.empty(k, dtype=np.int32)
    nsel = _load().orc_topk(_p(s), int(n_valid), int(k), _p(sel))
    return sel, int(nsel)


def topk_batch(scores, n_valid, k: int):
    s = _f32(scores)
    B, t_max = s.shape
    nv = _i32(n_valid)
    sel = np.empty((B, k), dtype=np.int32)
    nsel = np.empty(B, dtype=np.int32)
    _load().orc_topk_batch(_p(s), B, t_max, _p(nv), int(k), _p(sel), _p(nsel))
    return sel, nsel


def _decode(fn, q_nope, q_rope, kv_b, lc, rc, keys, nope, v, sm_scale):
    q_nope, q_rope, kv_b, lc, rc = _f32(q_nope), _f32(q_rope), _f32(kv_b), _f32(lc), _f32(rc)
    keys = _i32(keys)
    H = q_nope.shape[0]
    assert q_nope.shape == (H, nope)
    rope = q_rope.shape[1]
    L = lc.shape[1]
    assert kv_b.shape == (H * (nope + v), L) and rc.shape[1] == rope
    assert keys.size == 0 or (keys.min() >= 0 and keys.max() < lc.shape[0])
    out = np.empty((H, v), dtype=np.float64)
    fn(_p(q_nope), _p(q_rope), _p(kv_b), _p(lc), _p(rc), _p(keys), keys.size, H, nope, rope, v,
       L, float(sm_scale), _p(out))
    return out


def absorbed_decode(q_nope, q_rope, kv_b, lc, rc, keys, v: int, sm_scale: float) -> np.ndarray:
    """Absorbed MLA decode of one query over the cached positions ``keys``; [H, v] double.
    (colibri-analysis 06, sec. 2.3, absorbed path)"""
    return _decode(_load().orc_absorbed_decode, q_nope, q_rope, kv_b, lc, rc, keys,
                   np.asarray(q_nope).shape[1], v, sm_scale)


def nonabsorbed_decode(q_nope, q_rope, kv_b, lc, rc, keys, v: int, sm_scale: float) -> np.ndarray:
    """Non-absorbed (k/v rebuilt through kv_b) attention of one query; [H, v] double.
    (colibri-analysis 06, sec. 2.3, non-absorbed path)"""
    return _decode(_load().orc_nonabsorbed_decode, q_nope, q_rope, kv_b, lc, rc, keys,
                   np.asarray(q_nope).shape[1], v, sm_scale)


def prefill_rows(q, kv_b, lc, rc, pos_base: int, nope: int, v: int, sm_scale: float, rows) -> np.ndarray:
    """Causal non-absorbed prefill evaluated at query rows ``rows``.  q: [S, H, nope+rope]
    (rotated tail), lc: [T, L], rc: [T, rope] -> [len(rows), H, v] double.
    (colibri-analysis 06, sec. 2 and 2.3)"""
    q, kv_b, lc, rc = _f32(q), _f32(kv_b), _f32(lc), _f32(rc)
    rows = _i32(rows)
    S, H, qh = q.shape
    rope = qh - nope
    L = lc.shape[1]
    assert kv_b.shape == (H * (nope + v), L) and rc.shape[1] == rope
    assert rows.size > 0 and rows.min() >= 0 and rows.max() < S
    assert pos_base + rows.max() + 1 <= lc.shape[0]
    out = np.empty((rows.size, H, v), dtype=np.float64)
    _load().orc_prefill_rows(_p(q), _p(kv_b), _p(lc), _p(rc), S, int(pos_base), H, nope, rope, v,
                             L, float(sm_scale), _p(rows), rows.size, _p(out))
    return out


def tiny_layer(x, q_a, q_b, kv_a, H: int, nope: int, rope: int, L: int,
               eps: float = 1e-6, theta: float = 10000.0):
    """Projections of a tiny MLA layer (colibri-analysis 06, sec. 2.1).  Returns
    (lc [T, L], rc [T, rope] rotated, q [H, nope+rope] of the last token, tail rotated)."""
    x, q_a, q_b, kv_a = _f32(x), _f32(q_a), _f32(q_b), _f32(kv_a)
    T, hidden = x.shape
    q_lora = q_a.shape[0]
    assert q_a.shape == (q_lora, hidden) and q_b.shape == (H * (nope + rope), q_lora)
    assert kv_a.shape == (L + rope, hidden)
    lc = np.empty((T, L), dtype=np.float64)
    rc = np.empty((T, rope), dtype=np.float64)
    q = np.empty((H, nope + rope), dtype=np.float64)
    _load().orc_tiny_layer(_p(x), T, hidden, _p(q_a), q_lora, _p(q_b), _p(kv_a), H, nope, rope, L,
                           float(eps), float(theta), _p(lc), _p(rc), _p(q))
    return lc, rc, q


def o_proj(o_w, attn) -> np.ndarray:
    """Output projection y = o_w . attn (colibri-analysis 06, sec. 2.3)."""
    o_w = _f32(o_w)
    a = _f64(attn).reshape(-1)
    hidden, hv = o_w.shape
    assert a.size == hv
    y = np.empty(hidden, dtype=np.float64)
    _load().orc_o_proj(_p(o_w), _p(a), hidden, hv, _p(y))
    return y


def cache_write(comp, ik, seq, pos, L: int, rope: int, *, rows: int, hd: int = 0, kv_gain=None, gamma=None,
                beta=None, ix_off: int = 0, ix_rdim: int = 0, eps_kv: float = 1e-6, eps_ix: float = 1e-6,
                theta: float = 10000.0, block_table=None, block_size: int = 0, seq_stride: int = 0,
                lc=None, rc=None, ic=None):
    """Write new tokens into the cache pools (colibri-analysis 06, sec. 2.1 KV path and sec. 2.2
    indexer key): Lc = RMSNorm(comp[:L]) * kv_gain, Rc = RoPE(comp[L:]), Ic = RoPE over
    [ix_off, ix_off + ix_rdim) of LayerNorm(ik), at each token's position.  Pools are float64
    [rows, width]; pass existing pools (lc, rc, ic) to write into them, otherwise they start as NaN
    so that untouched rows stay recognisable.  Returns (lc, rc, ic)."""
    comp = _f32(comp)
    n = comp.shape[0]
    assert comp.shape == (n, L + rope)
    seq, pos = _i32(seq), _i32(pos)
    assert seq.shape == (n,) and pos.shape == (n,)
    if ik is not None:
        ik = _f32(ik)
        hd = ik.shape[1]
        assert ik.shape == (n, hd) and ix_rdim % 2 == 0 and ix_off + ix_rdim <= hd
    lc = np.full((rows, L), np.nan) if lc is None else lc
    rc = np.full((rows, rope), np.nan) if rc is None else rc
    ic = (np.full((rows, hd), np.nan) if ic is None else ic) if ik is not None else None
    assert lc.dtype == np.float64 and lc.flags.c_contiguous and lc.shape == (rows, L)
    assert rc.dtype == np.float64 and rc.flags.c_contiguous and rc.shape == (rows, rope)
    if ic is not None:
        assert ic.dtype == np.float64 and ic.flags.c_contiguous and ic.shape == (rows, hd)
    gains = [None if a is None else np.ascontiguousarray(_f32(a)) for a in (kv_gain, gamma, beta)]
    bt = None if block_table is None else _i32(block_table)
    _load().orc_cache_write(_p(comp), None if ik is None else _p(ik), n, _p(seq), _p(pos), L, rope, hd,
                            None if gains[0] is None else _p(gains[0]), None if gains[1] is None else _p(gains[1]),
                            None if gains[2] is None else _p(gains[2]), ix_off, ix_rdim, float(eps_kv),
                            float(eps_ix), float(theta), None if bt is None else _p(bt), int(block_size),
                            0 if bt is None else bt.shape[1], int(seq_stride), int(rows), _p(lc), _p(rc),
                            None if ic is None else _p(ic))
    return lc, rc, ic


QFMT_FP8_E4M3, QFMT_INT8, QFMT_MXFP4 = 1, 2, 3


def dequant_rows(codes, scales, fmt: int, cols: int) -> np.ndarray:
    """Decode quantized kv_b rows to float64 (aiknowledge.cn Ch.7 sec. 03, sec. 3/5: int8, FP8 and
    MXFP4 weight formats).  fmt 1: FP8 E4M3 codes [rows, cols] with an fp32 scale per row; fmt 2:
    int8 codes with an fp32 scale per row; fmt 3: MXFP4, FP4 E2M1 codes two per byte (even element in
    the low nibble) [rows, cols/2] with an E8M0 scale byte per 32 elements [rows, cols/32]."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    rows = codes.shape[0]
    if fmt in (1, 2):
        assert codes.shape == (rows, cols)
        sc = _f32(scales)
        assert sc.shape == (rows,)
    else:
        assert fmt == 3 and cols % 32 == 0 and codes.shape == (rows, cols // 2)
        sc = np.ascontiguousarray(scales, dtype=np.uint8)
        assert sc.shape == (rows, cols // 32)
    out = np.empty((rows, cols), dtype=np.float64)
    _load().orc_dequant_rows(_p(codes), _p(sc), int(fmt), rows, int(cols), _p(out))
    return out
