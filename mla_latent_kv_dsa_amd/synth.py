"""Seeded synthetic workloads for the MLA + DSA path.

This module draws inputs only: random numbers from ``numpy.random.default_rng(seed)`` in a
fixed order, bf16 rounding of those draws (round to nearest even on the bit pattern),
and the paged-pool layout (a seeded random block permutation).  It computes nothing of
the method itself, so the GPU tests, the benchmark and the CPU oracle can all consume the
same arrays.  No trained weights, prompts or datasets exist here: every value is synthetic,
shaped like a GLM-5.2-class MLA layer (64 heads, qk_nope 192, qk_rope 64, v_head 256,
kv_lora 512; a 32-head, 128-wide DSA indexer keeping 2048 keys).

Draw order (per workload, one generator each):
  tiny  (seed 1): x[T, hidden], q_a, q_b, kv_a, kv_b, o_w   -- all fp32
  decode(seed s): Lc[T, L], Rc[T, rope], q_nope[B, H, nope], q_rope[B, H, rope],
                  kv_b[H*(nope+v), L], then (DSA) Ic[T, hd], q_idx[B, n_ih, hd], w_idx[B, n_ih]
  prefill       : q[S, H, nope+rope], Lc, Rc, kv_b
  paged batch   : seq_len[B], block permutation, Lc pool, Rc pool, Ic pool, q_nope, q_rope,
                  kv_b, q_idx, w_idx
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# GLM-5.2-like dims
H, QK_NOPE, QK_ROPE, V_HEAD, KV_LORA = 64, 192, 64, 256, 512
N_IH, INDEX_HD, TOPK = 32, 128, 2048
BLOCK = 64


def to_bf16_bits(x) -> np.ndarray:
    """float32 -> bf16 bit pattern (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + r) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    """bf16 bit pattern -> float32 value (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def tile_index_keys(ic: np.ndarray) -> np.ndarray:
    """The indexer pool [rows, hd] rearranged into the MLA_IC_TILE64 layout: rows in aligned
    groups of 64, each group stored dims-major in quads of 4 (element d of row r at flat index
    (r // 64) * 64 * hd + (d // 4) * 256 + (r % 64) * 4 + d % 4).  Same values, same shape."""
    rows, hd = ic.shape
    assert rows % 64 == 0 and hd % 4 == 0
    if not isinstance(ic, np.ndarray):   # a torch tensor: the same rearrangement on its device
        return ic.reshape(rows // 64, 64, hd // 4, 4).permute(0, 2, 1, 3).contiguous().reshape(rows, hd)
    t = ic.reshape(rows // 64, 64, hd // 4, 4).transpose(0, 2, 1, 3)
    return np.ascontiguousarray(t).reshape(rows, hd)


def _normal(rng, shape, std=1.0, chunk=1 << 26) -> np.ndarray:
    """N(0, std^2) float32 draws, generated in chunks to bound peak memory."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        rng.standard_normal(e - s, dtype=np.float32, out=out[s:e])
    if std != 1.0:
        out *= np.float32(std)
    return out.reshape(shape)


def _normal_bf16(rng, shape, std=1.0, chunk=1 << 26) -> np.ndarray:
    """N(0, std^2) draws rounded to bf16, returned as uint16 bit patterns."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    buf = np.empty(min(n, chunk), dtype=np.float32)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        b = buf[: e - s]
        rng.standard_normal(e - s, dtype=np.float32, out=b)
        if std != 1.0:
            b *= np.float32(std)
        out[s:e] = to_bf16_bits(b)
    return out.reshape(shape)


@dataclass
class TinyLayer:
    """A tiny fp32 MLA layer: H=4, qk_nope=16, qk_rope=8, v_head=16, kv_lora=32, hidden=64,
    q_lora=32, T=64 cached tokens.  Activations N(0,1), weights N(0, 0.02^2)."""
    H: int = 4
    nope: int = 16
    rope: int = 8
    v: int = 16
    L: int = 32
    hidden: int = 64
    q_lora: int = 32
    T: int = 64
    x: np.ndarray = field(default=None, repr=False)
    q_a: np.ndarray = field(default=None, repr=False)
    q_b: np.ndarray = field(default=None, repr=False)
    kv_a: np.ndarray = field(default=None, repr=False)
    kv_b: np.ndarray = field(default=None, repr=False)
    o_w: np.ndarray = field(default=None, repr=False)


def tiny_layer(seed: int = 1) -> TinyLayer:
    t = TinyLayer()
    rng = np.random.default_rng(seed)
    t.x = _normal(rng, (t.T, t.hidden))
    t.q_a = _normal(rng, (t.q_lora, t.hidden), 0.02)
    t.q_b = _normal(rng, (t.H * (t.nope + t.rope), t.q_lora), 0.02)
    t.kv_a = _normal(rng, (t.L + t.rope, t.hidden), 0.02)
    t.kv_b = _normal(rng, (t.H * (t.nope + t.v), t.L), 0.02)
    t.o_w = _normal(rng, (t.hidden, t.H * t.v), 0.02)
    return t


@dataclass
class Decode:
    """One decode step over contiguous caches (B sequences of equal length T).
    Arrays are bf16 bit patterns (uint16) when ``bf16`` else float32; Ic/q_idx/w_idx are
    always float32.  Rc rows are the cached (already rotated) keys; q_rope is the query's
    tail before rotation.  The query sits at position T-1 and sees keys 0..T-1."""
    B: int
    T: int
    H: int
    nope: int
    rope: int
    v: int
    L: int
    bf16: bool
    lc: np.ndarray = field(repr=False)
    rc: np.ndarray = field(repr=False)
    q_nope: np.ndarray = field(repr=False)
    q_rope: np.ndarray = field(repr=False)
    kv_b: np.ndarray = field(repr=False)
    n_ih: int = 0
    hd: int = 0
    ic: np.ndarray = field(default=None, repr=False)
    q_idx: np.ndarray = field(default=None, repr=False)
    w_idx: np.ndarray = field(default=None, repr=False)


def decode(seed: int, T: int, B: int = 1, *, H_=H, nope=QK_NOPE, rope=QK_ROPE, v=V_HEAD,
           L=KV_LORA, bf16=True, dsa=False, n_ih=N_IH, hd=INDEX_HD, w_std=0.02) -> Decode:
    """Contiguous decode workload.  Lc/Rc: [B*T, *] (sequence b occupies rows b*T..b*T+T-1).
    Values: Lc, Rc, q ~ N(0,1); kv_b ~ N(0, w_std^2); Ic, q_idx, w_idx ~ N(0,1)."""
    rng = np.random.default_rng(seed)
    g = _normal_bf16 if bf16 else _normal
    lc = g(rng, (B * T, L))
    rc = g(rng, (B * T, rope))
    q_nope = g(rng, (B, H_, nope))
    q_rope = g(rng, (B, H_, rope))
    kv_b = g(rng, (H_ * (nope + v), L), w_std)
    d = Decode(B, T, H_, nope, rope, v, L, bf16, lc, rc, q_nope, q_rope, kv_b)
    if dsa:
        d.n_ih, d.hd = n_ih, hd
        d.ic = _normal(rng, (B * T, hd))
        d.q_idx = _normal(rng, (B, n_ih, hd))
        d.w_idx = _normal(rng, (B, n_ih))
    return d


@dataclass
class Prefill:
    S: int
    pos_base: int
    H: int
    nope: int
    rope: int
    v: int
    L: int
    bf16: bool
    q: np.ndarray = field(repr=False)      # [S, H, nope+rope], tail already rotated
    lc: np.ndarray = field(repr=False)     # [pos_base+S, L]
    rc: np.ndarray = field(repr=False)     # [pos_base+S, rope]
    kv_b: np.ndarray = field(repr=False)


def prefill(seed: int, S: int, pos_base: int = 0, *, H_=H, nope=QK_NOPE, rope=QK_ROPE,
            v=V_HEAD, L=KV_LORA, bf16=True, w_std=0.02) -> Prefill:
    rng = np.random.default_rng(seed)
    g = _normal_bf16 if bf16 else _normal
    T = pos_base + S
    q = g(rng, (S, H_, nope + rope))
    lc = g(rng, (T, L))
    rc = g(rng, (T, rope))
    kv_b = g(rng, (H_ * (nope + v), L), w_std)
    return Prefill(S, pos_base, H_, nope, rope, v, L, bf16, q, lc, rc, kv_b)


@dataclass
class PagedBatch:
    """Batched decode over paged caches: 64-token blocks, one shared block table.
    Physical block p of the pools holds tokens [64*j, 64*j+64) of sequence b when
    block_table[b, j] == p.  Unused table entries are -1."""
    B: int
    seq_len: np.ndarray                    # int32 [B], tokens cached including the query's own
    block_size: int
    max_blocks: int
    block_table: np.ndarray = field(repr=False)   # int32 [B, max_blocks]
    n_blocks: int = 0
    lc: np.ndarray = field(default=None, repr=False)      # bf16 bits [n_blocks*bs, L]
    rc: np.ndarray = field(default=None, repr=False)      # bf16 bits [n_blocks*bs, rope]
    ic: np.ndarray = field(default=None, repr=False)      # f32 [n_blocks*bs, hd]
    q_nope: np.ndarray = field(default=None, repr=False)
    q_rope: np.ndarray = field(default=None, repr=False)
    kv_b: np.ndarray = field(default=None, repr=False)
    q_idx: np.ndarray = field(default=None, repr=False)
    w_idx: np.ndarray = field(default=None, repr=False)
    H: int = H
    nope: int = QK_NOPE
    rope: int = QK_ROPE
    v: int = V_HEAD
    L: int = KV_LORA
    n_ih: int = N_IH
    hd: int = INDEX_HD

    def rows(self, b: int, t) -> np.ndarray:
        """Pool row index of logical token(s) t of sequence b (layout bookkeeping only)."""
        t = np.asarray(t, dtype=np.int64)
        return self.block_table[b, t // self.block_size].astype(np.int64) * self.block_size + t % self.block_size


def paged_batch(seed: int, B: int = 32, t_lo: int = 8192, t_hi: int = 131072, *,
                block_size: int = BLOCK, max_ctx: int = 131072, H_=H, nope=QK_NOPE,
                rope=QK_ROPE, v=V_HEAD, L=KV_LORA, n_ih=N_IH, hd=INDEX_HD,
                w_std=0.02, meta_only: bool = False) -> PagedBatch:
    """seq_len ~ U{t_lo..t_hi} (inclusive); pools filled in physical order after a seeded
    random permutation of the blocks; values distributed as in ``decode``.  meta_only: only the
    lengths and the block table (the same draws), no pools or queries."""
    rng = np.random.default_rng(seed)
    seq_len = rng.integers(t_lo, t_hi + 1, size=B).astype(np.int32)
    max_blocks = (max_ctx + block_size - 1) // block_size
    nb = [(int(s) + block_size - 1) // block_size for s in seq_len]
    n_blocks = int(sum(nb))
    perm = rng.permutation(n_blocks).astype(np.int32)
    bt = np.full((B, max_blocks), -1, dtype=np.int32)
    o = 0
    for b in range(B):
        bt[b, : nb[b]] = perm[o: o + nb[b]]
        o += nb[b]
    pb = PagedBatch(B, seq_len, block_size, max_blocks, bt, n_blocks, H=H_, nope=nope, rope=rope,
                    v=v, L=L, n_ih=n_ih, hd=hd)
    if meta_only:
        return pb
    rows = n_blocks * block_size
    pb.lc = _normal_bf16(rng, (rows, L))
    pb.rc = _normal_bf16(rng, (rows, rope))
    pb.ic = _normal(rng, (rows, hd))
    pb.q_nope = _normal_bf16(rng, (B, H_, nope))
    pb.q_rope = _normal_bf16(rng, (B, H_, rope))
    pb.kv_b = _normal_bf16(rng, (H_ * (nope + v), L), w_std)
    pb.q_idx = _normal(rng, (B, n_ih, hd))
    pb.w_idx = _normal(rng, (B, n_ih))
    return pb


def paged_values_torch(pb: PagedBatch, seed: int, device, w_std=0.02) -> dict:
    """Pool and query values for the lengths and block table of ``pb`` (from
    ``paged_batch(..., meta_only=True)``), drawn on a torch device with a seeded
    torch.Generator: the distributions of ``paged_batch`` (N(0, 1), kv_b N(0, w_std^2), bf16
    where the numpy draw is bf16), without the minutes a host draw of 2M cached rows takes.
    ic comes row-major (tile it with ``tile_index_keys``)."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    rows = pb.n_blocks * pb.block_size

    def rn(*shape, std=1.0, bf16=False):
        x = torch.randn(*shape, generator=g, device=device)
        if std != 1.0:
            x *= std
        return x.bfloat16() if bf16 else x

    return dict(lc=rn(rows, pb.L, bf16=True), rc=rn(rows, pb.rope, bf16=True), ic=rn(rows, pb.hd),
                q_nope=rn(pb.B, pb.H, pb.nope, bf16=True), q_rope=rn(pb.B, pb.H, pb.rope, bf16=True),
                kv_b=rn(pb.H * (pb.nope + pb.v), pb.L, std=w_std, bf16=True),
                q_idx=rn(pb.B, pb.n_ih, pb.hd), w_idx=rn(pb.B, pb.n_ih))


QFMT_FP8_E4M3, QFMT_INT8, QFMT_MXFP4 = 1, 2, 3


def quantized_kv_b(seed: int, fmt: int, rows: int, cols: int):
    """Random codes and scales of a quantized kv_b [rows, cols] (drawn directly in the format, with
    magnitudes like N(0, 0.02^2) weights; no weight is quantized here):
      FP8 E4M3: sign uniform, exponent field ~ round(N(7, 1.5)) clipped to [0, 15], mantissa uniform,
                the NaN code (exponent 15, mantissa 7) redrawn as mantissa 6; scale per row
                U(0.8, 1.2) * 0.02 / 1.5, float32
      INT8:     round(N(0, 40^2)) clipped to [-127, 127]; scale per row U(0.8, 1.2) * 0.02 / 40
      MXFP4:    nibbles uniform over the 16 E2M1 codes, two per byte; E8M0 scale per 32 columns
                uniform over 127 - 9 .. 127 - 7
    Returns (codes uint8, scales float32 [rows] or uint8 [rows, cols / 32])."""
    rng = np.random.default_rng(seed)
    if fmt == QFMT_FP8_E4M3:
        s = rng.integers(0, 2, (rows, cols))
        e = np.clip(np.rint(rng.normal(7.0, 1.5, (rows, cols))), 0, 15).astype(np.int64)
        m = rng.integers(0, 8, (rows, cols))
        m = np.where((e == 15) & (m == 7), 6, m)
        codes = ((s << 7) | (e << 3) | m).astype(np.uint8)
        scales = (rng.uniform(0.8, 1.2, rows) * 0.02 / 1.5).astype(np.float32)
    elif fmt == QFMT_INT8:
        codes = np.clip(np.rint(rng.normal(0.0, 40.0, (rows, cols))), -127, 127).astype(np.int8).view(np.uint8)
        scales = (rng.uniform(0.8, 1.2, rows) * 0.02 / 40.0).astype(np.float32)
    elif fmt == QFMT_MXFP4:
        assert cols % 32 == 0
        nib = rng.integers(0, 16, (rows, cols)).astype(np.uint8)
        codes = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
        scales = rng.integers(127 - 9, 127 - 6, (rows, cols // 32)).astype(np.uint8)
    else:
        raise ValueError(fmt)
    return codes, scales
