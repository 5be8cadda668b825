"""MI355X-native MLA latent-KV attention with a DSA lightning indexer.

Thin binding over ``libmla_dsa.so`` (HIP for gfx950, built by ``mla_latent_kv_dsa_amd.build``).
Each function has the name of the C entry point it calls and only marshals arguments:
torch tensors become device pointers, torch's current stream becomes the HIP stream,
and a non-OK status becomes an :class:`MlaError`.  Every step of the computation runs in
the library's kernels; there is no other implementation behind these names.  If the
library has not been built, every call raises.

Pages the operations follow: chen3feng, "colibri-analysis 06: MLA attention and KV cache"
(sec. 1, 2, 2.1, 2.2, 2.3) and aiknowledge.cn, "Ch.7 sec. 03: token-exact forward
validation and faithful DSA" (sec. 2).  The header ``include/mla_dsa.h`` states the exact
contract of each call.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla_dsa.so")

MLA_OK, MLA_ERR_ARG, MLA_ERR_UNSUPPORTED, MLA_ERR_WORKSPACE, MLA_ERR_HIP = 0, -1, -2, -3, -4
MLA_FP32, MLA_BF16 = 0, 1
MLA_IC_ROWS, MLA_IC_TILE64 = 0, 1
MLA_Q_FP8_E4M3, MLA_Q_INT8, MLA_Q_MXFP4 = 1, 2, 3

EXPORTED = (
    "mla_rope_interleave", "mla_cache_write", "dsa_index_scores", "dsa_topk_workspace_bytes", "dsa_topk_select",
    "dsa_index_select_workspace_bytes", "dsa_index_select",
    "mla_decode_workspace_bytes", "mla_absorbed_decode", "mla_decode_absorb", "mla_decode_attend",
    "mla_dsa_decode_workspace_bytes", "mla_dsa_decode", "mla_dsa_decode_noalloc",
    "mla_dsa_decode_shared_workspace_bytes", "mla_dsa_decode_shared",
    "mla_attention_absorbs", "mla_attention_workspace_bytes", "mla_attention",
    "dsa_prefill_select_workspace_bytes", "dsa_prefill_select", "mla_absorbed_decode_q", "mla_dsa_decode_q",
    "mla_prefill_workspace_bytes",
    "mla_prefill_nonabsorbed", "mla_status_string", "mla_last_error",
)


class MlaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


class mla_dims(ctypes.Structure):
    _fields_ = [("n_heads", ctypes.c_int32), ("qk_nope", ctypes.c_int32), ("qk_rope", ctypes.c_int32),
                ("v_head", ctypes.c_int32), ("kv_lora", ctypes.c_int32)]


class mla_kv_view(ctypes.Structure):
    _fields_ = [("lc", ctypes.c_void_p), ("rc", ctypes.c_void_p), ("ic", ctypes.c_void_p),
                ("rows", ctypes.c_int64), ("kv_dtype", ctypes.c_int), ("index_hd", ctypes.c_int32),
                ("block_table", ctypes.c_void_p), ("block_size", ctypes.c_int32),
                ("max_blocks", ctypes.c_int32), ("seq_stride", ctypes.c_int64),
                ("seq_len", ctypes.c_void_p), ("max_seq_len", ctypes.c_int64), ("ic_layout", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmla_dsa.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m mla_latent_kv_dsa_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    st = ctypes.c_int
    L.mla_rope_interleave.argtypes = [P, ctypes.c_int, i64, i32, i64, i64, i32, i32, P, ctypes.c_double, P]
    L.mla_rope_interleave.restype = st
    L.mla_cache_write.argtypes = [P, P, ctypes.c_int, i64, P, P, i32, i32, i32, P, P, P, i32, i32, ctypes.c_double,
                                  ctypes.c_double, ctypes.c_double, ctypes.POINTER(mla_kv_view), P]
    L.mla_cache_write.restype = st
    L.dsa_index_scores.argtypes = [P, P, i32, i32, ctypes.POINTER(mla_kv_view), i64, P, P]
    L.dsa_index_scores.restype = st
    L.dsa_topk_workspace_bytes.argtypes = [i32, i64, i32]
    L.dsa_topk_workspace_bytes.restype = ctypes.c_size_t
    L.dsa_topk_select.argtypes = [P, i32, i64, P, i32, P, P, P, ctypes.c_size_t, P]
    L.dsa_topk_select.restype = st
    L.dsa_index_select_workspace_bytes.argtypes = [i32, i64, i32]
    L.dsa_index_select_workspace_bytes.restype = ctypes.c_size_t
    L.dsa_index_select.argtypes = [P, P, i32, i32, ctypes.POINTER(mla_kv_view), i64, i32, P, P, P, P,
                                   ctypes.c_size_t, P]
    L.dsa_index_select.restype = st
    L.mla_decode_workspace_bytes.argtypes = [ctypes.POINTER(mla_dims), i32, i64]
    L.mla_decode_workspace_bytes.restype = ctypes.c_size_t
    L.mla_absorbed_decode.argtypes = [P, P, ctypes.c_int, P, ctypes.c_int, ctypes.POINTER(mla_dims), i32,
                                      ctypes.POINTER(mla_kv_view), P, P, i32, ctypes.c_float, P, P,
                                      ctypes.c_size_t, P]
    L.mla_absorbed_decode.restype = st
    L.mla_decode_absorb.argtypes = [P, ctypes.c_int, P, ctypes.c_int, ctypes.POINTER(mla_dims), i32, P,
                                    ctypes.c_size_t, P]
    L.mla_decode_absorb.restype = st
    L.mla_decode_attend.argtypes = [P, ctypes.c_int, P, ctypes.c_int, ctypes.POINTER(mla_dims), i32,
                                    ctypes.POINTER(mla_kv_view), P, P, i32, ctypes.c_float, P, P, ctypes.c_size_t, P]
    L.mla_decode_attend.restype = st
    L.mla_dsa_decode_workspace_bytes.argtypes = [ctypes.POINTER(mla_dims), i32, i64, i32]
    L.mla_dsa_decode_workspace_bytes.restype = ctypes.c_size_t
    L.mla_dsa_decode.argtypes = [P, P, ctypes.c_int, ctypes.c_double, P, P, i32, P, ctypes.c_int,
                                 ctypes.POINTER(mla_dims), i32, ctypes.POINTER(mla_kv_view), i64, i32, ctypes.c_float,
                                 P, P, P, P, P, ctypes.c_size_t, P]
    L.mla_dsa_decode.restype = st
    L.mla_dsa_decode_noalloc.argtypes = [P, P, ctypes.c_int, ctypes.c_double, P, P, i32, P, ctypes.c_int,
                                         ctypes.POINTER(mla_dims), i32, ctypes.POINTER(mla_kv_view), i64, i32,
                                         ctypes.c_float, P, P, P, P, P]
    L.mla_dsa_decode_noalloc.restype = st
    L.mla_dsa_decode_shared_workspace_bytes.argtypes = [ctypes.POINTER(mla_dims), i32, i32]
    L.mla_dsa_decode_shared_workspace_bytes.restype = ctypes.c_size_t
    L.mla_dsa_decode_shared.argtypes = [P, P, ctypes.c_int, ctypes.c_double, P, ctypes.c_int, ctypes.POINTER(mla_dims),
                                        i32, ctypes.POINTER(mla_kv_view), P, P, i32, ctypes.c_float, P, P,
                                        ctypes.c_size_t, P]
    L.mla_dsa_decode_shared.restype = st
    L.mla_prefill_workspace_bytes.argtypes = [ctypes.POINTER(mla_dims), i32, i64]
    L.mla_prefill_workspace_bytes.restype = ctypes.c_size_t
    L.mla_prefill_nonabsorbed.argtypes = [P, ctypes.c_int, P, ctypes.c_int, ctypes.POINTER(mla_dims),
                                          ctypes.POINTER(mla_kv_view), i32, i32, ctypes.c_float, P,
                                          ctypes.c_int, P, ctypes.c_size_t, P]
    L.mla_prefill_nonabsorbed.restype = st
    L.mla_attention_absorbs.argtypes = [i32, i32]
    L.mla_attention_absorbs.restype = i32
    L.mla_attention_workspace_bytes.argtypes = [ctypes.POINTER(mla_dims), i32, i32, i32, i32]
    L.mla_attention_workspace_bytes.restype = ctypes.c_size_t
    L.mla_attention.argtypes = [P, ctypes.c_int, P, ctypes.c_int, ctypes.POINTER(mla_dims), ctypes.POINTER(mla_kv_view),
                                i32, i32, P, P, i32, ctypes.c_float, i32, P, P, ctypes.c_size_t, P]
    L.mla_attention.restype = st
    L.dsa_prefill_select_workspace_bytes.argtypes = [i32, i32, i32]
    L.dsa_prefill_select_workspace_bytes.restype = ctypes.c_size_t
    L.dsa_prefill_select.argtypes = [P, P, i32, ctypes.POINTER(mla_kv_view), i32, i32, i32, P, P, P, P,
                                     ctypes.c_size_t, P]
    L.dsa_prefill_select.restype = st
    L.mla_absorbed_decode_q.argtypes = [P, P, ctypes.c_int, ctypes.POINTER(mla_qweights), ctypes.POINTER(mla_dims), i32,
                                        ctypes.POINTER(mla_kv_view), P, P, i32, ctypes.c_float, P, P, ctypes.c_size_t, P]
    L.mla_absorbed_decode_q.restype = st
    L.mla_dsa_decode_q.argtypes = [P, P, ctypes.c_int, ctypes.c_double, P, P, i32, ctypes.POINTER(mla_qweights),
                                   ctypes.POINTER(mla_dims), i32, ctypes.POINTER(mla_kv_view), i64, i32, ctypes.c_float,
                                   P, P, P, P, P, ctypes.c_size_t, P]
    L.mla_dsa_decode_q.restype = st
    L.mla_status_string.argtypes = [ctypes.c_int]
    L.mla_status_string.restype = ctypes.c_char_p
    L.mla_last_error.argtypes = []
    L.mla_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def mla_status_string(status: int) -> str:
    return lib().mla_status_string(int(status)).decode()


def mla_last_error() -> str:
    return lib().mla_last_error().decode()


def _check(status: int) -> None:
    if status != MLA_OK:
        raise MlaError(status, f"{mla_status_string(status)}: {mla_last_error()}")


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MLA_FP32
    if t.dtype == torch.bfloat16:
        return MLA_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dev(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must live on the GPU")


def _contig(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


class mla_qweights(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("format", ctypes.c_int32)]


class KvCache:
    """Caller-owned compressed KV pools plus their layout (maps to ``mla_kv_view``).

    lc: [rows, kv_lora] and rc: [rows, qk_rope] (float32 or bfloat16); ic: [rows, index_hd]
    float32 or None.  Contiguous layout: token t of sequence b is row b*seq_stride + t.
    Paged layout: block_table int32 [B, max_blocks], row = block_table[b, t//bs]*bs + t%bs.
    seq_len: int32 [B] on the GPU (tokens cached including the query's own).
    ic_layout: MLA_IC_ROWS (ic row-major) or MLA_IC_TILE64 (ic holds the same rows in aligned
    64-row tiles, dims-major in quads of 4; see synth.tile_index_keys)."""

    def __init__(self, lc, rc, ic=None, *, seq_len=None, max_seq_len: int, block_table=None,
                 block_size: int = 0, seq_stride: int = 0, ic_layout: int = 0):
        _dev(lc, rc, ic, seq_len, block_table)
        _contig(lc, rc, ic, seq_len, block_table)
        if seq_len is not None and seq_len.dtype != torch.int32:
            raise TypeError("seq_len must be int32")
        if block_table is not None and block_table.dtype != torch.int32:
            raise TypeError("block_table must be int32")
        if ic is not None and ic.dtype != torch.float32:
            raise TypeError("ic must be float32")
        self.lc, self.rc, self.ic = lc, rc, ic
        self.seq_len, self.block_table = seq_len, block_table
        v = mla_kv_view()
        v.lc, v.rc, v.ic = lc.data_ptr(), rc.data_ptr(), (ic.data_ptr() if ic is not None else None)
        v.rows = lc.shape[0]
        v.kv_dtype = _dt(lc)
        v.index_hd = ic.shape[1] if ic is not None else 0
        v.block_table = block_table.data_ptr() if block_table is not None else None
        v.block_size = block_size
        v.max_blocks = block_table.shape[1] if block_table is not None else 0
        v.seq_stride = seq_stride
        v.seq_len = seq_len.data_ptr() if seq_len is not None else None
        v.max_seq_len = max_seq_len
        v.ic_layout = ic_layout
        for t in (rc, ic):
            if t is not None and t.shape[0] != lc.shape[0]:
                raise ValueError("lc, rc and ic must have the same number of rows")
        self.view = v


def mla_rope_interleave(x: torch.Tensor, pos: torch.Tensor, rope_off: int, rope_dim: int,
                        theta: float = 10000.0) -> torch.Tensor:
    """In-place interleaved partial RoPE on x [n_tok, n_heads, head_dim] (last dim unit
    stride); pos int32 [n_tok].  Returns x."""
    _dev(x, pos)
    if x.dim() != 3 or x.stride(2) != 1:
        raise ValueError("x must be [n_tok, n_heads, head_dim] with a unit-stride last dim")
    if pos.dtype != torch.int32 or pos.shape != (x.shape[0],) or not pos.is_contiguous():
        raise ValueError("pos must be contiguous int32 [n_tok]")
    if rope_off + rope_dim > x.shape[2]:
        raise ValueError("rope_off + rope_dim exceeds head_dim")
    _check(lib().mla_rope_interleave(_ptr(x), _dt(x), x.shape[0], x.shape[1], x.stride(0), x.stride(1),
                                     rope_off, rope_dim, _ptr(pos), float(theta), _stream(x.device)))
    return x


def mla_cache_write(comp: torch.Tensor, seq: torch.Tensor, pos: torch.Tensor, kv: KvCache, n_seq: int,
                    ik: Optional[torch.Tensor] = None, kv_gain: Optional[torch.Tensor] = None,
                    ix_gamma: Optional[torch.Tensor] = None, ix_beta: Optional[torch.Tensor] = None,
                    ix_rope_off: int = 0, ix_rope_dim: int = 0, eps_kv: float = 1e-6, eps_ix: float = 1e-6,
                    theta: float = 10000.0) -> None:
    """Write new tokens into the cache pools of kv: comp [n, kv_lora + qk_rope] (the kv_a output) and
    optionally ik [n, index_hd] (the indexer key projection), same dtype; seq / pos int32 [n]."""
    _dev(comp, seq, pos, ik, kv_gain, ix_gamma, ix_beta)
    _contig(comp, seq, pos, ik, kv_gain, ix_gamma, ix_beta)
    n = comp.shape[0]
    L, rope = kv.lc.shape[1], kv.rc.shape[1]
    if comp.dim() != 2 or comp.shape[1] != L + rope:
        raise ValueError("comp must be [n, kv_lora + qk_rope]")
    if seq.dtype != torch.int32 or pos.dtype != torch.int32 or seq.shape != (n,) or pos.shape != (n,):
        raise ValueError("seq and pos must be int32 [n]")
    if ik is not None and (ik.dtype != comp.dtype or kv.ic is None or ik.shape != (n, kv.ic.shape[1])):
        raise ValueError("ik must be [n, index_hd] in comp's dtype, with an indexer pool in kv")
    for g in (kv_gain, ix_gamma, ix_beta):
        if g is not None and g.dtype != torch.float32:
            raise TypeError("gains must be float32")
    _check(lib().mla_cache_write(_ptr(comp), _ptr(ik), _dt(comp), n, _ptr(seq), _ptr(pos), n_seq, L, rope,
                                 _ptr(kv_gain), _ptr(ix_gamma), _ptr(ix_beta), ix_rope_off, ix_rope_dim,
                                 float(eps_kv), float(eps_ix), float(theta), ctypes.byref(kv.view),
                                 _stream(comp.device)))


def dsa_index_scores(q_idx: torch.Tensor, w_idx: torch.Tensor, kv: KvCache, t_max: int,
                     scores: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Indexer scores [B, t_max] float32 (fixed-order fp32; -inf beyond seq_len)."""
    _dev(q_idx, w_idx, scores)
    _contig(q_idx, w_idx, scores)
    B, n_ih, hd = q_idx.shape
    if w_idx.shape != (B, n_ih) or q_idx.dtype != torch.float32 or w_idx.dtype != torch.float32:
        raise ValueError("q_idx [B, n_ih, hd] and w_idx [B, n_ih] must be float32")
    if kv.ic is None or kv.ic.shape[1] != hd:
        raise ValueError("kv.ic width must equal q_idx's last dim")
    if scores is None:
        scores = torch.empty((B, t_max), dtype=torch.float32, device=q_idx.device)
    elif scores.shape != (B, t_max) or scores.dtype != torch.float32:
        raise ValueError("scores must be float32 [B, t_max]")
    _check(lib().dsa_index_scores(_ptr(q_idx), _ptr(w_idx), B, n_ih, ctypes.byref(kv.view), t_max,
                                  _ptr(scores), _stream(q_idx.device)))
    return scores


def dsa_topk_workspace_bytes(B: int, t_max: int, k: int) -> int:
    return int(lib().dsa_topk_workspace_bytes(B, t_max, k))


def dsa_topk_select(scores: torch.Tensor, n_valid: torch.Tensor, k: int, sel: Optional[torch.Tensor] = None,
                    nsel: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None):
    """Top-k positions per row (score desc, position asc), ascending; returns (sel [B, k]
    int32 with -1 padding, nsel [B] int32)."""
    _dev(scores, n_valid, sel, nsel, ws)
    _contig(scores, n_valid, sel, nsel, ws)
    B, t_max = scores.shape
    if scores.dtype != torch.float32 or n_valid.dtype != torch.int32 or n_valid.shape != (B,):
        raise ValueError("scores float32 [B, t_max], n_valid int32 [B]")
    dev = scores.device
    sel = torch.empty((B, k), dtype=torch.int32, device=dev) if sel is None else sel
    nsel = torch.empty((B,), dtype=torch.int32, device=dev) if nsel is None else nsel
    need = dsa_topk_workspace_bytes(B, t_max, k)
    if ws is None and need:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    _check(lib().dsa_topk_select(_ptr(scores), B, t_max, _ptr(n_valid), k, _ptr(sel), _ptr(nsel), _ptr(ws),
                                 ws.numel() * ws.element_size() if ws is not None else 0, _stream(dev)))
    return sel, nsel


def dsa_index_select_workspace_bytes(B: int, t_max: int, k: int) -> int:
    return int(lib().dsa_index_select_workspace_bytes(B, t_max, k))


def dsa_index_select(q_idx: torch.Tensor, w_idx: torch.Tensor, kv: KvCache, t_max: int, k: int,
                     scores: Optional[torch.Tensor] = None, sel: Optional[torch.Tensor] = None,
                     nsel: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None):
    """Indexer scores and the top-k of every row in one call; returns (scores [B, t_max],
    sel [B, k] int32 with -1 padding, nsel [B] int32), equal to dsa_index_scores followed
    by dsa_topk_select with n_valid = the rows' causal lengths."""
    _dev(q_idx, w_idx, scores, sel, nsel, ws)
    _contig(q_idx, w_idx, scores, sel, nsel, ws)
    B, n_ih, hd = q_idx.shape
    if w_idx.shape != (B, n_ih) or q_idx.dtype != torch.float32 or w_idx.dtype != torch.float32:
        raise ValueError("q_idx [B, n_ih, hd] and w_idx [B, n_ih] must be float32")
    if kv.ic is None or kv.ic.shape[1] != hd:
        raise ValueError("kv.ic width must equal q_idx's last dim")
    dev = q_idx.device
    if scores is None:
        scores = torch.empty((B, t_max), dtype=torch.float32, device=dev)
    elif scores.shape != (B, t_max) or scores.dtype != torch.float32:
        raise ValueError("scores must be float32 [B, t_max]")
    sel = torch.empty((B, k), dtype=torch.int32, device=dev) if sel is None else sel
    nsel = torch.empty((B,), dtype=torch.int32, device=dev) if nsel is None else nsel
    need = dsa_index_select_workspace_bytes(B, t_max, k)
    if ws is None and need:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    _check(lib().dsa_index_select(_ptr(q_idx), _ptr(w_idx), B, n_ih, ctypes.byref(kv.view), t_max, k, _ptr(scores),
                                  _ptr(sel), _ptr(nsel), _ptr(ws), ws.numel() * ws.element_size() if ws is not None else 0,
                                  _stream(dev)))
    return scores, sel, nsel


def _dims(H: int, nope: int, rope: int, v: int, L: int) -> mla_dims:
    d = mla_dims()
    d.n_heads, d.qk_nope, d.qk_rope, d.v_head, d.kv_lora = H, nope, rope, v, L
    return d


def mla_decode_workspace_bytes(H: int, nope: int, rope: int, v: int, L: int, B: int, max_keys: int) -> int:
    return int(lib().mla_decode_workspace_bytes(ctypes.byref(_dims(H, nope, rope, v, L)), B, max_keys))


def _decode_args(q_nope, q_rope, kv_b, kv, sel, nsel):
    B, H, nope = q_nope.shape
    rope = q_rope.shape[2]
    L = kv_b.shape[1]
    if q_rope.shape[:2] != (B, H) or kv_b.shape[0] % H:
        raise ValueError("shape mismatch between q_nope, q_rope and kv_b")
    v = kv_b.shape[0] // H - nope
    if kv.lc.shape[1] != L or kv.rc.shape[1] != rope:
        raise ValueError("cache widths must match kv_lora and qk_rope")
    sel_stride = 0
    if sel is not None:
        if sel.dtype != torch.int32 or sel.dim() != 2 or sel.shape[0] != B or nsel is None:
            raise ValueError("sel must be int32 [B, k] with nsel int32 [B]")
        if nsel.dtype != torch.int32 or nsel.shape != (B,):
            raise ValueError("nsel must be int32 [B]")
        sel_stride = sel.shape[1]
    max_keys = sel_stride if sel is not None else kv.view.max_seq_len
    return B, H, nope, rope, v, L, _dims(H, nope, rope, v, L), sel_stride, max_keys


def mla_absorbed_decode(q_nope: torch.Tensor, q_rope: torch.Tensor, kv_b: torch.Tensor, kv: KvCache,
                        sm_scale: float, sel: Optional[torch.Tensor] = None, nsel: Optional[torch.Tensor] = None,
                        out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Absorbed MLA decode: q_nope [B, H, nope], q_rope [B, H, rope] (rotated),
    kv_b [H*(nope+v), L]; sel int32 [B, k] / nsel int32 [B] or None for dense causal.
    Returns out [B, H, v] float32."""
    _dev(q_nope, q_rope, kv_b, sel, nsel, out, ws)
    _contig(q_nope, q_rope, kv_b, sel, nsel, out, ws)
    B, H, nope, rope, v, L, d, sel_stride, max_keys = _decode_args(q_nope, q_rope, kv_b, kv, sel, nsel)
    if out is None:
        out = torch.empty((B, H, v), dtype=torch.float32, device=q_nope.device)
    need = int(lib().mla_decode_workspace_bytes(ctypes.byref(d), B, max_keys))
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q_nope.device)
    _check(lib().mla_absorbed_decode(_ptr(q_nope), _ptr(q_rope), _dt(q_nope), _ptr(kv_b), _dt(kv_b),
                                     ctypes.byref(d), B, ctypes.byref(kv.view), _ptr(sel), _ptr(nsel),
                                     sel_stride, float(sm_scale), _ptr(out), _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream(q_nope.device)))
    return out


def mla_decode_absorb(q_nope: torch.Tensor, kv_b: torch.Tensor, ws: torch.Tensor, qk_rope: int = 64) -> None:
    """First step of the absorbed decode, q_abs = W_UK^T q_nope, written into ws for a later
    mla_decode_attend on the same ws (uint8 device tensor of at least
    mla_decode_workspace_bytes(...) bytes).  q_nope [B, H, nope], kv_b [H*(nope+v), L]."""
    _dev(q_nope, kv_b, ws)
    _contig(q_nope, kv_b, ws)
    B, H, nope = q_nope.shape
    if kv_b.shape[0] % H:
        raise ValueError("kv_b rows must be a multiple of the head count")
    d = _dims(H, nope, qk_rope, kv_b.shape[0] // H - nope, kv_b.shape[1])
    _check(lib().mla_decode_absorb(_ptr(q_nope), _dt(q_nope), _ptr(kv_b), _dt(kv_b), ctypes.byref(d), B, _ptr(ws),
                                   ws.numel() * ws.element_size(), _stream(q_nope.device)))


def mla_decode_attend(q_rope: torch.Tensor, kv_b: torch.Tensor, kv: KvCache, qk_nope: int, sm_scale: float,
                      ws: torch.Tensor, sel: Optional[torch.Tensor] = None, nsel: Optional[torch.Tensor] = None,
                      out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Second step of the absorbed decode: scores, softmax, latent accumulation and W_UV,
    reading q_abs from ws (written by mla_decode_absorb).  Returns out [B, H, v] float32."""
    _dev(q_rope, kv_b, sel, nsel, out, ws)
    _contig(q_rope, kv_b, sel, nsel, out, ws)
    B, H, _ = q_rope.shape
    shape_only = torch.empty((B, H, qk_nope), dtype=q_rope.dtype, device="meta")
    B, H, nope, rope, v, L, d, sel_stride, max_keys = _decode_args(shape_only, q_rope, kv_b, kv, sel, nsel)
    if out is None:
        out = torch.empty((B, H, v), dtype=torch.float32, device=q_rope.device)
    _check(lib().mla_decode_attend(_ptr(q_rope), _dt(q_rope), _ptr(kv_b), _dt(kv_b), ctypes.byref(d), B,
                                   ctypes.byref(kv.view), _ptr(sel), _ptr(nsel), sel_stride, float(sm_scale),
                                   _ptr(out), _ptr(ws), ws.numel() * ws.element_size(), _stream(q_rope.device)))
    return out


def mla_dsa_decode_workspace_bytes(H: int, nope: int, rope: int, v: int, L: int, B: int, t_max: int, k: int) -> int:
    return int(lib().mla_dsa_decode_workspace_bytes(ctypes.byref(_dims(H, nope, rope, v, L)), B, t_max, k))


def mla_dsa_decode(q_nope: torch.Tensor, q_rope: torch.Tensor, q_idx: torch.Tensor, w_idx: torch.Tensor,
                   kv_b: torch.Tensor, kv: KvCache, t_max: int, k: int, sm_scale: float, theta: float = 10000.0,
                   scores: Optional[torch.Tensor] = None, sel: Optional[torch.Tensor] = None,
                   nsel: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                   ws: Optional[torch.Tensor] = None, noalloc: bool = False):
    """The whole decode step: RoPE of q_rope [B, H, rope] (before rotation; not modified) at
    position seq_len - 1, indexer scores and top-k selection, absorbed attention over the
    selected keys.  Returns (out [B, H, v] float32, scores [B, t_max], sel [B, k], nsel [B]).
    noalloc=True calls mla_dsa_decode_noalloc (the library's static scratch; no ws)."""
    if noalloc and ws is not None:
        raise ValueError("noalloc takes no workspace")
    _dev(q_nope, q_rope, q_idx, w_idx, kv_b, scores, sel, nsel, out, ws)
    _contig(q_nope, q_rope, q_idx, w_idx, kv_b, scores, sel, nsel, out, ws)
    B, H, nope = q_nope.shape
    rope = q_rope.shape[2]
    L = kv_b.shape[1]
    if q_rope.shape[:2] != (B, H) or kv_b.shape[0] % H:
        raise ValueError("shape mismatch between q_nope, q_rope and kv_b")
    v = kv_b.shape[0] // H - nope
    Bi, n_ih, hd = q_idx.shape
    if Bi != B or w_idx.shape != (B, n_ih) or q_idx.dtype != torch.float32 or w_idx.dtype != torch.float32:
        raise ValueError("q_idx [B, n_ih, hd] and w_idx [B, n_ih] must be float32")
    if kv.ic is None or kv.ic.shape[1] != hd:
        raise ValueError("kv.ic width must equal q_idx's last dim")
    if kv.lc.shape[1] != L or kv.rc.shape[1] != rope:
        raise ValueError("cache widths must match kv_lora and qk_rope")
    dev = q_nope.device
    if scores is None:
        scores = torch.empty((B, t_max), dtype=torch.float32, device=dev)
    elif scores.shape != (B, t_max) or scores.dtype != torch.float32:
        raise ValueError("scores must be float32 [B, t_max]")
    sel = torch.empty((B, k), dtype=torch.int32, device=dev) if sel is None else sel
    nsel = torch.empty((B,), dtype=torch.int32, device=dev) if nsel is None else nsel
    if sel.shape != (B, k) or sel.dtype != torch.int32 or nsel.shape != (B,) or nsel.dtype != torch.int32:
        raise ValueError("sel must be int32 [B, k] and nsel int32 [B]")
    if out is None:
        out = torch.empty((B, H, v), dtype=torch.float32, device=dev)
    d = _dims(H, nope, rope, v, L)
    if noalloc:
        _check(lib().mla_dsa_decode_noalloc(_ptr(q_nope), _ptr(q_rope), _dt(q_nope), float(theta), _ptr(q_idx),
                                            _ptr(w_idx), n_ih, _ptr(kv_b), _dt(kv_b), ctypes.byref(d), B,
                                            ctypes.byref(kv.view), t_max, k, float(sm_scale), _ptr(scores),
                                            _ptr(sel), _ptr(nsel), _ptr(out), _stream(dev)))
        return out, scores, sel, nsel
    need = int(lib().mla_dsa_decode_workspace_bytes(ctypes.byref(d), B, t_max, k))
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check(lib().mla_dsa_decode(_ptr(q_nope), _ptr(q_rope), _dt(q_nope), float(theta), _ptr(q_idx), _ptr(w_idx), n_ih,
                                _ptr(kv_b), _dt(kv_b), ctypes.byref(d), B, ctypes.byref(kv.view), t_max, k,
                                float(sm_scale), _ptr(scores), _ptr(sel), _ptr(nsel), _ptr(out), _ptr(ws),
                                ws.numel() * ws.element_size(), _stream(dev)))
    return out, scores, sel, nsel


def mla_dsa_decode_shared(q_nope: torch.Tensor, q_rope: torch.Tensor, kv_b: torch.Tensor, kv: KvCache,
                          sel: torch.Tensor, nsel: torch.Tensor, sm_scale: float, theta: float = 10000.0,
                          out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The decode step of a DSA-shared layer: RoPE of q_rope [B, H, rope] (not modified) at seq_len - 1
    and absorbed attention over the given selection sel [B, k] / nsel [B] (an earlier layer's).
    Returns out [B, H, v] float32."""
    _dev(q_nope, q_rope, kv_b, sel, nsel, out, ws)
    _contig(q_nope, q_rope, kv_b, sel, nsel, out, ws)
    B, H, nope = q_nope.shape
    rope = q_rope.shape[2]
    L = kv_b.shape[1]
    if q_rope.shape[:2] != (B, H) or kv_b.shape[0] % H:
        raise ValueError("shape mismatch between q_nope, q_rope and kv_b")
    v = kv_b.shape[0] // H - nope
    if sel.dtype != torch.int32 or nsel.dtype != torch.int32 or sel.dim() != 2 or sel.shape[0] != B \
            or nsel.shape != (B,):
        raise ValueError("sel must be int32 [B, k] and nsel int32 [B]")
    k = sel.shape[1]
    if out is None:
        out = torch.empty((B, H, v), dtype=torch.float32, device=q_nope.device)
    d = _dims(H, nope, rope, v, L)
    if ws is None:
        need = int(lib().mla_dsa_decode_shared_workspace_bytes(ctypes.byref(d), B, k))
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q_nope.device)
    _check(lib().mla_dsa_decode_shared(_ptr(q_nope), _ptr(q_rope), _dt(q_nope), float(theta), _ptr(kv_b), _dt(kv_b),
                                       ctypes.byref(d), B, ctypes.byref(kv.view), _ptr(sel), _ptr(nsel), k,
                                       float(sm_scale), _ptr(out), _ptr(ws), ws.numel() * ws.element_size(),
                                       _stream(q_nope.device)))
    return out


def mla_prefill_workspace_bytes(H: int, nope: int, rope: int, v: int, L: int, S: int, T: int) -> int:
    return int(lib().mla_prefill_workspace_bytes(ctypes.byref(_dims(H, nope, rope, v, L)), S, T))


def mla_prefill_nonabsorbed(q: torch.Tensor, kv_b: torch.Tensor, kv: KvCache, qk_nope: int, pos_base: int,
                            sm_scale: float, out_dtype: torch.dtype = torch.float32,
                            out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Non-absorbed causal prefill: q [S, H, nope+rope] (rotated tail), kv_b
    [H*(nope+v), L]; query i at position pos_base+i.  Returns out [S, H, v]."""
    _dev(q, kv_b, out, ws)
    _contig(q, kv_b, out, ws)
    S, H, qh = q.shape
    rope = qh - qk_nope
    L = kv_b.shape[1]
    if kv_b.shape[0] % H:
        raise ValueError("kv_b rows must be a multiple of the head count")
    v = kv_b.shape[0] // H - qk_nope
    d = _dims(H, qk_nope, rope, v, L)
    if out is None:
        out = torch.empty((S, H, v), dtype=out_dtype, device=q.device)
    need = int(lib().mla_prefill_workspace_bytes(ctypes.byref(d), S, pos_base + S))
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(lib().mla_prefill_nonabsorbed(_ptr(q), _dt(q), _ptr(kv_b), _dt(kv_b), ctypes.byref(d),
                                         ctypes.byref(kv.view), S, pos_base, float(sm_scale), _ptr(out),
                                         _dt(out), _ptr(ws), ws.numel() * ws.element_size(),
                                         _stream(q.device)))
    return out


def mla_attention_absorbs(S: int, g_absorb: int = -1) -> bool:
    """True when mla_attention takes the absorbed path for S queries under g_absorb."""
    return bool(lib().mla_attention_absorbs(int(S), int(g_absorb)))


def mla_attention(q: torch.Tensor, kv_b: torch.Tensor, kv: KvCache, qk_nope: int, pos_base: int, sm_scale: float,
                  g_absorb: int = -1, sel: Optional[torch.Tensor] = None, nsel: Optional[torch.Tensor] = None,
                  out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """S queries q [S, H, nope+rope] (rotated tail) of one sequence at positions pos_base .. pos_base+S-1,
    on the path g_absorb picks (-1: absorbed when S <= 4; 0: never; 1: always), optionally restricted to
    per-query selections sel [S, k] / nsel [S].  Returns out [S, H, v] float32."""
    _dev(q, kv_b, sel, nsel, out, ws)
    _contig(q, kv_b, sel, nsel, out, ws)
    S, H, qh = q.shape
    rope = qh - qk_nope
    L = kv_b.shape[1]
    if kv_b.shape[0] % H:
        raise ValueError("kv_b rows must be a multiple of the head count")
    v = kv_b.shape[0] // H - qk_nope
    sel_stride = 0
    if sel is not None:
        if sel.dtype != torch.int32 or sel.dim() != 2 or sel.shape[0] != S or nsel is None \
                or nsel.dtype != torch.int32 or nsel.shape != (S,):
            raise ValueError("sel must be int32 [S, k] with nsel int32 [S]")
        sel_stride = sel.shape[1]
    d = _dims(H, qk_nope, rope, v, L)
    if out is None:
        out = torch.empty((S, H, v), dtype=torch.float32, device=q.device)
    if ws is None:
        need = int(lib().mla_attention_workspace_bytes(ctypes.byref(d), S, pos_base, sel_stride, g_absorb))
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(lib().mla_attention(_ptr(q), _dt(q), _ptr(kv_b), _dt(kv_b), ctypes.byref(d), ctypes.byref(kv.view), S,
                               pos_base, _ptr(sel), _ptr(nsel), sel_stride, float(sm_scale), int(g_absorb), _ptr(out),
                               _ptr(ws), ws.numel() * ws.element_size(), _stream(q.device)))
    return out


def dsa_prefill_select(q_idx: torch.Tensor, w_idx: torch.Tensor, kv: KvCache, pos_base: int, k: int,
                       scores: Optional[torch.Tensor] = None, sel: Optional[torch.Tensor] = None,
                       nsel: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None):
    """Per-query DSA selection of S prefill queries (query i at pos_base + i): q_idx [S, n_ih, hd],
    w_idx [S, n_ih] float32.  Returns (scores [S, pos_base+S], sel [S, k], nsel [S])."""
    _dev(q_idx, w_idx, scores, sel, nsel, ws)
    _contig(q_idx, w_idx, scores, sel, nsel, ws)
    S, n_ih, hd = q_idx.shape
    if w_idx.shape != (S, n_ih) or q_idx.dtype != torch.float32 or w_idx.dtype != torch.float32:
        raise ValueError("q_idx [S, n_ih, hd] and w_idx [S, n_ih] must be float32")
    if kv.ic is None or kv.ic.shape[1] != hd:
        raise ValueError("kv.ic width must equal q_idx's last dim")
    T = pos_base + S
    dev = q_idx.device
    scores = torch.empty((S, T), dtype=torch.float32, device=dev) if scores is None else scores
    sel = torch.empty((S, k), dtype=torch.int32, device=dev) if sel is None else sel
    nsel = torch.empty((S,), dtype=torch.int32, device=dev) if nsel is None else nsel
    if scores.shape != (S, T) or sel.shape != (S, k) or nsel.shape != (S,):
        raise ValueError("scores [S, pos_base+S], sel [S, k], nsel [S]")
    if ws is None:
        ws = torch.empty(max(int(lib().dsa_prefill_select_workspace_bytes(S, pos_base, k)), 1), dtype=torch.uint8,
                         device=dev)
    _check(lib().dsa_prefill_select(_ptr(q_idx), _ptr(w_idx), n_ih, ctypes.byref(kv.view), S, pos_base, k, _ptr(scores),
                                    _ptr(sel), _ptr(nsel), _ptr(ws), ws.numel() * ws.element_size(), _stream(dev)))
    return scores, sel, nsel


def _qweights(codes: torch.Tensor, scales: torch.Tensor, fmt: int):
    _dev(codes, scales)
    _contig(codes, scales)
    if codes.dtype != torch.uint8:
        raise TypeError("codes must be uint8")
    if fmt in (MLA_Q_FP8_E4M3, MLA_Q_INT8) and scales.dtype != torch.float32:
        raise TypeError("FP8 / INT8 scales are float32, one per row")
    if fmt == MLA_Q_MXFP4 and scales.dtype != torch.uint8:
        raise TypeError("MXFP4 scales are E8M0 bytes")
    w = mla_qweights()
    w.codes, w.scales, w.format = codes.data_ptr(), scales.data_ptr(), int(fmt)
    return w


def mla_absorbed_decode_q(q_nope: torch.Tensor, q_rope: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor,
                          fmt: int, kv: KvCache, sm_scale: float, sel: Optional[torch.Tensor] = None,
                          nsel: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                          ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Absorbed decode with a quantized kv_b (codes uint8 [N, kv_lora] for FP8 / INT8 or [N, kv_lora/2] for
    MXFP4; scales float32 [N] or E8M0 uint8 [N, kv_lora/32]; N = H * (qk_nope + v_head)).  Returns out
    [B, H, v] float32."""
    _dev(q_nope, q_rope, sel, nsel, out, ws)
    _contig(q_nope, q_rope, sel, nsel, out, ws)
    B, H, nope = q_nope.shape
    rope = q_rope.shape[2]
    L = kv.lc.shape[1]
    if q_rope.shape[:2] != (B, H) or codes.shape[0] % H or kv.rc.shape[1] != rope:
        raise ValueError("shape mismatch between q_nope, q_rope, the cache and the codes")
    v = codes.shape[0] // H - nope
    stride = 0
    if sel is not None:
        if sel.dtype != torch.int32 or sel.dim() != 2 or sel.shape[0] != B or nsel is None \
                or nsel.dtype != torch.int32 or nsel.shape != (B,):
            raise ValueError("sel must be int32 [B, k] with nsel int32 [B]")
        stride = sel.shape[1]
    sel_p, nsel_p = _ptr(sel), _ptr(nsel)
    w = _qweights(codes, scales, fmt)
    d = _dims(H, nope, rope, v, L)
    if out is None:
        out = torch.empty((B, H, v), dtype=torch.float32, device=q_nope.device)
    max_keys = stride if sel is not None else kv.view.max_seq_len
    if ws is None:
        need = int(lib().mla_decode_workspace_bytes(ctypes.byref(d), B, max_keys))
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q_nope.device)
    _check(lib().mla_absorbed_decode_q(_ptr(q_nope), _ptr(q_rope), _dt(q_nope), ctypes.byref(w), ctypes.byref(d), B,
                                       ctypes.byref(kv.view), sel_p, nsel_p, stride, float(sm_scale), _ptr(out),
                                       _ptr(ws), ws.numel() * ws.element_size(), _stream(q_nope.device)))
    return out


def mla_dsa_decode_q(q_nope: torch.Tensor, q_rope: torch.Tensor, q_idx: torch.Tensor, w_idx: torch.Tensor,
                     codes: torch.Tensor, scales: torch.Tensor, fmt: int, kv: KvCache, t_max: int, k: int,
                     sm_scale: float, theta: float = 10000.0, scores: Optional[torch.Tensor] = None,
                     sel: Optional[torch.Tensor] = None, nsel: Optional[torch.Tensor] = None,
                     out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None):
    """mla_dsa_decode with a quantized kv_b.  Returns (out, scores, sel, nsel)."""
    _dev(q_nope, q_rope, q_idx, w_idx, scores, sel, nsel, out, ws)
    _contig(q_nope, q_rope, q_idx, w_idx, scores, sel, nsel, out, ws)
    B, H, nope = q_nope.shape
    rope = q_rope.shape[2]
    L = kv.lc.shape[1]
    v = codes.shape[0] // H - nope
    n_ih = q_idx.shape[1]
    w = _qweights(codes, scales, fmt)
    dev = q_nope.device
    scores = torch.empty((B, t_max), dtype=torch.float32, device=dev) if scores is None else scores
    sel = torch.empty((B, k), dtype=torch.int32, device=dev) if sel is None else sel
    nsel = torch.empty((B,), dtype=torch.int32, device=dev) if nsel is None else nsel
    out = torch.empty((B, H, v), dtype=torch.float32, device=dev) if out is None else out
    d = _dims(H, nope, rope, v, L)
    if ws is None:
        need = int(lib().mla_dsa_decode_workspace_bytes(ctypes.byref(d), B, t_max, k))
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check(lib().mla_dsa_decode_q(_ptr(q_nope), _ptr(q_rope), _dt(q_nope), float(theta), _ptr(q_idx), _ptr(w_idx), n_ih,
                                  ctypes.byref(w), ctypes.byref(d), B, ctypes.byref(kv.view), t_max, k,
                                  float(sm_scale), _ptr(scores), _ptr(sel), _ptr(nsel), _ptr(out), _ptr(ws),
                                  ws.numel() * ws.element_size(), _stream(dev)))
    return out, scores, sel, nsel
