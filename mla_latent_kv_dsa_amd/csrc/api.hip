// api.hip -- the extern "C" entry points of libmla_dsa.so: argument validation (before any
// HIP call), workspace queries, and dispatch to the kernel launchers.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "common.h"

namespace mla {

static thread_local char g_err[512];

void set_error(const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
}

mla_status fail(mla_status s, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

mla_status check_launch(const char *what)
{
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return MLA_OK;
}

static bool valid_dtype(mla_dtype d) { return d == MLA_FP32 || d == MLA_BF16; }

// Host-side checks of a KV view.  need_lc_rc / need_ic select which pools must exist.
static mla_status check_view(const mla_kv_view *kv, int32_t B, bool need_lc_rc, bool need_ic,
                             bool need_seq_len)
{
    if (!kv) return fail(MLA_ERR_ARG, "kv view is NULL");
    if (need_lc_rc && (!kv->lc || !kv->rc)) return fail(MLA_ERR_ARG, "kv->lc / kv->rc is NULL");
    if (need_ic && !kv->ic) return fail(MLA_ERR_ARG, "kv->ic is NULL");
    if (!valid_dtype(kv->kv_dtype)) return fail(MLA_ERR_ARG, "kv->kv_dtype invalid");
    if (kv->rows <= 0) return fail(MLA_ERR_ARG, "kv->rows must be positive");
    if (need_seq_len && !kv->seq_len) return fail(MLA_ERR_ARG, "kv->seq_len is NULL");
    if (kv->max_seq_len < 0) return fail(MLA_ERR_ARG, "kv->max_seq_len negative");
    if (kv->max_seq_len >= ((int64_t)1 << 31)) return fail(MLA_ERR_UNSUPPORTED, "kv->max_seq_len >= 2^31");
    if (kv->ic_layout != MLA_IC_ROWS && kv->ic_layout != MLA_IC_TILE64) return fail(MLA_ERR_ARG, "kv->ic_layout invalid");
    if (kv->ic_layout == MLA_IC_TILE64 && kv->ic) {
        if (kv->rows % 64 != 0) return fail(MLA_ERR_ARG, "tiled indexer pool: rows must be a multiple of 64");
        if (kv->index_hd % 4 != 0) return fail(MLA_ERR_ARG, "tiled indexer pool: index_hd must be a multiple of 4");
        if (kv->block_table && kv->block_size % 64 != 0)
            return fail(MLA_ERR_ARG, "tiled indexer pool: block_size must be a multiple of 64");
        if (!kv->block_table && B > 1 && kv->seq_stride % 64 != 0)
            return fail(MLA_ERR_ARG, "tiled indexer pool: seq_stride must be a multiple of 64");
    }
    if (kv->block_table) {
        if (kv->block_size <= 0 || kv->max_blocks <= 0)
            return fail(MLA_ERR_ARG, "paged view needs block_size > 0 and max_blocks > 0");
        if ((int64_t)kv->max_blocks * kv->block_size < kv->max_seq_len)
            return fail(MLA_ERR_ARG, "max_blocks * block_size (%lld) < max_seq_len (%lld)",
                        (long long)kv->max_blocks * kv->block_size, (long long)kv->max_seq_len);
        if (kv->rows % kv->block_size != 0)
            return fail(MLA_ERR_ARG, "paged pools must hold whole blocks (rows %% block_size != 0)");
    } else {
        if (kv->seq_stride < 0) return fail(MLA_ERR_ARG, "kv->seq_stride negative");
        if (B > 1 && kv->seq_stride < kv->max_seq_len)
            return fail(MLA_ERR_ARG, "contiguous view: seq_stride < max_seq_len overlaps sequences");
        if ((int64_t)(B > 0 ? B - 1 : 0) * kv->seq_stride + kv->max_seq_len > kv->rows)
            return fail(MLA_ERR_ARG, "contiguous view: (B-1)*seq_stride + max_seq_len > rows");
    }
    return MLA_OK;
}

static mla_status check_dims(const mla_dims *d)
{
    if (!d) return fail(MLA_ERR_ARG, "dims is NULL");
    if (d->n_heads <= 0 || d->qk_nope <= 0 || d->qk_rope <= 0 || d->v_head <= 0 || d->kv_lora <= 0)
        return fail(MLA_ERR_ARG, "dims must be positive");
    if (d->n_heads > 256 || d->qk_nope > 1024 || d->qk_rope > 512 || d->v_head > 1024 || d->kv_lora > 2048)
        return fail(MLA_ERR_UNSUPPORTED, "dims beyond the supported range "
                    "(n_heads<=256, qk_nope<=1024, qk_rope<=512, v_head<=1024, kv_lora<=2048)");
    return MLA_OK;
}

}  // namespace mla

using namespace mla;

extern "C" {

const char *mla_status_string(mla_status s)
{
    switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_ARG: return "MLA_ERR_ARG";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE";
    case MLA_ERR_HIP: return "MLA_ERR_HIP";
    }
    return "MLA_ERR_UNKNOWN";
}

const char *mla_last_error(void) { return g_err; }

mla_status mla_rope_interleave(void *x, mla_dtype dt, int64_t n_tok, int32_t n_heads,
                               int64_t tok_stride, int64_t head_stride, int32_t rope_off,
                               int32_t rope_dim, const int32_t *pos, double theta, void *stream)
{
    g_err[0] = 0;
    if (!valid_dtype(dt)) return fail(MLA_ERR_ARG, "rope: dtype invalid");
    if (n_tok < 0 || n_heads <= 0) return fail(MLA_ERR_ARG, "rope: n_tok < 0 or n_heads <= 0");
    if (rope_dim <= 0 || (rope_dim & 1)) return fail(MLA_ERR_ARG, "rope: rope_dim must be even and positive");
    if (rope_dim > 512) return fail(MLA_ERR_UNSUPPORTED, "rope: rope_dim > 512");
    if (rope_off < 0 || tok_stride < 0 || head_stride < 0) return fail(MLA_ERR_ARG, "rope: negative offset or stride");
    if (!(theta > 0.0) || !isfinite(theta)) return fail(MLA_ERR_ARG, "rope: theta must be positive and finite");
    if (n_tok == 0) return MLA_OK;
    if (!x || !pos) return fail(MLA_ERR_ARG, "rope: x or pos is NULL");
    if (n_heads > 1 && head_stride < rope_off + rope_dim)
        return fail(MLA_ERR_ARG, "rope: head_stride smaller than rope_off + rope_dim");
    if (n_tok > 1 && tok_stride < (int64_t)(n_heads - 1) * head_stride + rope_off + rope_dim)
        return fail(MLA_ERR_ARG, "rope: tok_stride overlaps tokens");
    return launch_rope(x, dt, n_tok, n_heads, tok_stride, head_stride, rope_off, rope_dim, pos, theta,
                       (hipStream_t)stream);
}

mla_status dsa_index_scores(const float *q_idx, const float *w_idx, int32_t B, int32_t n_ih,
                            const mla_kv_view *kv, int64_t t_max, float *scores, void *stream)
{
    g_err[0] = 0;
    if (B < 0 || t_max < 0) return fail(MLA_ERR_ARG, "index: B or t_max negative");
    if (n_ih <= 0) return fail(MLA_ERR_ARG, "index: n_ih must be positive");
    if (n_ih > 64) return fail(MLA_ERR_UNSUPPORTED, "index: n_ih > 64");
    mla_status st = check_view(kv, B, false, true, true);
    if (st) return st;
    if (kv->index_hd <= 0 || kv->index_hd % 4 != 0) return fail(MLA_ERR_ARG, "index: index_hd must be a positive multiple of 4");
    if (kv->index_hd > 256) return fail(MLA_ERR_UNSUPPORTED, "index: index_hd > 256");
    if (t_max >= ((int64_t)1 << 31)) return fail(MLA_ERR_UNSUPPORTED, "index: t_max >= 2^31");
    if (B == 0 || t_max == 0) return MLA_OK;
    if (!q_idx || !w_idx || !scores) return fail(MLA_ERR_ARG, "index: NULL tensor");
    KvView v = to_view(*kv);
    if (v.max_seq_len > t_max) v.max_seq_len = t_max;
    return launch_index_scores(q_idx, w_idx, B, n_ih, kv->index_hd, v, t_max, scores, nullptr, (hipStream_t)stream);
}

size_t dsa_topk_workspace_bytes(int32_t B, int64_t t_max, int32_t k)
{
    if (B <= 0 || t_max <= 0 || k <= 0) return 0;
    return topk_workspace_bytes(B, t_max, k);
}

mla_status dsa_topk_select(const float *scores, int32_t B, int64_t t_max, const int32_t *n_valid,
                           int32_t k, int32_t *sel, int32_t *nsel, void *ws, size_t ws_bytes,
                           void *stream)
{
    g_err[0] = 0;
    if (B < 0 || t_max < 0) return fail(MLA_ERR_ARG, "topk: B or t_max negative");
    if (k <= 0) return fail(MLA_ERR_ARG, "topk: k must be positive");
    if (k > 65536) return fail(MLA_ERR_UNSUPPORTED, "topk: k > 65536");
    if (t_max >= ((int64_t)1 << 31)) return fail(MLA_ERR_UNSUPPORTED, "topk: t_max >= 2^31");
    if (B == 0) return MLA_OK;
    if (!scores && t_max > 0) return fail(MLA_ERR_ARG, "topk: scores is NULL");
    if (!n_valid || !sel || !nsel) return fail(MLA_ERR_ARG, "topk: NULL tensor");
    size_t need = dsa_topk_workspace_bytes(B, t_max, k);
    if (need && (!ws || ws_bytes < need))
        return fail(MLA_ERR_WORKSPACE, "topk: workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : (size_t)0);
    return launch_topk(scores, B, t_max, n_valid, t_max, k, sel, nsel, ws, ws_bytes, (hipStream_t)stream);
}

size_t dsa_index_select_workspace_bytes(int32_t B, int64_t t_max, int32_t k)
{
    if (B <= 0 || t_max <= 0 || k <= 0) return 0;
    return index_select_workspace_bytes(B, t_max, k);
}

mla_status dsa_index_select(const float *q_idx, const float *w_idx, int32_t B, int32_t n_ih, const mla_kv_view *kv,
                            int64_t t_max, int32_t k, float *scores, int32_t *sel, int32_t *nsel, void *ws,
                            size_t ws_bytes, void *stream)
{
    g_err[0] = 0;
    if (B < 0 || t_max < 0) return fail(MLA_ERR_ARG, "select: B or t_max negative");
    if (n_ih <= 0) return fail(MLA_ERR_ARG, "select: n_ih must be positive");
    if (n_ih > 64) return fail(MLA_ERR_UNSUPPORTED, "select: n_ih > 64");
    if (k <= 0) return fail(MLA_ERR_ARG, "select: k must be positive");
    if (k > 65536) return fail(MLA_ERR_UNSUPPORTED, "select: k > 65536");
    mla_status st = check_view(kv, B, false, true, true);
    if (st) return st;
    if (kv->index_hd <= 0 || kv->index_hd % 4 != 0)
        return fail(MLA_ERR_ARG, "select: index_hd must be a positive multiple of 4");
    if (kv->index_hd > 256) return fail(MLA_ERR_UNSUPPORTED, "select: index_hd > 256");
    if (t_max >= ((int64_t)1 << 31)) return fail(MLA_ERR_UNSUPPORTED, "select: t_max >= 2^31");
    if (B == 0) return MLA_OK;
    if (!q_idx || !w_idx || !sel || !nsel || (!scores && t_max > 0)) return fail(MLA_ERR_ARG, "select: NULL tensor");
    size_t need = dsa_index_select_workspace_bytes(B, t_max, k);
    if (need && (!ws || ws_bytes < need))
        return fail(MLA_ERR_WORKSPACE, "select: workspace of %zu bytes needed, %zu given", need,
                    ws ? ws_bytes : (size_t)0);
    KvView v = to_view(*kv);
    if (v.max_seq_len > t_max) v.max_seq_len = t_max;
    return launch_index_select(q_idx, w_idx, B, n_ih, kv->index_hd, v, t_max, k, scores, sel, nsel, ws, ws_bytes,
                               (hipStream_t)stream);
}

size_t mla_decode_workspace_bytes(const mla_dims *d, int32_t B, int64_t max_keys)
{
    if (!d || B <= 0 || max_keys < 0) return 0;
    if (check_dims(d) != MLA_OK) return 0;
    return decode_workspace_bytes(*d, B, max_keys, MLA_BF16) > decode_workspace_bytes(*d, B, max_keys, MLA_FP32)
               ? decode_workspace_bytes(*d, B, max_keys, MLA_BF16)
               : decode_workspace_bytes(*d, B, max_keys, MLA_FP32);
}

// Checks shared by the decode entry points (everything but the tensors each step reads).
static mla_status check_decode_common(const mla_dims *d, int32_t B, mla_dtype q_dt, mla_dtype w_dt)
{
    mla_status st = check_dims(d);
    if (st) return st;
    if (B < 0) return fail(MLA_ERR_ARG, "decode: B negative");
    if (!valid_dtype(q_dt) || !valid_dtype(w_dt)) return fail(MLA_ERR_ARG, "decode: dtype invalid");
    if (q_dt != w_dt) return fail(MLA_ERR_UNSUPPORTED, "decode: q and kv_b dtypes must match");
    return MLA_OK;
}

static mla_status check_decode_attend(const mla_dims *d, int32_t B, mla_dtype q_dt, mla_dtype w_dt,
                                      const mla_kv_view *kv, const int32_t *sel, const int32_t *nsel,
                                      int32_t sel_stride, float sm_scale)
{
    mla_status st = check_decode_common(d, B, q_dt, w_dt);
    if (st) return st;
    st = check_view(kv, B, true, false, true);
    if (st) return st;
    if (q_dt != kv->kv_dtype) return fail(MLA_ERR_UNSUPPORTED, "decode: q, kv_b and cache dtypes must match");
    if (!isfinite(sm_scale)) return fail(MLA_ERR_ARG, "decode: sm_scale not finite");
    if (sel) {
        if (!nsel) return fail(MLA_ERR_ARG, "decode: sel given without nsel");
        if (sel_stride <= 0) return fail(MLA_ERR_ARG, "decode: sel_stride must be positive");
    }
    return MLA_OK;
}

static mla_status check_ws(const char *what, size_t need, const void *ws, size_t ws_bytes)
{
    if (need && (!ws || ws_bytes < need))
        return fail(MLA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", what, need,
                    ws ? ws_bytes : (size_t)0);
    return MLA_OK;
}

mla_status mla_absorbed_decode(const void *q_nope, const void *q_rope, mla_dtype q_dt,
                               const void *kv_b, mla_dtype w_dt, const mla_dims *d, int32_t B,
                               const mla_kv_view *kv, const int32_t *sel, const int32_t *nsel,
                               int32_t sel_stride, float sm_scale, float *out, void *ws,
                               size_t ws_bytes, void *stream)
{
    g_err[0] = 0;
    mla_status st = check_decode_attend(d, B, q_dt, w_dt, kv, sel, nsel, sel_stride, sm_scale);
    if (st) return st;
    if (B == 0) return MLA_OK;
    if (!q_nope || !q_rope || !kv_b || !out) return fail(MLA_ERR_ARG, "decode: NULL tensor");
    const int64_t max_keys = sel ? (int64_t)sel_stride : kv->max_seq_len;
    st = check_ws("decode", decode_workspace_bytes(*d, B, max_keys, q_dt), ws, ws_bytes);
    if (st) return st;
    return launch_decode(q_nope, q_rope, kv_b, q_dt, *d, B, to_view(*kv), sel, nsel, sel_stride, max_keys,
                         sm_scale, out, ws, ws_bytes, (hipStream_t)stream);
}

mla_status mla_decode_absorb(const void *q_nope, mla_dtype q_dt, const void *kv_b, mla_dtype w_dt,
                             const mla_dims *d, int32_t B, void *ws, size_t ws_bytes, void *stream)
{
    g_err[0] = 0;
    mla_status st = check_decode_common(d, B, q_dt, w_dt);
    if (st) return st;
    if (B == 0) return MLA_OK;
    if (!q_nope || !kv_b) return fail(MLA_ERR_ARG, "decode absorb: NULL tensor");
    st = check_ws("decode absorb", decode_absorb_workspace_bytes(*d, B, q_dt), ws, ws_bytes);
    if (st) return st;
    return launch_decode_absorb(q_nope, kv_b, q_dt, *d, B, ws, (hipStream_t)stream);
}

mla_status mla_decode_attend(const void *q_rope, mla_dtype q_dt, const void *kv_b, mla_dtype w_dt,
                             const mla_dims *d, int32_t B, const mla_kv_view *kv, const int32_t *sel,
                             const int32_t *nsel, int32_t sel_stride, float sm_scale, float *out, void *ws,
                             size_t ws_bytes, void *stream)
{
    g_err[0] = 0;
    mla_status st = check_decode_attend(d, B, q_dt, w_dt, kv, sel, nsel, sel_stride, sm_scale);
    if (st) return st;
    if (B == 0) return MLA_OK;
    if (!q_rope || !kv_b || !out) return fail(MLA_ERR_ARG, "decode attend: NULL tensor");
    const int64_t max_keys = sel ? (int64_t)sel_stride : kv->max_seq_len;
    st = check_ws("decode attend", decode_workspace_bytes(*d, B, max_keys, q_dt), ws, ws_bytes);
    if (st) return st;
    return launch_decode_attend(q_rope, kv_b, q_dt, *d, B, to_view(*kv), sel, nsel, sel_stride, max_keys, sm_scale,
                                out, ws, (hipStream_t)stream);
}

size_t mla_dsa_decode_workspace_bytes(const mla_dims *d, int32_t B, int64_t t_max, int32_t k)
{
    if (!d || B <= 0 || t_max < 0 || k <= 0) return 0;
    if (check_dims(d) != MLA_OK) return 0;
    const size_t a = dsa_decode_workspace_bytes(*d, B, t_max, k, MLA_BF16);
    const size_t b = dsa_decode_workspace_bytes(*d, B, t_max, k, MLA_FP32);
    return a > b ? a : b;
}

}  // extern "C"

// Checks of the whole decode step, everything but the workspace (shared by the call that takes a
// workspace and the one that uses the library's static scratch).
static mla_status check_dsa_decode(const void *q_nope, const void *q_rope, mla_dtype q_dt, double rope_theta,
                                   const float *q_idx, const float *w_idx, int32_t n_ih, const void *kv_b,
                                   mla_dtype w_dt, const mla_dims *d, int32_t B, const mla_kv_view *kv,
                                   int64_t t_max, int32_t k, float sm_scale, const float *scores, const int32_t *sel,
                                   const int32_t *nsel, const float *out)
{
    mla_status st = check_decode_common(d, B, q_dt, w_dt);
    if (st) return st;
    st = check_view(kv, B, true, true, true);
    if (st) return st;
    if (q_dt != kv->kv_dtype) return fail(MLA_ERR_UNSUPPORTED, "dsa decode: q, kv_b and cache dtypes must match");
    if (!isfinite(sm_scale)) return fail(MLA_ERR_ARG, "dsa decode: sm_scale not finite");
    if (!(rope_theta > 0.0) || !isfinite(rope_theta)) return fail(MLA_ERR_ARG, "dsa decode: rope_theta must be positive and finite");
    if (d->qk_rope > 512) return fail(MLA_ERR_UNSUPPORTED, "dsa decode: qk_rope > 512");
    if (t_max < 0) return fail(MLA_ERR_ARG, "dsa decode: t_max negative");
    if (t_max >= ((int64_t)1 << 31)) return fail(MLA_ERR_UNSUPPORTED, "dsa decode: t_max >= 2^31");
    if (n_ih <= 0) return fail(MLA_ERR_ARG, "dsa decode: n_ih must be positive");
    if (n_ih > 64) return fail(MLA_ERR_UNSUPPORTED, "dsa decode: n_ih > 64");
    if (k <= 0) return fail(MLA_ERR_ARG, "dsa decode: k must be positive");
    if (k > 65536) return fail(MLA_ERR_UNSUPPORTED, "dsa decode: k > 65536");
    if (kv->index_hd <= 0 || kv->index_hd % 4 != 0)
        return fail(MLA_ERR_ARG, "dsa decode: index_hd must be a positive multiple of 4");
    if (kv->index_hd > 256) return fail(MLA_ERR_UNSUPPORTED, "dsa decode: index_hd > 256");
    if (B == 0) return MLA_OK;
    if (!q_nope || !q_rope || !q_idx || !w_idx || !kv_b || !sel || !nsel || !out || (!scores && t_max > 0))
        return fail(MLA_ERR_ARG, "dsa decode: NULL tensor");
    return MLA_OK;
}

static mla_status run_dsa_decode(const void *q_nope, const void *q_rope, mla_dtype q_dt, double rope_theta,
                                 const float *q_idx, const float *w_idx, int32_t n_ih, const void *kv_b,
                                 const mla_dims *d, int32_t B, const mla_kv_view *kv, int64_t t_max, int32_t k,
                                 float sm_scale, float *scores, int32_t *sel, int32_t *nsel, float *out, void *ws,
                                 void *stream)
{
    const KvView v = to_view(*kv);
    KvView vs = v;
    if (vs.max_seq_len > t_max) vs.max_seq_len = t_max;
    return launch_dsa_decode(q_nope, q_rope, q_dt, rope_theta, q_idx, w_idx, n_ih, kv->index_hd, kv_b, *d, B, vs, v,
                             t_max, k, sm_scale, scores, sel, nsel, out, ws, (hipStream_t)stream);
}

extern "C" {

mla_status mla_dsa_decode(const void *q_nope, const void *q_rope, mla_dtype q_dt, double rope_theta,
                          const float *q_idx, const float *w_idx, int32_t n_ih, const void *kv_b, mla_dtype w_dt,
                          const mla_dims *d, int32_t B, const mla_kv_view *kv, int64_t t_max, int32_t k,
                          float sm_scale, float *scores, int32_t *sel, int32_t *nsel, float *out, void *ws,
                          size_t ws_bytes, void *stream)
{
    g_err[0] = 0;
    mla_status st = check_dsa_decode(q_nope, q_rope, q_dt, rope_theta, q_idx, w_idx, n_ih, kv_b, w_dt, d, B, kv,
                                     t_max, k, sm_scale, scores, sel, nsel, out);
    if (st || B == 0) return st;
    st = check_ws("dsa decode", dsa_decode_workspace_bytes(*d, B, t_max, k, q_dt), ws, ws_bytes);
    if (st) return st;
    return run_dsa_decode(q_nope, q_rope, q_dt, rope_theta, q_idx, w_idx, n_ih, kv_b, d, B, kv, t_max, k, sm_scale,
                          scores, sel, nsel, out, ws, stream);
}

mla_status mla_dsa_decode_noalloc(const void *q_nope, const void *q_rope, mla_dtype q_dt, double rope_theta,
                                  const float *q_idx, const float *w_idx, int32_t n_ih, const void *kv_b,
                                  mla_dtype w_dt, const mla_dims *d, int32_t B, const mla_kv_view *kv,
                                  int64_t t_max, int32_t k, float sm_scale, float *scores, int32_t *sel,
                                  int32_t *nsel, float *out, void *stream)
{
    g_err[0] = 0;
    mla_status st = check_dsa_decode(q_nope, q_rope, q_dt, rope_theta, q_idx, w_idx, n_ih, kv_b, w_dt, d, B, kv,
                                     t_max, k, sm_scale, scores, sel, nsel, out);
    if (st || B == 0) return st;
    const size_t need = dsa_decode_workspace_bytes(*d, B, t_max, k, q_dt);
    if (need > NOALLOC_SCRATCH_BYTES)
        return fail(MLA_ERR_WORKSPACE,
                    "dsa decode (no allocation): this step needs %zu bytes of scratch, the library's static "
                    "scratch holds %zu (use mla_dsa_decode with a workspace)", need, NOALLOC_SCRATCH_BYTES);
    void *scratch = nullptr;
    st = noalloc_scratch(&scratch);
    if (st) return st;
    return run_dsa_decode(q_nope, q_rope, q_dt, rope_theta, q_idx, w_idx, n_ih, kv_b, d, B, kv, t_max, k, sm_scale,
                          scores, sel, nsel, out, scratch, stream);
}

static mla_status check_qweights(const mla_qweights *w, const mla_dims *d)
{
    if (!w) return fail(MLA_ERR_ARG, "quantized kv_b: weights struct is NULL");
    if (w->format != MLA_Q_FP8_E4M3 && w->format != MLA_Q_INT8 && w->format != MLA_Q_MXFP4)
        return fail(MLA_ERR_ARG, "quantized kv_b: unknown format %d", (int)w->format);
    if (!w->codes || !w->scales) return fail(MLA_ERR_ARG, "quantized kv_b: codes or scales is NULL");
    if (((reinterpret_cast<uintptr_t>(w->codes) | reinterpret_cast<uintptr_t>(w->scales)) & 3u) != 0)
        return fail(MLA_ERR_UNSUPPORTED, "quantized kv_b: codes and scales must be 4-byte aligned");
    if (!decode_quant_supported(*d, MLA_BF16))
        return fail(MLA_ERR_UNSUPPORTED, "quantized kv_b: needs 64 heads, kv_lora 512, qk_rope 64, qk_nope a multiple "
                    "of 8 up to 256, v_head a multiple of 32");
    return MLA_OK;
}

static bool al16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

mla_status mla_absorbed_decode_q(const void *q_nope, const void *q_rope, mla_dtype q_dt, const mla_qweights *kv_b,
                                 const mla_dims *d, int32_t B, const mla_kv_view *kv, const int32_t *sel,
                                 const int32_t *nsel, int32_t sel_stride, float sm_scale, float *out, void *ws,
                                 size_t ws_bytes, void *stream)
{
    g_err[0] = 0;
    mla_status st = check_decode_attend(d, B, q_dt, q_dt, kv, sel, nsel, sel_stride, sm_scale);
    if (st) return st;
    if (q_dt != MLA_BF16) return fail(MLA_ERR_UNSUPPORTED, "quantized decode: bf16 queries and cache only");
    st = check_qweights(kv_b, d);
    if (st) return st;
    if (B == 0) return MLA_OK;
    if (!q_nope || !q_rope || !out) return fail(MLA_ERR_ARG, "quantized decode: NULL tensor");
    if (!al16(q_nope) || !al16(q_rope) || !al16(kv->lc) || !al16(kv->rc))
        return fail(MLA_ERR_UNSUPPORTED, "quantized decode: q_nope, q_rope, Lc and Rc must be 16-byte aligned");
    const int64_t max_keys = sel ? (int64_t)sel_stride : kv->max_seq_len;
    st = check_ws("quantized decode", decode_workspace_bytes(*d, B, max_keys, q_dt), ws, ws_bytes);
    if (st) return st;
    return launch_decode_quant(q_nope, q_rope, (const uint8_t *)kv_b->codes, kv_b->scales, kv_b->format, *d, B,
                               to_view(*kv), sel, nsel, sel ? sel_stride : 0, max_keys, sm_scale, out, ws,
                               (hipStream_t)stream);
}

mla_status mla_dsa_decode_q(const void *q_nope, const void *q_rope, mla_dtype q_dt, double rope_theta,
                            const float *q_idx, const float *w_idx, int32_t n_ih, const mla_qweights *kv_b,
                            const mla_dims *d, int32_t B, const mla_kv_view *kv, int64_t t_max, int32_t k,
                            float sm_scale, float *scores, int32_t *sel, int32_t *nsel, float *out, void *ws,
                            size_t ws_bytes, void *stream)
{
    g_err[0] = 0;
    const void *codes = kv_b ? kv_b->codes : nullptr;
    mla_status st = check_dsa_decode(q_nope, q_rope, q_dt, rope_theta, q_idx, w_idx, n_ih, codes, q_dt, d, B, kv,
                                     t_max, k, sm_scale, scores, sel, nsel, out);
    if (st || B == 0) return st;
    if (q_dt != MLA_BF16) return fail(MLA_ERR_UNSUPPORTED, "quantized decode: bf16 queries and cache only");
    st = check_qweights(kv_b, d);
    if (st) return st;
    if (!al16(q_nope) || !al16(q_rope) || !al16(kv->lc) || !al16(kv->rc))
        return fail(MLA_ERR_UNSUPPORTED, "quantized decode: q_nope, q_rope, Lc and Rc must be 16-byte aligned");
    st = check_ws("quantized dsa decode", dsa_decode_workspace_bytes(*d, B, t_max, k, q_dt), ws, ws_bytes);
    if (st) return st;
    const KvView v = to_view(*kv);
    KvView vs = v;
    if (vs.max_seq_len > t_max) vs.max_seq_len = t_max;
    return launch_dsa_decode_quant(q_nope, q_rope, rope_theta, q_idx, w_idx, n_ih, kv->index_hd,
                                   (const uint8_t *)kv_b->codes, kv_b->scales, kv_b->format, *d, B, vs, v, t_max, k,
                                   sm_scale, scores, sel, nsel, out, ws, (hipStream_t)stream);
}

int32_t mla_attention_absorbs(int32_t S, int32_t g_absorb) { return attention_absorbs(S, g_absorb) ? 1 : 0; }

size_t mla_attention_workspace_bytes(const mla_dims *d, int32_t S, int32_t pos_base, int32_t sel_stride,
                                     int32_t g_absorb)
{
    if (!d || S <= 0 || pos_base < 0 || sel_stride < 0) return 0;
    if (check_dims(d) != MLA_OK) return 0;
    const bool ab = attention_absorbs(S, g_absorb);
    const int64_t T = (int64_t)pos_base + S;
    const size_t a = attention_workspace_bytes(*d, S, T, sel_stride, ab, MLA_BF16);
    const size_t b = attention_workspace_bytes(*d, S, T, sel_stride, ab, MLA_FP32);
    return a > b ? a : b;
}

mla_status mla_attention(const void *q, mla_dtype q_dt, const void *kv_b, mla_dtype w_dt, const mla_dims *d,
                         const mla_kv_view *kv, int32_t S, int32_t pos_base, const int32_t *sel, const int32_t *nsel,
                         int32_t sel_stride, float sm_scale, int32_t g_absorb, float *out, void *ws, size_t ws_bytes,
                         void *stream)
{
    g_err[0] = 0;
    mla_status st = check_dims(d);
    if (st) return st;
    if (S < 0 || pos_base < 0) return fail(MLA_ERR_ARG, "attention: S or pos_base negative");
    if (S > 65535) return fail(MLA_ERR_UNSUPPORTED, "attention: S > 65535");
    if (g_absorb < -1 || g_absorb > 1) return fail(MLA_ERR_ARG, "attention: g_absorb must be -1, 0 or 1");
    if (!valid_dtype(q_dt) || !valid_dtype(w_dt)) return fail(MLA_ERR_ARG, "attention: dtype invalid");
    if (!kv) return fail(MLA_ERR_ARG, "attention: kv view is NULL");
    const int64_t T = (int64_t)pos_base + S;
    if (T >= ((int64_t)1 << 31)) return fail(MLA_ERR_UNSUPPORTED, "attention: pos_base + S >= 2^31");
    mla_kv_view v1 = *kv;
    if (v1.max_seq_len < T) v1.max_seq_len = T;   // sequence 0 spans rows for t < T
    st = check_view(&v1, 1, true, false, false);
    if (st) return st;
    if (q_dt != w_dt || q_dt != kv->kv_dtype) return fail(MLA_ERR_UNSUPPORTED, "attention: q, kv_b and cache dtypes must match");
    if (!isfinite(sm_scale)) return fail(MLA_ERR_ARG, "attention: sm_scale not finite");
    if (sel && (!nsel || sel_stride <= 0)) return fail(MLA_ERR_ARG, "attention: sel needs nsel and sel_stride > 0");
    const bool ab = attention_absorbs(S, g_absorb);
    if (sel && !ab && sel_stride >= (1 << 19))
        return fail(MLA_ERR_UNSUPPORTED, "attention: sel_stride >= 2^19 on the non-absorbed path");
    if (S == 0) return MLA_OK;
    if (!q || !kv_b || !out) return fail(MLA_ERR_ARG, "attention: NULL tensor");
    st = check_ws("attention", attention_workspace_bytes(*d, S, T, sel ? sel_stride : 0, ab, q_dt), ws, ws_bytes);
    if (st) return st;
    return launch_attention(q, q_dt, kv_b, *d, to_view(v1), S, pos_base, sel, nsel, sel ? sel_stride : 0, sm_scale, ab,
                            out, ws, (hipStream_t)stream);
}

size_t dsa_prefill_select_workspace_bytes(int32_t S, int32_t pos_base, int32_t k)
{
    if (S <= 0 || pos_base < 0 || k <= 0) return 0;
    return index_select_workspace_bytes(S, (int64_t)pos_base + S, k);
}

mla_status dsa_prefill_select(const float *q_idx, const float *w_idx, int32_t n_ih, const mla_kv_view *kv, int32_t S,
                              int32_t pos_base, int32_t k, float *scores, int32_t *sel, int32_t *nsel, void *ws,
                              size_t ws_bytes, void *stream)
{
    g_err[0] = 0;
    if (S < 0 || pos_base < 0) return fail(MLA_ERR_ARG, "prefill select: S or pos_base negative");
    if (S > 65535) return fail(MLA_ERR_UNSUPPORTED, "prefill select: S > 65535");
    if (n_ih <= 0) return fail(MLA_ERR_ARG, "prefill select: n_ih must be positive");
    if (n_ih > 64) return fail(MLA_ERR_UNSUPPORTED, "prefill select: n_ih > 64");
    if (k <= 0) return fail(MLA_ERR_ARG, "prefill select: k must be positive");
    if (k > 65536) return fail(MLA_ERR_UNSUPPORTED, "prefill select: k > 65536");
    if (!kv) return fail(MLA_ERR_ARG, "prefill select: kv view is NULL");
    const int64_t T = (int64_t)pos_base + S;
    if (T >= ((int64_t)1 << 31)) return fail(MLA_ERR_UNSUPPORTED, "prefill select: pos_base + S >= 2^31");
    mla_kv_view v1 = *kv;
    if (v1.max_seq_len < T) v1.max_seq_len = T;
    mla_status st = check_view(&v1, 1, false, true, false);
    if (st) return st;
    if (kv->index_hd <= 0 || kv->index_hd % 4 != 0)
        return fail(MLA_ERR_ARG, "prefill select: index_hd must be a positive multiple of 4");
    if (kv->index_hd > 256) return fail(MLA_ERR_UNSUPPORTED, "prefill select: index_hd > 256");
    if (S == 0) return MLA_OK;
    if (!q_idx || !w_idx || !scores || !sel || !nsel) return fail(MLA_ERR_ARG, "prefill select: NULL tensor");
    st = check_ws("prefill select", index_select_workspace_bytes(S, T, k), ws, ws_bytes);
    if (st) return st;
    KvView v = to_view(v1);
    v.seq_len = nullptr;
    v.max_seq_len = T;
    v.qps = S;   // launch row i = query i at position pos_base + i
    return launch_index_select(q_idx, w_idx, S, n_ih, kv->index_hd, v, T, k, scores, sel, nsel, ws, ws_bytes,
                               (hipStream_t)stream);
}

size_t mla_dsa_decode_shared_workspace_bytes(const mla_dims *d, int32_t B, int32_t k)
{
    if (!d || B <= 0 || k <= 0) return 0;
    if (check_dims(d) != MLA_OK) return 0;
    const size_t a = dsa_shared_workspace_bytes(*d, B, k, MLA_BF16), b = dsa_shared_workspace_bytes(*d, B, k, MLA_FP32);
    return a > b ? a : b;
}

mla_status mla_dsa_decode_shared(const void *q_nope, const void *q_rope, mla_dtype q_dt, double rope_theta,
                                 const void *kv_b, mla_dtype w_dt, const mla_dims *d, int32_t B,
                                 const mla_kv_view *kv, const int32_t *sel, const int32_t *nsel, int32_t k,
                                 float sm_scale, float *out, void *ws, size_t ws_bytes, void *stream)
{
    g_err[0] = 0;
    if (!sel || !nsel) return fail(MLA_ERR_ARG, "shared decode: sel and nsel are inputs and must be given");
    if (k <= 0) return fail(MLA_ERR_ARG, "shared decode: k must be positive");
    if (k > 65536) return fail(MLA_ERR_UNSUPPORTED, "shared decode: k > 65536");
    mla_status st = check_decode_attend(d, B, q_dt, w_dt, kv, sel, nsel, k, sm_scale);
    if (st) return st;
    if (!(rope_theta > 0.0) || !isfinite(rope_theta))
        return fail(MLA_ERR_ARG, "shared decode: rope_theta must be positive and finite");
    if (B == 0) return MLA_OK;
    if (!q_nope || !q_rope || !kv_b || !out) return fail(MLA_ERR_ARG, "shared decode: NULL tensor");
    st = check_ws("shared decode", dsa_shared_workspace_bytes(*d, B, k, q_dt), ws, ws_bytes);
    if (st) return st;
    return launch_dsa_shared(q_nope, q_rope, q_dt, rope_theta, kv_b, *d, B, to_view(*kv), sel, nsel, k, sm_scale,
                             out, ws, (hipStream_t)stream);
}

mla_status mla_cache_write(const void *comp, const void *ik, mla_dtype in_dt, int64_t n_tok, const int32_t *seq,
                           const int32_t *pos, int32_t n_seq, int32_t kv_lora, int32_t qk_rope, const float *kv_gain,
                           const float *ix_gamma, const float *ix_beta, int32_t ix_rope_off, int32_t ix_rope_dim,
                           double eps_kv, double eps_ix, double theta, const mla_kv_view *kv, void *stream)
{
    g_err[0] = 0;
    if (!valid_dtype(in_dt)) return fail(MLA_ERR_ARG, "cache write: dtype invalid");
    if (n_tok < 0 || n_seq <= 0) return fail(MLA_ERR_ARG, "cache write: n_tok < 0 or n_seq <= 0");
    if (kv_lora <= 0 || qk_rope <= 0 || (qk_rope & 1)) return fail(MLA_ERR_ARG, "cache write: kv_lora / qk_rope invalid");
    if (kv_lora > 2048 || qk_rope > 512) return fail(MLA_ERR_UNSUPPORTED, "cache write: kv_lora > 2048 or qk_rope > 512");
    if (!(eps_kv > 0.0) || !isfinite(eps_kv) || !(eps_ix > 0.0) || !isfinite(eps_ix))
        return fail(MLA_ERR_ARG, "cache write: eps must be positive and finite");
    if (!(theta > 0.0) || !isfinite(theta)) return fail(MLA_ERR_ARG, "cache write: theta must be positive and finite");
    mla_status st = check_view(kv, n_seq, true, ik != nullptr, false);
    if (st) return st;
    if (ik) {
        const int32_t hd = kv->index_hd;
        if (hd <= 0 || hd % 4 != 0) return fail(MLA_ERR_ARG, "cache write: index_hd must be a positive multiple of 4");
        if (hd > 256) return fail(MLA_ERR_UNSUPPORTED, "cache write: index_hd > 256");
        if (ix_rope_off < 0 || ix_rope_dim < 0 || (ix_rope_dim & 1) || ix_rope_off + ix_rope_dim > hd)
            return fail(MLA_ERR_ARG, "cache write: indexer rope slice outside the key");
    }
    if (n_tok == 0) return MLA_OK;
    if (!comp || !seq || !pos) return fail(MLA_ERR_ARG, "cache write: NULL tensor");
    return launch_cache_write(comp, ik, in_dt, n_tok, seq, pos, n_seq, to_view(*kv), kv->kv_dtype, kv_lora, qk_rope,
                              ik ? kv->index_hd : 0, kv_gain, ix_gamma, ix_beta, ix_rope_off, ix_rope_dim,
                              (float)eps_kv, (float)eps_ix, theta, (hipStream_t)stream);
}

size_t mla_prefill_workspace_bytes(const mla_dims *d, int32_t S, int64_t T)
{
    if (!d || S <= 0 || T <= 0) return 0;
    if (check_dims(d) != MLA_OK) return 0;
    size_t a = prefill_workspace_bytes(*d, S, T, MLA_BF16), b = prefill_workspace_bytes(*d, S, T, MLA_FP32);
    return a > b ? a : b;
}

mla_status mla_prefill_nonabsorbed(const void *q, mla_dtype q_dt, const void *kv_b, mla_dtype w_dt,
                                   const mla_dims *d, const mla_kv_view *kv, int32_t S,
                                   int32_t pos_base, float sm_scale, void *out, mla_dtype out_dt,
                                   void *ws, size_t ws_bytes, void *stream)
{
    g_err[0] = 0;
    mla_status st = check_dims(d);
    if (st) return st;
    if (S < 0 || pos_base < 0) return fail(MLA_ERR_ARG, "prefill: S or pos_base negative");
    if (!valid_dtype(q_dt) || !valid_dtype(w_dt) || !valid_dtype(out_dt)) return fail(MLA_ERR_ARG, "prefill: dtype invalid");
    if (!kv) return fail(MLA_ERR_ARG, "prefill: kv view is NULL");
    int64_t T = (int64_t)pos_base + S;
    if (T >= ((int64_t)1 << 31)) return fail(MLA_ERR_UNSUPPORTED, "prefill: pos_base + S >= 2^31");
    mla_kv_view v1 = *kv;
    if (v1.max_seq_len < T) v1.max_seq_len = T;   // the prefill covers rows 0..T-1 of sequence 0
    st = check_view(&v1, 1, true, false, false);
    if (st) return st;
    if (q_dt != w_dt || q_dt != kv->kv_dtype)
        return fail(MLA_ERR_UNSUPPORTED, "prefill: q, kv_b and cache dtypes must match");
    if (!isfinite(sm_scale)) return fail(MLA_ERR_ARG, "prefill: sm_scale not finite");
    if (S == 0) return MLA_OK;
    if (!q || !kv_b || !out) return fail(MLA_ERR_ARG, "prefill: NULL tensor");
    size_t need = prefill_workspace_bytes(*d, S, T, q_dt);
    if (need && (!ws || ws_bytes < need))
        return fail(MLA_ERR_WORKSPACE, "prefill: workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : (size_t)0);
    KvView v = to_view(v1);
    v.seq_len = nullptr;   // sequence 0 spans rows for t < T
    v.max_seq_len = T;
    return launch_prefill(q, kv_b, q_dt, *d, v, S, pos_base, sm_scale, out, out_dt, ws, ws_bytes, (hipStream_t)stream);
}

}  // extern "C"
