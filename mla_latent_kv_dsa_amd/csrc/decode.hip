// decode.hip -- chooses the kernels of the absorbed decode for a given shape and dtype: the
// matrix-core kernels for bf16 caches with 64 heads, kv_lora 512 and qk_rope 64, the generic
// kernels for every other geometry.  The decode runs in two steps that share one workspace:
// absorb (W_UK folded into the query; needs only q_nope and kv_b) and attend (scores,
// softmax, latent accumulation, W_UV).  The absorb step can therefore be issued early, e.g.
// on a second stream while the indexer and the top-k run.
#include <initializer_list>

#include "decode_plan.h"

namespace mla {

static bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The matrix-core kernels serve their geometry (decode_mfma_supported) only.  They read every
// operand in 16-byte pieces, so on that geometry a tensor that is not 16-byte aligned is
// rejected with MLA_ERR_UNSUPPORTED by every decode entry point alike: no call switches
// kernels because of where a pointer sits.  Other geometries and fp32 take the generic kernels.
static bool use_mfma(const mla_dims &d, mla_dtype dt) { return decode_mfma_supported(d, dt); }

static mla_status need_aligned(const char *what, std::initializer_list<const void *> ps)
{
    for (const void *p : ps)
        if (!aligned16(p))
            return fail(MLA_ERR_UNSUPPORTED, "%s: on the matrix-core geometry (bf16, 64 heads, kv_lora 512, "
                        "qk_rope 64) every tensor must be 16-byte aligned", what);
    return MLA_OK;
}

size_t decode_workspace_bytes(const mla_dims &d, int32_t B, int64_t max_keys, mla_dtype dt)
{
    size_t g = decode_generic_ws(d, B, max_keys);
    if (decode_mfma_supported(d, dt)) {
        size_t m = decode_mfma_ws(d, B, max_keys);
        return m > g ? m : g;
    }
    return g;
}

size_t decode_absorb_workspace_bytes(const mla_dims &d, int32_t B, mla_dtype dt)
{
    size_t g = decode_generic_absorb_ws(d, B);
    if (decode_mfma_supported(d, dt)) {
        size_t m = decode_mfma_absorb_ws(B);
        return m > g ? m : g;
    }
    return g;
}

mla_status launch_decode_absorb(const void *q_nope, const void *kv_b, mla_dtype dt, const mla_dims &d, int32_t B,
                                void *ws, hipStream_t s)
{
    if (use_mfma(d, dt)) {
        mla_status st = need_aligned("decode absorb", {q_nope, kv_b});
        if (st) return st;
        return launch_absorb_mfma(q_nope, kv_b, d, B, ws, s);
    }
    return launch_absorb_generic(q_nope, kv_b, dt, d, B, ws, s);
}

mla_status launch_decode_attend(const void *q_rope, const void *kv_b, mla_dtype dt, const mla_dims &d, int32_t B,
                                const KvView &kv, const int32_t *sel, const int32_t *nsel, int32_t sel_stride,
                                int64_t max_keys, float sm_scale, float *out, void *ws, hipStream_t s)
{
    if (use_mfma(d, dt)) {
        mla_status st = need_aligned("decode attend", {q_rope, kv_b, kv.lc, kv.rc});
        if (st) return st;
        return launch_attend_mfma(q_rope, kv_b, d, B, kv, sel, nsel, sel_stride, max_keys, sm_scale, out, ws, s);
    }
    return launch_attend_generic(q_rope, kv_b, dt, d, B, kv, sel, nsel, sel_stride, max_keys, sm_scale, out, ws, s);
}

mla_status launch_decode(const void *q_nope, const void *q_rope, const void *kv_b, mla_dtype dt,
                         const mla_dims &d, int32_t B, const KvView &kv, const int32_t *sel,
                         const int32_t *nsel, int32_t sel_stride, int64_t max_keys, float sm_scale,
                         float *out, void *ws, size_t, hipStream_t s)
{
    mla_status st;
    if (use_mfma(d, dt)) {
        st = need_aligned("decode", {q_nope, q_rope, kv_b, kv.lc, kv.rc});
        if (st) return st;
        st = launch_absorb_mfma(q_nope, kv_b, d, B, ws, s);
        if (st) return st;
        return launch_attend_mfma(q_rope, kv_b, d, B, kv, sel, nsel, sel_stride, max_keys, sm_scale, out, ws, s);
    }
    st = launch_absorb_generic(q_nope, kv_b, dt, d, B, ws, s);
    if (st) return st;
    return launch_attend_generic(q_rope, kv_b, dt, d, B, kv, sel, nsel, sel_stride, max_keys, sm_scale, out, ws, s);
}

// ------------------------------------------------------------------------------ decode step
// The whole decode hot path in one call: RoPE of the query tails (at seq_len - 1, out of place),
// indexer scores and top-k selection, absorbed attention over the selected keys.
// Workspace: select part | decode part | rotated query tails.
static size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t dsa_decode_workspace_bytes(const mla_dims &d, int32_t B, int64_t t_max, int32_t k, mla_dtype dt)
{
    const size_t esz = dt == MLA_FP32 ? 4 : 2;
    return 256 + al256(index_select_workspace_bytes(B, t_max, k)) + al256(decode_workspace_bytes(d, B, k, dt)) +
           al256((size_t)B * d.n_heads * d.qk_rope * esz);
}

// The side work of a matrix-core decode step (absorption, and the rotation of the query tails into
// qr_out unless it is nullptr).  fmt != 0: w holds the codes of a quantized kv_b.
static SideAbsorb side_of(const void *q_nope, const void *q_rope, const void *w, const void *scales, int fmt,
                          void *qr_out, void *dec_ws, int32_t B, const mla_dims &d, double theta)
{
    SideAbsorb sa{};
    sa.q_nope = (const bf16_t *)q_nope;
    sa.kv_b = w;
    sa.scales = scales;
    sa.fmt = fmt;
    sa.q_abs = decode_mfma_qabs(dec_ws);
    sa.q_rope = (const bf16_t *)q_rope;
    sa.q_rope_out = (bf16_t *)qr_out;
    sa.B = B;
    sa.nope = d.qk_nope;
    sa.v = d.v_head;
    sa.rope = d.qk_rope;
    sa.theta = theta;
    return sa;
}

// fmt != 0: kv_b holds the codes of a quantized kv_b (matrix-core geometry only)
static mla_status dsa_decode_step(const void *q_nope, const void *q_rope, mla_dtype dt, double theta,
                                  const float *q_idx, const float *w_idx, int32_t n_ih, int32_t hd, const void *kv_b,
                                  const void *scales, int fmt, const mla_dims &d, int32_t B, const KvView &kv_sel,
                                  const KvView &kv, int64_t t_max, int32_t k, float sm_scale, float *scores,
                                  int32_t *sel, int32_t *nsel, float *out, void *ws, hipStream_t s)
{
    char *p = reinterpret_cast<char *>((reinterpret_cast<uintptr_t>(ws) + 255) & ~(uintptr_t)255);
    const size_t sel_bytes = index_select_workspace_bytes(B, t_max, k);
    void *sel_ws = p;
    p += al256(sel_bytes);
    void *dec_ws = p;
    p += al256(decode_workspace_bytes(d, B, k, dt));
    void *qr = p;
    mla_status st;
    const bool mfma = use_mfma(d, dt);
    if (fmt != 0 && !mfma) return fail(MLA_ERR_UNSUPPORTED, "dsa decode: quantized kv_b needs the matrix-core geometry");
    if (mfma) {
        st = need_aligned("dsa decode", {q_nope, q_rope, kv_b, kv.lc, kv.rc});
        if (st) return st;
    }
    if (mfma && B <= SIDE_MAXB) {
        // the query absorption and the rotation run as extra workgroups of the selection's
        // resolve step, which occupies only B workgroups
        const SideAbsorb sa = side_of(q_nope, q_rope, kv_b, scales, fmt, qr, dec_ws, B, d, theta);
        bool done = false;
        st = launch_index_select(q_idx, w_idx, B, n_ih, hd, kv_sel, t_max, k, scores, sel, nsel, sel_ws, sel_bytes, s,
                                 &sa, &done);
        if (st) return st;
        if (!done) {
            st = launch_absorb_rope(sa, kv_sel, s);
            if (st) return st;
        }
        return launch_attend_mfma(qr, kv_b, d, B, kv, sel, nsel, k, k, sm_scale, out, dec_ws, s, scales, fmt);
    }
    st = launch_rope_decode(q_rope, qr, dt, B, d.n_heads, d.qk_rope, kv_sel, theta, s);
    if (st) return st;
    st = launch_index_select(q_idx, w_idx, B, n_ih, hd, kv_sel, t_max, k, scores, sel, nsel, sel_ws, sel_bytes, s);
    if (st) return st;
    if (fmt != 0)
        return launch_decode_quant(q_nope, qr, (const uint8_t *)kv_b, scales, fmt, d, B, kv, sel, nsel, k, k, sm_scale,
                                   out, dec_ws, s);
    return launch_decode(q_nope, qr, kv_b, dt, d, B, kv, sel, nsel, k, k, sm_scale, out, dec_ws, 0, s);
}

mla_status launch_dsa_decode(const void *q_nope, const void *q_rope, mla_dtype dt, double theta, const float *q_idx,
                             const float *w_idx, int32_t n_ih, int32_t hd, const void *kv_b, const mla_dims &d,
                             int32_t B, const KvView &kv_sel, const KvView &kv, int64_t t_max, int32_t k,
                             float sm_scale, float *scores, int32_t *sel, int32_t *nsel, float *out, void *ws,
                             hipStream_t s)
{
    return dsa_decode_step(q_nope, q_rope, dt, theta, q_idx, w_idx, n_ih, hd, kv_b, nullptr, 0, d, B, kv_sel, kv, t_max,
                           k, sm_scale, scores, sel, nsel, out, ws, s);
}

// ------------------------------------------------------------------------------ shared layer
// A DSA-shared layer reuses the selection of an earlier layer: RoPE of its query tails at
// seq_len - 1 (out of place) and the absorbed decode over the given keys.
// Workspace: decode part | rotated query tails.
size_t dsa_shared_workspace_bytes(const mla_dims &d, int32_t B, int32_t k, mla_dtype dt)
{
    const size_t esz = dt == MLA_FP32 ? 4 : 2;
    return 256 + al256(decode_workspace_bytes(d, B, k, dt)) + al256((size_t)B * d.n_heads * d.qk_rope * esz);
}

mla_status launch_dsa_shared(const void *q_nope, const void *q_rope, mla_dtype dt, double theta, const void *kv_b,
                             const mla_dims &d, int32_t B, const KvView &kv, const int32_t *sel, const int32_t *nsel,
                             int32_t k, float sm_scale, float *out, void *ws, hipStream_t s)
{
    char *p = reinterpret_cast<char *>((reinterpret_cast<uintptr_t>(ws) + 255) & ~(uintptr_t)255);
    void *dec_ws = p;
    void *qr = p + al256(decode_workspace_bytes(d, B, k, dt));
    mla_status st;
    if (use_mfma(d, dt)) {
        st = need_aligned("shared decode", {q_nope, q_rope, kv_b, kv.lc, kv.rc});
        if (st) return st;
        // the absorption and the query rotation in one launch
        const SideAbsorb sa = side_of(q_nope, q_rope, kv_b, nullptr, 0, qr, dec_ws, B, d, theta);
        if (side_absorb_ok(sa)) {
            st = launch_absorb_rope(sa, kv, s);
            if (st) return st;
            return launch_attend_mfma(qr, kv_b, d, B, kv, sel, nsel, k, k, sm_scale, out, dec_ws, s);
        }
    }
    st = launch_rope_decode(q_rope, qr, dt, B, d.n_heads, d.qk_rope, kv, theta, s);
    if (st) return st;
    return launch_decode(q_nope, qr, kv_b, dt, d, B, kv, sel, nsel, k, k, sm_scale, out, dec_ws, 0, s);
}

// The decode step with a quantized kv_b: the same launches as the bf16 step, the absorption and
// W_UV reading the codes.  Same workspace layout as the bf16 step.
mla_status launch_dsa_decode_quant(const void *q_nope, const void *q_rope, double theta, const float *q_idx,
                                   const float *w_idx, int32_t n_ih, int32_t hd, const uint8_t *codes,
                                   const void *scales, int32_t fmt, const mla_dims &d, int32_t B, const KvView &kv_sel,
                                   const KvView &kv, int64_t t_max, int32_t k, float sm_scale, float *scores,
                                   int32_t *sel, int32_t *nsel, float *out, void *ws, hipStream_t s)
{
    return dsa_decode_step(q_nope, q_rope, MLA_BF16, theta, q_idx, w_idx, n_ih, hd, codes, scales, fmt, d, B, kv_sel,
                           kv, t_max, k, sm_scale, scores, sel, nsel, out, ws, s);
}

}  // namespace mla
