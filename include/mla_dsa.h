/*
 * mla_dsa.h -- C ABI of libmla_dsa.so: Multi-head Latent Attention over a compressed KV
 * cache, with a DSA lightning indexer, for AMD Instinct MI355X (gfx950).
 *
 * The operations follow two public pages:
 *   chen3feng, "colibri-analysis 06: MLA attention and KV cache"  (cited below as [MLA])
 *   aiknowledge.cn, "Ch.7 sec. 03: token-exact forward validation and faithful DSA" ([FDSA])
 *
 * Conventions for every entry point
 *   - Tensor pointers are DEVICE pointers allocated and owned by the caller.  The library
 *     never allocates, frees or synchronizes; scratch space is a caller-provided workspace
 *     whose size the matching *_workspace_bytes() query returns.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Work is queued
 *     asynchronously on it; results are ready when the stream reaches that point.
 *   - Arguments that live on the host are validated before any HIP call.  A failed check
 *     returns a negative status with nothing launched; mla_last_error() then holds a
 *     message (thread-local).  Launch failures return MLA_ERR_HIP.
 *   - Device-resident sizes (seq_len, n_valid, nsel, block tables) are read by the kernels.
 *     They are clamped to the host-declared capacities, so contract violations give
 *     unspecified values but never an out-of-bounds access.
 *   - Row-major layouts; all strides are in elements.
 *   - Shapes outside what the library implements return MLA_ERR_UNSUPPORTED.
 *   - The matrix-core kernels serve bf16 with 64 heads, kv_lora 512 and qk_rope 64 (decode),
 *     plus v_head 256 and qk_nope 128/192 (prefill).  They read in 16-byte pieces: on that
 *     geometry every tensor pointer a call takes must be 16-byte aligned, or the call returns
 *     MLA_ERR_UNSUPPORTED (every entry point alike; no call changes kernels because of where a
 *     pointer sits).  fp32 and every other geometry run on generic kernels.
 */
#ifndef MLA_DSA_H
#define MLA_DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MLA_OK = 0,
    MLA_ERR_ARG = -1,         /* invalid pointer, size or stride                       */
    MLA_ERR_UNSUPPORTED = -2, /* valid, but a shape/dtype this library does not build  */
    MLA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than the query returned  */
    MLA_ERR_HIP = -4          /* a HIP launch or runtime call failed                   */
} mla_status;

typedef enum { MLA_FP32 = 0, MLA_BF16 = 1 } mla_dtype;

/* Head geometry of one MLA layer ([MLA] sec. 2: qh = qk_nope + qk_rope,
 * kvb_dim = n_heads * (qk_nope + v_head)). */
typedef struct {
    int32_t n_heads;
    int32_t qk_nope;
    int32_t qk_rope;
    int32_t v_head;
    int32_t kv_lora;
} mla_dims;

/* Compressed KV cache of a batch of sequences ([MLA] sec. 1; [FDSA] sec. 2).
 * Each cached token is one row in three pools:
 *   lc: latent row   [kv_lora]   (kv_dtype)   -- the RMS-normed latent Lc
 *   rc: rope-key row [qk_rope]   (kv_dtype)   -- the rotated key Rc shared by all heads
 *   ic: indexer row  [index_hd]  (fp32)       -- the DSA indexer key Ic (may be NULL
 *                                                when no indexer call uses this view)
 * Row of token t of sequence b:
 *   paged      (block_table != NULL): block_table[b*max_blocks + t/block_size]*block_size
 *                                     + t % block_size
 *   contiguous (block_table == NULL): b*seq_stride + t
 * seq_len[b] (device int32) counts the cached tokens of sequence b INCLUDING the current
 * query's own token: a decode query sits at position seq_len[b]-1 and sees keys
 * 0..seq_len[b]-1.  Rows outside [0, rows) are never touched.
 * ic_layout places the indexer rows in their pool (the same 4 * index_hd bytes per token):
 *   MLA_IC_ROWS   element d of row r at ic[r*index_hd + d]
 *   MLA_IC_TILE64 rows in aligned groups of 64 stored dims-major in quads of 4:
 *                 element d of row r at ic[(r/64)*64*index_hd + (d/4)*256 + (r%64)*4 + d%4]
 *                 (a 64-row group is one contiguous 64*index_hd*4-byte tile).  Needs rows
 *                 a multiple of 64, and block_size (paged) or seq_stride (contiguous,
 *                 B > 1) a multiple of 64.  One lane per key then reads its key's four
 *                 dims from 1 KB contiguous per instruction: the indexer's fast layout. */
typedef enum { MLA_IC_ROWS = 0, MLA_IC_TILE64 = 1 } mla_ic_layout;
typedef struct {
    const void *lc;
    const void *rc;
    const float *ic;
    int64_t rows;             /* rows in each pool                                      */
    mla_dtype kv_dtype;       /* dtype of lc and rc                                     */
    int32_t index_hd;         /* width of an ic row (0 if ic is NULL)                   */
    const int32_t *block_table; /* device [B][max_blocks], or NULL for contiguous       */
    int32_t block_size;       /* tokens per block (paged)                               */
    int32_t max_blocks;       /* block-table row length (paged)                         */
    int64_t seq_stride;       /* rows between consecutive sequences (contiguous)        */
    const int32_t *seq_len;   /* device [B]                                             */
    int64_t max_seq_len;      /* host bound: every seq_len[b] <= max_seq_len            */
    int32_t ic_layout;        /* mla_ic_layout of the ic pool                           */
} mla_kv_view;

/* ---------------------------------------------------------------------------------
 * Interleaved partial RoPE, in place.  [MLA] sec. 2.1 (rope_interleave): only the
 * qk_rope tail of each head rotates; the even/odd input pair (a, b) = (x[2j], x[2j+1])
 * of the tail becomes out[j] = a*cos - b*sin, out[half+j] = b*cos + a*sin, half =
 * rope_dim/2, angle = pos * theta^(-2j/rope_dim) (angle formed in double).  Used on each
 * query head's tail (rope_off = qk_nope) and on the shared key Rc (n_heads = 1).
 *   x          device, dtype dt; element (n, h, e) at n*tok_stride + h*head_stride + e
 *   pos        device int32 [n_tok], the token positions
 *   rope_dim   even, 2..512; dims outside [rope_off, rope_off+rope_dim) are untouched
 * --------------------------------------------------------------------------------- */
mla_status mla_rope_interleave(void *x, mla_dtype dt, int64_t n_tok, int32_t n_heads,
                               int64_t tok_stride, int64_t head_stride, int32_t rope_off,
                               int32_t rope_dim, const int32_t *pos, double theta,
                               void *stream);

/* ---------------------------------------------------------------------------------
 * Cache write of new tokens.  [MLA] sec. 2.1 (KV path: the kv_a output comp[kv_lora + qk_rope]
 * splits into a kv_lora part, RMS-normalised (kv_a_ln) into the latent row Lc[pos], and a qk_rope
 * part, rotated by the interleaved RoPE shared by all heads into Rc[pos]) and sec. 2.2 (indexer
 * key: the ix_wk output, LayerNorm'd and rotated, into Ic[pos]).  For token j:
 *   row      = the view's row of (sequence seq[j], position pos[j]); tokens whose row falls
 *              outside the view (seq outside [0, n_seq), a block-table hole, a row outside the
 *              pools) are skipped
 *   Lc[row]  = comp[j][0:kv_lora] / sqrt(mean(comp[j][0:kv_lora]^2) + eps_kv) * kv_gain
 *   Rc[row]  = RoPE(comp[j][kv_lora:], pos[j])          (exactly as mla_rope_interleave)
 *   Ic[row]  = RoPE over dims [ix_rope_off, ix_rope_off + ix_rope_dim) at pos[j] of
 *              (ik[j] - mean) / sqrt(var + eps_ix) * ix_gamma + ix_beta   (var: mean square
 *              deviation; nothing rotates when ix_rope_dim = 0)
 * in fp32 arithmetic, stored in kv->kv_dtype (Lc, Rc) and fp32 (Ic, either ic_layout).
 *   comp     device [n_tok][kv_lora + qk_rope], in_dt;  ik: device [n_tok][kv->index_hd], in_dt,
 *            or NULL (Ic not written)
 *   seq, pos device int32 [n_tok]
 *   kv_gain  device fp32 [kv_lora] or NULL (ones); ix_gamma / ix_beta device fp32 [index_hd] or
 *            NULL (ones / zeros)
 *   eps_kv, eps_ix  positive (the page gives 1e-6); theta as for mla_rope_interleave
 *   kv       host struct: the pools written (lc, rc, and ic when ik is given); seq_len is not read
 * Two tokens with the same row race (their order is unspecified).
 * Supported: kv_lora <= 2048, qk_rope <= 512 (even), index_hd a multiple of 4 up to 256.
 * --------------------------------------------------------------------------------- */
mla_status mla_cache_write(const void *comp, const void *ik, mla_dtype in_dt, int64_t n_tok,
                           const int32_t *seq, const int32_t *pos, int32_t n_seq, int32_t kv_lora,
                           int32_t qk_rope, const float *kv_gain, const float *ix_gamma,
                           const float *ix_beta, int32_t ix_rope_off, int32_t ix_rope_dim,
                           double eps_kv, double eps_ix, double theta, const mla_kv_view *kv,
                           void *stream);

/* ---------------------------------------------------------------------------------
 * DSA lightning-indexer scores.  [MLA] sec. 2.2: per query and causal key t, a
 * ReLU-gated, per-head-weighted score; [FDSA] sec. 2: the key cache Ic is fp32.
 *   scores[b][t] = sum_h w_idx[b][h] * ReLU( sum_d q_idx[b][h][d] * Ic(b,t)[d] )
 * evaluated in fp32 in a FIXED order (heads ascending; dims ascending; one fused
 * multiply-add per product; ReLU; one fused multiply-add per head weight), so that the
 * result is reproducible bit for bit and the selected key set is exact.
 *   q_idx   device fp32 [B][n_ih][kv->index_hd]
 *   w_idx   device fp32 [B][n_ih]
 *   kv      host struct; kv->ic, kv->index_hd, layout and seq_len are used
 *   scores  device fp32 [B][t_max]; t < min(seq_len[b], t_max) get the score, the rest of
 *           the row is set to -INFINITY
 * Supported: 1 <= n_ih <= 64, index_hd a multiple of 4 in [4, 256].
 * --------------------------------------------------------------------------------- */
mla_status dsa_index_scores(const float *q_idx, const float *w_idx, int32_t B, int32_t n_ih,
                            const mla_kv_view *kv, int64_t t_max, float *scores, void *stream);

/* ---------------------------------------------------------------------------------
 * Top-k causal key selection.  [MLA] sec. 2.2 (sort + threshold scan into
 * dsa_sel / dsa_nsel; the top-2048 causal keys).  For each row b, among
 * t < n = min(n_valid[b], t_max): order by score descending, then position ascending
 * (-0.0 equals +0.0); keep the first nsel[b] = min(k, n); write them to sel[b][0..nsel)
 * sorted by position ascending; sel[b][nsel..k) = -1.  No full sort is performed.
 *   scores   device fp32 [B][t_max] (NaN is outside the contract)
 *   n_valid  device int32 [B] (for decode: seq_len)
 *   sel      device int32 [B][k];  nsel: device int32 [B]
 *   ws       device workspace of at least dsa_topk_workspace_bytes(B, t_max, k) bytes
 * Supported: 1 <= k <= 65536, t_max < 2^31.
 * --------------------------------------------------------------------------------- */
size_t dsa_topk_workspace_bytes(int32_t B, int64_t t_max, int32_t k);
mla_status dsa_topk_select(const float *scores, int32_t B, int64_t t_max,
                           const int32_t *n_valid, int32_t k, int32_t *sel, int32_t *nsel,
                           void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------------
 * The indexer and the top-k of every row in one call ([MLA] sec. 2.2: score every causal key,
 * keep the top-k).  The result equals dsa_index_scores(...) followed by dsa_topk_select(...)
 * with n_valid[b] = the row's causal length (seq_len[b], or max_seq_len without seq_len,
 * clamped to [0, t_max]): the same scores, the same sel and nsel, bit for bit.  Fewer passes
 * over the scores: the first histogram of the selection is taken while the scores are
 * produced.
 *   q_idx, w_idx, kv, t_max, scores   as for dsa_index_scores (scores is written too)
 *   k, sel, nsel                      as for dsa_topk_select
 *   ws   device workspace of at least dsa_index_select_workspace_bytes(B, t_max, k) bytes
 *        (its content on entry does not matter; it is scratch)
 * Supported: 1 <= k <= 65536, t_max < 2^31 (rows up to 262144 keys take the single-pass
 * selection, longer ones the general top-k).
 * --------------------------------------------------------------------------------- */
size_t dsa_index_select_workspace_bytes(int32_t B, int64_t t_max, int32_t k);
mla_status dsa_index_select(const float *q_idx, const float *w_idx, int32_t B, int32_t n_ih,
                            const mla_kv_view *kv, int64_t t_max, int32_t k, float *scores,
                            int32_t *sel, int32_t *nsel, void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------------
 * Absorbed MLA decode, one query per sequence.  [MLA] sec. 2.3 (absorbed path):
 *   q_abs[b][h]   = W_UK[h]^T q_nope[b][h]                    (fold W_UK into the query)
 *   s[b][h][t]    = sm_scale * (q_abs[b][h] . Lc(b,t) + q_rope[b][h] . Rc(b,t))
 *   p             = softmax over the attended keys t
 *   clat[b][h]    = sum_t p[b][h][t] Lc(b,t)                   (softmax-weighted latent)
 *   out[b][h]     = W_UV[h] clat[b][h]                         (apply W_UV)
 * with W_UK[h] = kv_b rows [h*(qk_nope+v_head), +qk_nope) and W_UV[h] = the following
 * v_head rows ([MLA] sec. 2: kvb_dim = H*(qk_nope+v_head)).
 * Attended keys: sel == NULL -> every t < seq_len[b] (dense causal);
 *                sel != NULL -> the positions sel[b*sel_stride + j], j < nsel[b]
 *                (logical positions; entries >= seq_len[b] or < 0 are skipped).
 *   q_nope  device [B][H][qk_nope], q_rope device [B][H][qk_rope] (already rotated), q_dt
 *   kv_b    device [H*(qk_nope+v_head)][kv_lora], w_dt
 *   out     device fp32 [B][H][v_head]
 *   ws      workspace of at least mla_decode_workspace_bytes(d, B, max_keys) bytes, where
 *           max_keys bounds the keys one sequence attends (sel_stride, or max_seq_len)
 * A sequence with no attended key produces zeros.  q_dt, w_dt and kv->kv_dtype must match.
 * --------------------------------------------------------------------------------- */
size_t mla_decode_workspace_bytes(const mla_dims *d, int32_t B, int64_t max_keys);
mla_status mla_absorbed_decode(const void *q_nope, const void *q_rope, mla_dtype q_dt,
                               const void *kv_b, mla_dtype w_dt, const mla_dims *d, int32_t B,
                               const mla_kv_view *kv, const int32_t *sel, const int32_t *nsel,
                               int32_t sel_stride, float sm_scale, float *out, void *ws,
                               size_t ws_bytes, void *stream);
/* The same decode in its two steps, for callers that overlap the query absorption with other
 * work (it needs neither the cache nor the selection, e.g. it can run on a second stream
 * while dsa_index_scores and dsa_topk_select run):
 *   mla_decode_absorb   q_abs = W_UK^T q_nope into the workspace       ([MLA] sec. 2.3, first step)
 *   mla_decode_attend   everything after it, reading q_abs from the same workspace
 * Arguments mean what they mean for mla_absorbed_decode.  The two calls must see the same
 * d, B, dtypes and kv_b, and the same ws (of at least mla_decode_workspace_bytes(d, B,
 * max_keys) bytes; the absorb step alone uses only its first part), in stream order, and
 * with no other decode on that workspace in between. */
mla_status mla_decode_absorb(const void *q_nope, mla_dtype q_dt, const void *kv_b, mla_dtype w_dt,
                             const mla_dims *d, int32_t B, void *ws, size_t ws_bytes, void *stream);
mla_status mla_decode_attend(const void *q_rope, mla_dtype q_dt, const void *kv_b, mla_dtype w_dt,
                             const mla_dims *d, int32_t B, const mla_kv_view *kv, const int32_t *sel,
                             const int32_t *nsel, int32_t sel_stride, float sm_scale, float *out, void *ws,
                             size_t ws_bytes, void *stream);


/* ---------------------------------------------------------------------------------
 * The whole DSA decode step in one call, for one query per sequence at its position
 * seq_len[b] - 1 ([MLA] sec. 2.1 RoPE, sec. 2.2 indexer and top-k, sec. 2.3 absorbed path):
 *   1. q_rope' = RoPE(q_rope) at position seq_len[b] - 1 (as mla_rope_interleave, written
 *      to the workspace: q_rope itself is not modified)
 *   2. scores, sel, nsel = dsa_index_select(q_idx, w_idx, kv, t_max, k)
 *   3. out = mla_absorbed_decode(q_nope, q_rope', sel, nsel) over the selected keys
 * Rows with seq_len[b] <= k keep every key (sel = 0..seq_len-1), which is the dense decode.
 * The results equal those of the separate calls bit for bit; the call only schedules
 * them together (on the matrix-core decode path the query absorption and the rotation run
 * beside the selection's final pass instead of as launches of their own).
 *   q_nope, q_rope, q_dt, kv_b, w_dt, d, B, sm_scale   as for mla_absorbed_decode (q_rope
 *                                                     before rotation), rope_theta as the
 *                                                     theta of mla_rope_interleave
 *   q_idx, w_idx, n_ih, kv, t_max, k, scores, sel, nsel as for dsa_index_select (kv must
 *                                                     carry Lc, Rc, Ic and seq_len; sel is
 *                                                     [B][k]); t_max >= every seq_len[b]
 *   out   device fp32 [B][H][v_head]
 *   ws    device workspace of at least mla_dsa_decode_workspace_bytes(d, B, t_max, k)
 *         bytes (scratch; its content on entry does not matter)
 * --------------------------------------------------------------------------------- */
size_t mla_dsa_decode_workspace_bytes(const mla_dims *d, int32_t B, int64_t t_max, int32_t k);
mla_status mla_dsa_decode(const void *q_nope, const void *q_rope, mla_dtype q_dt, double rope_theta,
                          const float *q_idx, const float *w_idx, int32_t n_ih, const void *kv_b,
                          mla_dtype w_dt, const mla_dims *d, int32_t B, const mla_kv_view *kv,
                          int64_t t_max, int32_t k, float sm_scale, float *scores, int32_t *sel,
                          int32_t *nsel, float *out, void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------------
 * The decode step of a DSA-shared layer.  [MLA] sec. 2.2: the indexer runs on the full layers
 * only; the shared layers that follow reuse its selection (dsa_sel / dsa_nsel).  Equals
 * mla_rope_interleave (on a copy of q_rope, at position seq_len[b] - 1) followed by
 * mla_absorbed_decode over the keys sel[b][0 .. nsel[b]) of this layer's own cache, bit for bit.
 *   sel, nsel  device int32 [B][k], [B]: INPUTS (e.g. the sel / nsel an earlier mla_dsa_decode of
 *              the same step wrote); entries outside [0, seq_len[b]) are skipped
 *   other arguments as for mla_dsa_decode (kv needs Lc, Rc and seq_len; Ic is not read)
 *   ws         device workspace of at least mla_dsa_decode_shared_workspace_bytes(d, B, k) bytes
 * --------------------------------------------------------------------------------- */
size_t mla_dsa_decode_shared_workspace_bytes(const mla_dims *d, int32_t B, int32_t k);
mla_status mla_dsa_decode_shared(const void *q_nope, const void *q_rope, mla_dtype q_dt, double rope_theta,
                                 const void *kv_b, mla_dtype w_dt, const mla_dims *d, int32_t B,
                                 const mla_kv_view *kv, const int32_t *sel, const int32_t *nsel, int32_t k,
                                 float sm_scale, float *out, void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------------
 * mla_dsa_decode without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, serving loops or harnesses that forbid hipMalloc).  Same
 * arguments, results (bit for bit) and errors as mla_dsa_decode, minus ws / ws_bytes: the scratch
 * is a static device array of the library, 64 MiB (MLA_NOALLOC_SCRATCH_BYTES), one copy per GPU,
 * held from the library's first use on that GPU until the process ends.  The call uses the copy of
 * the calling thread's current device (the stream must belong to it), allocates nothing and calls
 * no allocating routine.  A step whose workspace (mla_dsa_decode_workspace_bytes) exceeds the
 * array returns MLA_ERR_WORKSPACE: at the GLM geometry that admits e.g. B = 8 at t_max = 131072,
 * k = 2048 (57.3 MiB).  Every call on a GPU shares that GPU's array: calls that overlap on one GPU
 * (two streams, two threads) race; calls in stream order do not.
 * --------------------------------------------------------------------------------- */
#define MLA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
mla_status mla_dsa_decode_noalloc(const void *q_nope, const void *q_rope, mla_dtype q_dt, double rope_theta,
                                  const float *q_idx, const float *w_idx, int32_t n_ih, const void *kv_b,
                                  mla_dtype w_dt, const mla_dims *d, int32_t B, const mla_kv_view *kv,
                                  int64_t t_max, int32_t k, float sm_scale, float *scores, int32_t *sel,
                                  int32_t *nsel, float *out, void *stream);

/* ---------------------------------------------------------------------------------
 * Non-absorbed causal prefill of S queries of one sequence.  [MLA] sec. 2.3
 * (non-absorbed path): one kv_b matmul rebuilds k_nope and v for every token,
 *   [k_nope | v](t, h) = kv_b[h*(qk_nope+v_head) .. +qk_nope+v_head) . Lc(t),
 * then causal attention: query i sits at position pos_base + i ([MLA] sec. 2:
 * Tk = pos_base + S) and attends keys t <= pos_base + i with
 *   s = sm_scale * (q[i][h][:qk_nope] . k_nope(t,h) + q[i][h][qk_nope:] . Rc(t)),
 * softmax, out[i][h] = sum_t p v(t,h).
 *   q     device [S][H][qk_nope+qk_rope] (tail already rotated), q_dt
 *   kv    host struct for sequence 0 (seq_len is not read); rows 0..pos_base+S-1 used.
 *         Every position 0..pos_base+S-1 must map to a pool row: a block-table hole there
 *         gives unspecified values (never an access outside the pools).
 *   out   device [S][H][v_head], out_dt
 *   ws    workspace of at least mla_prefill_workspace_bytes(d, S, pos_base+S) bytes
 * q_dt, w_dt and kv->kv_dtype must match.
 * --------------------------------------------------------------------------------- */
size_t mla_prefill_workspace_bytes(const mla_dims *d, int32_t S, int64_t T);
mla_status mla_prefill_nonabsorbed(const void *q, mla_dtype q_dt, const void *kv_b,
                                   mla_dtype w_dt, const mla_dims *d, const mla_kv_view *kv,
                                   int32_t S, int32_t pos_base, float sm_scale, void *out,
                                   mla_dtype out_dt, void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------------
 * Attention of S queries of one sequence, on the path the g_absorb rule picks.  [MLA] sec. 2
 * (attention over Tk = pos_base + S keys; query i at position pos_base + i sees keys 0 .. pos_base
 * + i) and sec. 2.3 (g_absorb: -1 auto = absorbed when S <= 4, the decode and draft-verification
 * case; 0 never; 1 always).  Both paths compute the same function (they differ in rounding only):
 *   absorbed      q_abs = W_UK^T q_nope per query and head, scores against Lc / Rc, softmax,
 *                 latent accumulation, W_UV (as mla_absorbed_decode, one query per position)
 *   non-absorbed  one kv_b matmul rebuilds k_nope and v of keys 0 .. Tk-1, then causal softmax
 *                 attention (as mla_prefill_nonabsorbed)
 * With sel != NULL (DSA, [MLA] sec. 2.2) query i attends only the keys sel[i][0 .. nsel[i]) that
 * are <= pos_base + i (entries outside that range are skipped; a query with none gives zeros).
 *   q      device [S][H][qk_nope + qk_rope] (tail already rotated), q_dt
 *   kv     host struct for sequence 0 (seq_len is not read; rows 0 .. pos_base + S - 1 used, every
 *          one mapped to a pool row)
 *   sel    device int32 [S][sel_stride] or NULL; nsel device int32 [S]; on the non-absorbed path
 *          sel_stride must stay below 2^19 (MLA_ERR_UNSUPPORTED otherwise)
 *   out    device fp32 [S][H][v_head]
 *   ws     at least mla_attention_workspace_bytes(d, S, pos_base, sel ? sel_stride : 0, g_absorb)
 * mla_attention_absorbs(S, g_absorb) returns 1 when the call takes the absorbed path.
 * --------------------------------------------------------------------------------- */
int32_t mla_attention_absorbs(int32_t S, int32_t g_absorb);
size_t mla_attention_workspace_bytes(const mla_dims *d, int32_t S, int32_t pos_base, int32_t sel_stride,
                                     int32_t g_absorb);
mla_status mla_attention(const void *q, mla_dtype q_dt, const void *kv_b, mla_dtype w_dt, const mla_dims *d,
                         const mla_kv_view *kv, int32_t S, int32_t pos_base, const int32_t *sel,
                         const int32_t *nsel, int32_t sel_stride, float sm_scale, int32_t g_absorb, float *out,
                         void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------------
 * DSA selection for S queries of one sequence (prefill).  [MLA] sec. 2.2: the indexer is active
 * whenever the context exceeds the top-k, prefill included; every query keeps its own top-k
 * causal keys.  Query i sits at position pos_base + i: row i of the result equals dsa_index_select
 * for a sequence of pos_base + i + 1 keys with query q_idx[i], w_idx[i] -- the same scores
 * (bit for bit, -INFINITY past the row's causal end), sel and nsel (= min(k, pos_base + i + 1)).
 *   q_idx   device fp32 [S][n_ih][kv->index_hd];  w_idx device fp32 [S][n_ih]
 *   kv      host struct for sequence 0 (Ic used; seq_len is not read)
 *   scores  device fp32 [S][pos_base + S];  sel device int32 [S][k];  nsel device int32 [S]
 *   ws      at least dsa_prefill_select_workspace_bytes(S, pos_base, k) bytes
 * --------------------------------------------------------------------------------- */
size_t dsa_prefill_select_workspace_bytes(int32_t S, int32_t pos_base, int32_t k);
mla_status dsa_prefill_select(const float *q_idx, const float *w_idx, int32_t n_ih, const mla_kv_view *kv,
                              int32_t S, int32_t pos_base, int32_t k, float *scores, int32_t *sel,
                              int32_t *nsel, void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------------
 * Absorbed decode with a quantized kv_b.  [MLA] sec. 2.3: the absorbed path touches kv_b only in
 * the per-head products qt_addrow (W_UK folded into the query) and qt_matvec_rows (W_UV applied to
 * the latent), over quantized rows; [FDSA] sec. 3 and 5: int8 / FP8 / MXFP4 are bounded-loss forms
 * of the same weights, each gated by a correctness check.  The result is mla_absorbed_decode's with
 * kv_b replaced by the decoded weights (a row of kv_b = kv_lora columns, rows as in kv_b):
 *   MLA_Q_FP8_E4M3  codes [N][kv_lora] bytes, OCP FP8 E4M3 (no infinities; the NaN codes 0x7F / 0xFF
 *                   are outside the contract); scales fp32 [N]: w = scales[row] * e4m3(code)
 *   MLA_Q_INT8      codes [N][kv_lora] signed bytes; scales fp32 [N]: w = scales[row] * code
 *   MLA_Q_MXFP4     OCP Microscaling MXFP4: codes [N][kv_lora / 2] bytes, FP4 E2M1, column 2i in the
 *                   low nibble of byte i; scales [N][kv_lora / 32] E8M0 bytes (255 = NaN, outside the
 *                   contract): w = 2^(scale - 127) * e2m1(nibble)
 * with N = n_heads * (qk_nope + v_head).  Products and sums run in fp32 (q_abs rounded to bf16 for
 * the matrix cores, as on the bf16 path).  codes and scales are device pointers, 4-byte aligned.
 * Supported: bf16 queries and cache, 64 heads, kv_lora 512, qk_rope 64, qk_nope a multiple of 8 up
 * to 256, v_head a multiple of 32.  Other arguments and the workspace size as for
 * mla_absorbed_decode (mla_decode_workspace_bytes).
 * mla_dsa_decode_q is mla_dsa_decode with such a kv_b (the same scores, sel and nsel, bit for bit).
 * --------------------------------------------------------------------------------- */
typedef enum { MLA_Q_FP8_E4M3 = 1, MLA_Q_INT8 = 2, MLA_Q_MXFP4 = 3 } mla_qformat;
typedef struct {
    const void *codes;
    const void *scales;
    int32_t format;   /* mla_qformat */
} mla_qweights;
mla_status mla_absorbed_decode_q(const void *q_nope, const void *q_rope, mla_dtype q_dt, const mla_qweights *kv_b,
                                 const mla_dims *d, int32_t B, const mla_kv_view *kv, const int32_t *sel,
                                 const int32_t *nsel, int32_t sel_stride, float sm_scale, float *out, void *ws,
                                 size_t ws_bytes, void *stream);
mla_status mla_dsa_decode_q(const void *q_nope, const void *q_rope, mla_dtype q_dt, double rope_theta,
                            const float *q_idx, const float *w_idx, int32_t n_ih, const mla_qweights *kv_b,
                            const mla_dims *d, int32_t B, const mla_kv_view *kv, int64_t t_max, int32_t k,
                            float sm_scale, float *scores, int32_t *sel, int32_t *nsel, float *out, void *ws,
                            size_t ws_bytes, void *stream);

/* Human-readable name of a status, and the detail of the last failure on this thread. */
const char *mla_status_string(mla_status s);
const char *mla_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MLA_DSA_H */
