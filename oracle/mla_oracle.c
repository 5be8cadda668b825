/*
 * mla_oracle.c -- plain, slow, CPU reference for the MLA + DSA decode/prefill path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product (the HIP library and its Python
 * binding) may include, link, load or call this file.  Only the test suite, the smoke
 * check and the CPU-baseline leg of the benchmark use it.  It shares no code, header,
 * table or helper with the GPU path.
 *
 * Sources (the text of public web pages; cited by page title and section):
 *   [P2]  chen3feng, "colibri-analysis 06: MLA attention and KV cache"
 *         sec. 1   compressed KV cache: each token keeps a kv_lora latent (Lc) and one
 *                  qk_rope key shared by all heads (Rc); k_nope and v are rebuilt via kv_b.
 *         sec. 2   attention() dimensions: kvb_dim = H*(qk_nope+v_head), Tk = pos_base+S.
 *         sec. 2.1 interleaved partial RoPE (only the qk_rope tail of each head rotates;
 *                  even/odd input pairs (a,b) go to v[j]=a*cs-b*sn, v[half+j]=b*cs+a*sn).
 *         sec. 2.2 DSA lightning indexer: ReLU-gated per-head-weighted scores over the
 *                  indexer-key cache Ic, top-2048 causal keys by sort + threshold scan.
 *         sec. 2.3 absorbed path (fold W_UK into the query, score against Lc/Rc, accumulate
 *                  the latent, apply W_UV) and non-absorbed path (one kv_b matmul rebuilds
 *                  k_nope and v for all tokens, then causal softmax attention with
 *                  score = q_pass.k_nope + q_rot.k_rot).
 *   [P1]  aiknowledge.cn, "Ch.7 sec. 03: token-exact forward validation and faithful DSA"
 *         sec. 2   Ic is stored at index_hd x 4 bytes (fp32) per token per DSA layer.
 *
 * Readings taken where the pages are silent (each is restated at its function):
 *   - softmax scale is an argument; no extra scale in the indexer;
 *   - RoPE frequency theta^(-2j/rope_dim), angle computed in double;
 *   - the indexer is fixed-order fp32: heads ascending, dims ascending, one fmaf per
 *     product, ReLU, then one fmaf per head weight -- this order is the contract that
 *     makes the selected index set reproducible bit for bit;
 *   - top-k: score descending, position ascending on ties (-0.0 == +0.0), output sorted by
 *     position, nsel = min(k, n_valid);
 *   - kv_b rows are head-major blocks of (qk_nope + v_head) rows: first the W_UK rows of
 *     that head, then its W_UV rows;
 *   - a decode query sees every cached key including its own (keys 0..seq_len-1).
 *
 * Floating point: everything except the indexer's fp32 contract is computed in double.
 * Inputs arrive as float arrays (fp32 values, or bf16 values widened exactly to fp32).
 * Build: gcc -O2 -ffp-contract=off -fopenmp, no fast-math.  Parallel loops only run
 * independent units (keys, heads, tokens); every sum is taken in index order.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void orc_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ------------------------------------------------------------------------------------
 * Interleaved partial RoPE  [P2 sec. 2.1]
 * x, y: [n_tok][n_heads][head_dim] (double).  Only dims [rope_off, rope_off+rope_dim)
 * rotate; every other dim is copied.  Pair j takes input (a, b) = (x[2j], x[2j+1]) of the
 * tail and writes y[j] = a cos(phi) - b sin(phi), y[half + j] = b cos(phi) + a sin(phi),
 * phi = pos * theta^(-2j / rope_dim)  (frequency formula: reading, the page gives none).
 * ----------------------------------------------------------------------------------*/
void orc_rope_interleave(const double *x, double *y, int64_t n_tok, int32_t n_heads,
                         int32_t head_dim, int32_t rope_off, int32_t rope_dim,
                         const int32_t *pos, double theta)
{
    const int32_t half = rope_dim / 2;
    for (int64_t n = 0; n < n_tok; ++n) {
        for (int32_t h = 0; h < n_heads; ++h) {
            const double *xi = x + (n * n_heads + h) * (int64_t)head_dim;
            double *yo = y + (n * n_heads + h) * (int64_t)head_dim;
            for (int32_t d = 0; d < head_dim; ++d) yo[d] = xi[d];
            for (int32_t j = 0; j < half; ++j) {
                double inv = pow(theta, -2.0 * (double)j / (double)rope_dim);
                double phi = (double)pos[n] * inv;
                double c = cos(phi), s = sin(phi);
                double a = xi[rope_off + 2 * j];
                double b = xi[rope_off + 2 * j + 1];
                yo[rope_off + j] = a * c - b * s;
                yo[rope_off + half + j] = b * c + a * s;
            }
        }
    }
}

/* ------------------------------------------------------------------------------------
 * DSA lightning-indexer scores  [P2 sec. 2.2; P1 sec. 2 for fp32 Ic]
 *   I[t] = sum_h w[h] * ReLU( sum_d q[h][d] * Ic[t][d] )
 * in the fixed fp32 order: s = +0; for h ascending { a = +0; for d ascending
 * a = fmaf(q[h][d], Ic[t][d], a); r = (a > 0) ? a : +0; s = fmaf(w[h], r, s); }.
 * q: [n_ih][hd], w: [n_ih], ic: [T][hd], out: [T].
 * ----------------------------------------------------------------------------------*/
void orc_index_scores_f32(const float *q, const float *w, const float *ic, int64_t T,
                          int32_t n_ih, int32_t hd, float *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const float *k = ic + t * (int64_t)hd;
        float s = 0.0f;
        for (int32_t h = 0; h < n_ih; ++h) {
            float a = 0.0f;
            for (int32_t d = 0; d < hd; ++d) a = fmaf(q[h * hd + d], k[d], a);
            float r = (a > 0.0f) ? a : 0.0f;
            s = fmaf(w[h], r, s);
        }
        out[t] = s;
    }
}

/* The same scores in double (a sanity reference for the fp32 error bound). */
void orc_index_scores_f64(const float *q, const float *w, const float *ic, int64_t T,
                          int32_t n_ih, int32_t hd, double *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const float *k = ic + t * (int64_t)hd;
        double s = 0.0;
        for (int32_t h = 0; h < n_ih; ++h) {
            double a = 0.0;
            for (int32_t d = 0; d < hd; ++d) a += (double)q[h * hd + d] * (double)k[d];
            s += (double)w[h] * (a > 0.0 ? a : 0.0);
        }
        out[t] = s;
    }
}

/* ------------------------------------------------------------------------------------
 * Top-k causal key selection  [P2 sec. 2.2: "qsort + threshold scan" into dsa_sel/dsa_nsel]
 * Sort (score, position) by score descending, position ascending; keep the first
 * nsel = min(k, n_valid); return those positions sorted ascending.  -0.0 and +0.0 compare
 * equal (IEEE comparison).  sel[nsel..k) is filled with -1.  Returns nsel.
 * ----------------------------------------------------------------------------------*/
typedef struct {
    float s;
    int32_t t;
} orc_pair;

static int orc_cmp_pair(const void *pa, const void *pb)
{
    const orc_pair *a = (const orc_pair *)pa, *b = (const orc_pair *)pb;
    if (a->s > b->s) return -1;
    if (a->s < b->s) return 1;
    return (a->t > b->t) - (a->t < b->t);
}

static int orc_cmp_i32(const void *pa, const void *pb)
{
    int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
    return (a > b) - (a < b);
}

int32_t orc_topk(const float *scores, int64_t n_valid, int32_t k, int32_t *sel)
{
    int64_t nsel = n_valid < (int64_t)k ? n_valid : (int64_t)k;
    if (nsel < 0) nsel = 0;
    orc_pair *p = (orc_pair *)malloc(sizeof(orc_pair) * (size_t)(n_valid > 0 ? n_valid : 1));
    for (int64_t t = 0; t < n_valid; ++t) {
        p[t].s = scores[t];
        p[t].t = (int32_t)t;
    }
    qsort(p, (size_t)n_valid, sizeof(orc_pair), orc_cmp_pair);
    for (int64_t i = 0; i < nsel; ++i) sel[i] = p[i].t;
    qsort(sel, (size_t)nsel, sizeof(int32_t), orc_cmp_i32);
    for (int64_t i = nsel; i < k; ++i) sel[i] = -1;
    free(p);
    return (int32_t)nsel;
}

void orc_topk_batch(const float *scores, int32_t B, int64_t t_max, const int32_t *n_valid,
                    int32_t k, int32_t *sel, int32_t *nsel)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t b = 0; b < B; ++b)
        nsel[b] = orc_topk(scores + (int64_t)b * t_max, n_valid[b], k, sel + (int64_t)b * k);
}

/* ------------------------------------------------------------------------------------
 * Absorbed MLA decode for one query  [P2 sec. 2.3, absorbed path]
 *   q_abs[h][c]  = sum_i q_nope[h][i] * W_UK[h][i][c]          (fold W_UK into the query)
 *   s[h][t]      = sm_scale * (q_abs[h] . Lc[t] + q_rope[h] . Rc[t])
 *   p            = softmax over the key set (max subtracted)
 *   clat[h][c]   = sum_t p[h][t] * Lc[t][c]                     (softmax-weighted latent)
 *   out[h][j]    = sum_c W_UV[h][j][c] * clat[h][c]             (apply W_UV)
 * W_UK[h] = kv_b rows [h*(nope+v), h*(nope+v)+nope), W_UV[h] = the next v rows.
 * q_nope: [H][nope], q_rope: [H][rope] (already rotated), kv_b: [H*(nope+v)][L],
 * lc: [*][L], rc: [*][rope], keys: the n_keys cached positions attended (any order),
 * out: [H][v] double.
 * ----------------------------------------------------------------------------------*/
void orc_absorbed_decode(const float *q_nope, const float *q_rope, const float *kv_b,
                         const float *lc, const float *rc, const int32_t *keys, int64_t n_keys,
                         int32_t H, int32_t nope, int32_t rope, int32_t v, int32_t L,
                         double sm_scale, double *out)
{
    const int64_t rows_per_head = (int64_t)nope + v;
#pragma omp parallel for schedule(static)
    for (int32_t h = 0; h < H; ++h) {
        double *qabs = (double *)calloc((size_t)L, sizeof(double));
        double *clat = (double *)calloc((size_t)L, sizeof(double));
        double *s = (double *)malloc(sizeof(double) * (size_t)(n_keys > 0 ? n_keys : 1));
        const float *wuk = kv_b + (int64_t)h * rows_per_head * L;
        const float *wuv = wuk + (int64_t)nope * L;
        for (int32_t i = 0; i < nope; ++i) {
            double qi = (double)q_nope[(int64_t)h * nope + i];
            for (int32_t c = 0; c < L; ++c) qabs[c] += qi * (double)wuk[(int64_t)i * L + c];
        }
        double m = -INFINITY;
        for (int64_t j = 0; j < n_keys; ++j) {
            const float *l = lc + (int64_t)keys[j] * L;
            const float *r = rc + (int64_t)keys[j] * rope;
            double dl = 0.0, dr = 0.0;
            for (int32_t c = 0; c < L; ++c) dl += qabs[c] * (double)l[c];
            for (int32_t c = 0; c < rope; ++c) dr += (double)q_rope[(int64_t)h * rope + c] * (double)r[c];
            s[j] = sm_scale * (dl + dr);
            if (s[j] > m) m = s[j];
        }
        double den = 0.0;
        for (int64_t j = 0; j < n_keys; ++j) {
            double p = exp(s[j] - m);
            den += p;
            const float *l = lc + (int64_t)keys[j] * L;
            for (int32_t c = 0; c < L; ++c) clat[c] += p * (double)l[c];
        }
        for (int32_t c = 0; c < L; ++c) clat[c] /= den;
        for (int32_t jv = 0; jv < v; ++jv) {
            double acc = 0.0;
            for (int32_t c = 0; c < L; ++c) acc += (double)wuv[(int64_t)jv * L + c] * clat[c];
            out[(int64_t)h * v + jv] = acc;
        }
        free(qabs);
        free(clat);
        free(s);
    }
}

/* ------------------------------------------------------------------------------------
 * Non-absorbed MLA attention for one query  [P2 sec. 2.3, non-absorbed path]
 * Rebuilds k_nope[t][h] = W_UK[h] Lc[t] and v[t][h] = W_UV[h] Lc[t] per key, then plain
 * softmax attention with score = sm_scale * (q_nope . k_nope + q_rope . Rc[t]).
 * Same arguments and output as orc_absorbed_decode.
 * ----------------------------------------------------------------------------------*/
void orc_nonabsorbed_decode(const float *q_nope, const float *q_rope, const float *kv_b,
                            const float *lc, const float *rc, const int32_t *keys, int64_t n_keys,
                            int32_t H, int32_t nope, int32_t rope, int32_t v, int32_t L,
                            double sm_scale, double *out)
{
    const int64_t rows_per_head = (int64_t)nope + v;
#pragma omp parallel for schedule(static)
    for (int32_t h = 0; h < H; ++h) {
        double *kn = (double *)malloc(sizeof(double) * (size_t)(nope > 0 ? nope : 1));
        double *vv = (double *)malloc(sizeof(double) * (size_t)v);
        double *s = (double *)malloc(sizeof(double) * (size_t)(n_keys > 0 ? n_keys : 1));
        double *acc = (double *)calloc((size_t)v, sizeof(double));
        const float *wuk = kv_b + (int64_t)h * rows_per_head * L;
        const float *wuv = wuk + (int64_t)nope * L;
        double m = -INFINITY;
        for (int64_t j = 0; j < n_keys; ++j) {
            const float *l = lc + (int64_t)keys[j] * L;
            const float *r = rc + (int64_t)keys[j] * rope;
            double dn = 0.0, dr = 0.0;
            for (int32_t i = 0; i < nope; ++i) {
                double a = 0.0;
                for (int32_t c = 0; c < L; ++c) a += (double)wuk[(int64_t)i * L + c] * (double)l[c];
                kn[i] = a;
            }
            for (int32_t i = 0; i < nope; ++i) dn += (double)q_nope[(int64_t)h * nope + i] * kn[i];
            for (int32_t c = 0; c < rope; ++c) dr += (double)q_rope[(int64_t)h * rope + c] * (double)r[c];
            s[j] = sm_scale * (dn + dr);
            if (s[j] > m) m = s[j];
        }
        double den = 0.0;
        for (int64_t j = 0; j < n_keys; ++j) {
            const float *l = lc + (int64_t)keys[j] * L;
            for (int32_t jv = 0; jv < v; ++jv) {
                double a = 0.0;
                for (int32_t c = 0; c < L; ++c) a += (double)wuv[(int64_t)jv * L + c] * (double)l[c];
                vv[jv] = a;
            }
            double p = exp(s[j] - m);
            den += p;
            for (int32_t jv = 0; jv < v; ++jv) acc[jv] += p * vv[jv];
        }
        for (int32_t jv = 0; jv < v; ++jv) out[(int64_t)h * v + jv] = acc[jv] / den;
        free(kn);
        free(vv);
        free(s);
        free(acc);
    }
}

/* ------------------------------------------------------------------------------------
 * Non-absorbed causal prefill, evaluated on a subset of query rows  [P2 sec. 2, 2.3]
 * Query i sits at position pos_base + i and attends keys t = 0 .. pos_base + i.
 * Step 1 (the kv_b matmul): for every needed token t and head h,
 *   k_nope[t][h][i] = sum_c W_UK[h][i][c] Lc[t][c],  v[t][h][j] = sum_c W_UV[h][j][c] Lc[t][c]
 * each sum in ascending c.  Step 2: per row and head, softmax over the causal keys of
 *   sm_scale * (q[i][h][:nope] . k_nope[t][h] + q[i][h][nope:] . Rc[t]), then sum p v.
 * q: [S][H][nope+rope] (tail already rotated), lc: [T][L], rc: [T][rope], rows: n_rows query
 * indices in [0, S), out: [n_rows][H][v] double.
 * ----------------------------------------------------------------------------------*/
void orc_prefill_rows(const float *q, const float *kv_b, const float *lc, const float *rc,
                      int32_t S, int32_t pos_base, int32_t H, int32_t nope, int32_t rope,
                      int32_t v, int32_t L, double sm_scale, const int32_t *rows,
                      int32_t n_rows, double *out)
{
    const int32_t R = nope + v; /* kv_b rows per head */
    const int32_t qh = nope + rope;
    int32_t max_row = -1;
    for (int32_t r = 0; r < n_rows; ++r)
        if (rows[r] > max_row) max_row = rows[r];
    if (max_row < 0) return;
    (void)S;
    const int64_t Tn = (int64_t)pos_base + max_row + 1; /* keys any requested row can see */
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t h = 0; h < H; ++h) {
        /* kv_b block of head h, stored column-major (wt[c][r]) so that the per-token
         * rebuild below walks it contiguously; values are the same kv_b entries. */
        double *wt = (double *)malloc(sizeof(double) * (size_t)L * R);
        const float *wh = kv_b + (int64_t)h * R * L;
        for (int32_t r = 0; r < R; ++r)
            for (int32_t c = 0; c < L; ++c) wt[(int64_t)c * R + r] = (double)wh[(int64_t)r * L + c];
        double *kv = (double *)malloc(sizeof(double) * (size_t)Tn * R); /* [t][k_nope | v] */
        for (int64_t t = 0; t < Tn; ++t) {
            double *o = kv + t * R;
            for (int32_t r = 0; r < R; ++r) o[r] = 0.0;
            const float *l = lc + t * L;
            for (int32_t c = 0; c < L; ++c) {
                double lv = (double)l[c];
                const double *wc = wt + (int64_t)c * R;
                for (int32_t r = 0; r < R; ++r) o[r] += wc[r] * lv;
            }
        }
        double *s = (double *)malloc(sizeof(double) * (size_t)Tn);
        double *acc = (double *)malloc(sizeof(double) * (size_t)v);
        for (int32_t ri = 0; ri < n_rows; ++ri) {
            const int32_t i = rows[ri];
            const int64_t nk = (int64_t)pos_base + i + 1;
            const float *qi = q + ((int64_t)i * H + h) * qh;
            double m = -INFINITY;
            for (int64_t t = 0; t < nk; ++t) {
                const double *kt = kv + t * R;
                const float *r = rc + t * rope;
                double dn = 0.0, dr = 0.0;
                for (int32_t d = 0; d < nope; ++d) dn += (double)qi[d] * kt[d];
                for (int32_t d = 0; d < rope; ++d) dr += (double)qi[nope + d] * (double)r[d];
                s[t] = sm_scale * (dn + dr);
                if (s[t] > m) m = s[t];
            }
            double den = 0.0;
            for (int32_t j = 0; j < v; ++j) acc[j] = 0.0;
            for (int64_t t = 0; t < nk; ++t) {
                double p = exp(s[t] - m);
                den += p;
                const double *vt = kv + t * R + nope;
                for (int32_t j = 0; j < v; ++j) acc[j] += p * vt[j];
            }
            double *o = out + ((int64_t)ri * H + h) * v;
            for (int32_t j = 0; j < v; ++j) o[j] = acc[j] / den;
        }
        free(wt);
        free(kv);
        free(s);
        free(acc);
    }
}

/* ------------------------------------------------------------------------------------
 * Tiny full MLA layer (projections around the hot path)  [P2 sec. 2.1, 2.3 (o projection)]
 * For every token t < T with hidden state x[t] (hidden wide):
 *   Q path : qa = q_a x;  qn = RMSNorm(qa);  qfull = q_b qn  -> [H][nope+rope]
 *   KV path: comp = kv_a x -> [L + rope];  Lc[t] = RMSNorm(comp[:L]);  Rc[t] = RoPE(comp[L:])
 * RMSNorm(u) = u / sqrt(mean(u^2) + eps) with unit gain (eps: reading, 1e-6).
 * The query of the last token gets its qk_rope tail rotated at position T-1.
 * Outputs (double): lc [T][L], rc [T][rope] (rotated), q [H][nope+rope] (tail rotated),
 * which the caller feeds to the attention functions above; o_proj is applied by
 * orc_o_proj.  Weights are row-major [out][in].
 * ----------------------------------------------------------------------------------*/
static void orc_matvec(const float *W, const double *x, int32_t n_out, int32_t n_in, double *y)
{
    for (int32_t r = 0; r < n_out; ++r) {
        double a = 0.0;
        for (int32_t c = 0; c < n_in; ++c) a += (double)W[(int64_t)r * n_in + c] * x[c];
        y[r] = a;
    }
}

static void orc_rmsnorm(double *u, int32_t n, double eps)
{
    double ms = 0.0;
    for (int32_t i = 0; i < n; ++i) ms += u[i] * u[i];
    ms /= (double)n;
    double inv = 1.0 / sqrt(ms + eps);
    for (int32_t i = 0; i < n; ++i) u[i] *= inv;
}

void orc_tiny_layer(const float *x, int32_t T, int32_t hidden, const float *q_a, int32_t q_lora,
                    const float *q_b, const float *kv_a, int32_t H, int32_t nope, int32_t rope,
                    int32_t L, double eps, double theta, double *lc, double *rc, double *q)
{
    const int32_t qh = nope + rope;
    double *xd = (double *)malloc(sizeof(double) * (size_t)hidden);
    double *qa = (double *)malloc(sizeof(double) * (size_t)q_lora);
    double *comp = (double *)malloc(sizeof(double) * (size_t)(L + rope));
    double *qf = (double *)malloc(sizeof(double) * (size_t)H * qh);
    for (int32_t t = 0; t < T; ++t) {
        for (int32_t i = 0; i < hidden; ++i) xd[i] = (double)x[(int64_t)t * hidden + i];
        orc_matvec(kv_a, xd, L + rope, hidden, comp);
        orc_rmsnorm(comp, L, eps);
        for (int32_t c = 0; c < L; ++c) lc[(int64_t)t * L + c] = comp[c];
        int32_t pos = t;
        orc_rope_interleave(comp + L, rc + (int64_t)t * rope, 1, 1, rope, 0, rope, &pos, theta);
        if (t == T - 1) {
            orc_matvec(q_a, xd, q_lora, hidden, qa);
            orc_rmsnorm(qa, q_lora, eps);
            orc_matvec(q_b, qa, H * qh, q_lora, qf);
            orc_rope_interleave(qf, q, 1, H, qh, nope, rope, &pos, theta);
        }
    }
    free(xd);
    free(qa);
    free(comp);
    free(qf);
}

/* Output projection  [P2 sec. 2.3: both paths end with the o projection]
 * y[hidden] = o_w[hidden][H*v] . attn[H*v] */
void orc_o_proj(const float *o_w, const double *attn, int32_t hidden, int32_t hv, double *y)
{
    orc_matvec(o_w, attn, hidden, hv, y);
}

/* ------------------------------------------------------------------------------------
 * Cache write of new tokens  [P2 sec. 2.1 KV path; sec. 2.2 indexer key]
 * For each new token j (sequence seq[j], position pos[j]) with kv_a output comp[j] (L + rope
 * wide) and indexer key projection ik[j] (hd wide, the ix_wk output):
 *   Lc[row]  = RMSNorm(comp[0:L]) * kv_gain           (u / sqrt(mean(u^2) + eps_kv))
 *   Rc[row]  = RoPE(comp[L:L+rope]) at pos[j]          (interleaved, as orc_rope_interleave)
 *   Ic[row]  = RoPE over dims [ix_off, ix_off + ix_rdim) of
 *              LayerNorm(ik) = (ik - mean) / sqrt(var + eps_ix) * gamma + beta   (var: mean of
 *              squared deviations), at pos[j]
 * row = block_table[seq*max_blocks + pos/bs]*bs + pos%bs (paged, bt != NULL) or
 * seq*seq_stride + pos (contiguous); a row outside [0, rows) is skipped.  kv_gain, gamma, beta
 * NULL mean ones / ones / zeros; ik NULL skips Ic.  Pools are double [rows][width].
 * Readings: the pages name RMSNorm(kv_a_ln) and "layernorm(eps 1e-6) + RoPE" without the
 * rotated slice of the indexer key; the slice is an argument (the MLA query puts its rotated
 * part in the tail), both eps are arguments (1e-6 is the only value the pages give).
 * ----------------------------------------------------------------------------------*/
void orc_cache_write(const float *comp, const float *ik, int64_t n, const int32_t *seq, const int32_t *pos,
                     int32_t L, int32_t rope, int32_t hd, const float *kv_gain, const float *gamma,
                     const float *beta, int32_t ix_off, int32_t ix_rdim, double eps_kv, double eps_ix,
                     double theta, const int32_t *bt, int32_t bs, int32_t max_blocks, int64_t seq_stride,
                     int64_t rows, double *lc, double *rc, double *ic)
{
    double *u = (double *)malloc(sizeof(double) * (size_t)(L + rope + hd + 1));
    double *y = (double *)malloc(sizeof(double) * (size_t)(hd + rope + 1));
    for (int64_t j = 0; j < n; ++j) {
        int64_t row;
        if (bt) {
            int32_t blk = bt[(int64_t)seq[j] * max_blocks + pos[j] / bs];
            row = blk < 0 ? -1 : (int64_t)blk * bs + pos[j] % bs;
        } else {
            row = (int64_t)seq[j] * seq_stride + pos[j];
        }
        if (row < 0 || row >= rows) continue;
        const float *cj = comp + j * (int64_t)(L + rope);
        double ms = 0.0;
        for (int32_t c = 0; c < L; ++c) ms += (double)cj[c] * (double)cj[c];
        ms /= (double)L;
        double inv = 1.0 / sqrt(ms + eps_kv);
        for (int32_t c = 0; c < L; ++c)
            lc[row * L + c] = (double)cj[c] * inv * (kv_gain ? (double)kv_gain[c] : 1.0);
        for (int32_t c = 0; c < rope; ++c) u[c] = (double)cj[L + c];
        orc_rope_interleave(u, rc + row * rope, 1, 1, rope, 0, rope, pos + j, theta);
        if (!ik) continue;
        const float *kj = ik + j * (int64_t)hd;
        double mean = 0.0, var = 0.0;
        for (int32_t c = 0; c < hd; ++c) mean += (double)kj[c];
        mean /= (double)hd;
        for (int32_t c = 0; c < hd; ++c) var += ((double)kj[c] - mean) * ((double)kj[c] - mean);
        var /= (double)hd;
        double is = 1.0 / sqrt(var + eps_ix);
        for (int32_t c = 0; c < hd; ++c)
            y[c] = ((double)kj[c] - mean) * is * (gamma ? (double)gamma[c] : 1.0) + (beta ? (double)beta[c] : 0.0);
        orc_rope_interleave(y, ic + row * hd, 1, 1, hd, ix_off, ix_rdim, pos + j, theta);
    }
    free(u);
    free(y);
}

/* ------------------------------------------------------------------------------------
 * Quantized kv_b rows  [P1 sec. 3 item 1 and sec. 5: int8 / FP8 / MXFP4 weight formats, each
 * a bounded-loss representation of the same weights; P2 sec. 2.3: the absorbed path reads kv_b
 * through qt_addrow / qt_matvec_rows over quantized rows]
 * The pages name the formats, not their layout; the definitions used (readings):
 *   fmt 1  FP8 E4M3 (OCP 8-bit floating point, "fn": no infinities, S.1111.111 is NaN):
 *          code byte b: s = b>>7, e = (b>>3)&15, m = b&7; e == 0: (-1)^s m 2^-9;
 *          else (-1)^s (1 + m/8) 2^(e-7).  One fp32 scale per row: w = scale[row] * value.
 *   fmt 2  INT8: w = scale[row] * (signed byte).
 *   fmt 3  MXFP4 (OCP Microscaling v1.0): blocks of 32 consecutive elements of a row share an
 *          E8M0 scale byte x (2^(x-127); 255 is NaN); elements are FP4 E2M1, two per byte (the
 *          even element in the low nibble): nibble n: s = n>>3, e = (n>>1)&3, m = n&1; e == 0:
 *          (-1)^s m/2; else (-1)^s (1 + m/2) 2^(e-1).
 * codes: fmt 1/2 [rows][cols] bytes, fmt 3 [rows][cols/2] bytes; scales: fmt 1/2 float [rows],
 * fmt 3 bytes [rows][cols/32].  out: double [rows][cols].
 * ----------------------------------------------------------------------------------*/
static double orc_e4m3(uint8_t b)
{
    int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
    double v = e == 0 ? ldexp((double)m, -9) : ldexp(1.0 + (double)m / 8.0, e - 7);
    if (e == 15 && m == 7) v = NAN;
    return s ? -v : v;
}

static double orc_e2m1(unsigned n)
{
    int s = (n >> 3) & 1, e = (n >> 1) & 3, m = n & 1;
    double v = e == 0 ? 0.5 * (double)m : ldexp(1.0 + 0.5 * (double)m, e - 1);
    return s ? -v : v;
}

void orc_dequant_rows(const uint8_t *codes, const void *scales, int32_t fmt, int64_t rows, int32_t cols, double *out)
{
    for (int64_t r = 0; r < rows; ++r) {
        double *o = out + r * cols;
        if (fmt == 1 || fmt == 2) {
            double sc = (double)((const float *)scales)[r];
            const uint8_t *c = codes + r * cols;
            for (int32_t j = 0; j < cols; ++j)
                o[j] = sc * (fmt == 1 ? orc_e4m3(c[j]) : (double)(int8_t)c[j]);
        } else {
            const uint8_t *c = codes + r * (cols / 2);
            const uint8_t *x = (const uint8_t *)scales + r * (cols / 32);
            for (int32_t j = 0; j < cols; ++j) {
                unsigned nib = (j & 1) ? (c[j / 2] >> 4) : (c[j / 2] & 15);
                double sc = x[j / 32] == 255 ? NAN : ldexp(1.0, (int)x[j / 32] - 127);
                o[j] = sc * orc_e2m1(nib);
            }
        }
    }
}
