/*
 * LoopVQ CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, single-purpose C for what the LoopVQ hot path computes.  Only
 * the test suite, the package smoke check and the benchmark's CPU-baseline
 * leg load this library; the product path never does.  It shares no code,
 * header, table or helper with the HIP library: every layout rule below is
 * re-derived here from its plain statement.
 *
 * Sources (the LoopVQ pages):
 *  - LoopVQ project page (mscheong01.github.io/loopvq), "Method" and the
 *    "Overview of LoopVQ" figure: one sub-vector spans G/Tc channels at each of
 *    Tc consecutive loop steps; one index serves all of those steps; loop step
 *    t reads the shared index through its own slice of the codebook.
 *  - same page, "Component 1 -- Loop-axis vector quantization".
 *  - same page, "Serving in SGLang": "Write in bf16", "Encode in pages",
 *    "Attend from indices" (dequantised keys/values from the shared indices,
 *    merged with bf16 attention over the sink and recent tokens).
 *  - same page, "Results -- Long-context retrieval": the first 64 and the most
 *    recent 256 tokens stay bf16.
 *  - "Looped transformer cache compressed to 0.5 bits" (notatechguy.com),
 *    "How LoopVQ works": vector quantisation = replace each sub-vector by the
 *    index of an entry in a shared table.
 *
 * The pages do not state the distance, its arithmetic or the tie rule.  The
 * reading taken: squared Euclidean distance, each operation a separate IEEE
 * fp32 operation rounded to nearest even (no fused multiply-add; build with
 * -ffp-contract=off), sum over elements in ascending order, the lowest index
 * winning ties.  Attention is the exact definition on the dequantised cache,
 * accumulated in fp64 with libm exp.
 *
 * Data layouts (shared with the library's documented boundary, implemented
 * here independently):
 *  A model with R loop steps (R a multiple of Tc) keeps R / Tc index rows per
 *  token: group g covers loop steps g*Tc .. g*Tc + Tc - 1.
 *  x        bf16  [n_tokens][H][R][d] with element strides (tok, head, step),
 *                 channel stride 1
 *  codebook f32/bf16 [R][H][256][S][cg], cg = G/Tc, S = d/cg; codeword k of
 *                 (g, h, j) has entry i = t*cg + c at [g*Tc + t][h][k][j][c]
 *  index    u8    [R/Tc][B][H][T_max][S]; row = absolute token position
 *  window   bf16  [B][R][H][n_sink + n_recent][d]; sink token p in slot p,
 *                 recent token p in slot n_sink + ((p - n_sink) mod n_recent)
 *  q        bf16  [B][H][d]
 *
 * Parity pins: tests/test_oracle_encode.py, tests/test_oracle_attention.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define LVQO_CODES 256

static float bf16_bits_to_float(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Entry i of codeword k for (group g, head h, sub-vector j) as fp32
 * (conversion of bf16 to fp32 is exact): loop step r = g*Tc + i/cg. */
static float codeword_entry(const void *cb, int cb_bf16, int H, int S, int cg, int Tc,
                            int g, int h, int j, int k, int i)
{
    int r = g * Tc + i / cg, c = i % cg;
    size_t off = ((((size_t)r * H + h) * LVQO_CODES + k) * S + j) * cg + c;
    if (cb_bf16)
        return bf16_bits_to_float(((const uint16_t *)cb)[off]);
    return ((const float *)cb)[off];
}

static int check_shape(int H, int d, int Tc, int G)
{
    if (H <= 0 || d <= 0 || Tc <= 0 || G <= 0) return -1;
    if (G % Tc != 0) return -1;
    if (d % (G / Tc) != 0) return -1;
    return 0;
}

/* ---------------------------------------------------------------------------
 * Encoding: nearest codeword by squared distance.
 *   E1  x and codebook entries as fp32.
 *   E2  sub-vector j of (token n, head h, group g): x_i = X[n][h][g*Tc + t][j*cg + c],
 *       i = t*cg + c (loop-step-major, contiguous channels); its codewords
 *       are those of group g.
 *   E3  D_k = sum_{i=0}^{G-1} (x_i - c_{k,i})^2, one fp32 op at a time.
 *   E4  scan k = 0..255, keep k when D_k < best (strict): lowest index wins.
 * Writes index[g][seq][h][first_token + n][j] for every group g < R/Tc; the
 * index cache holds `batch` sequences per group.
 * ------------------------------------------------------------------------- */
int lvqo_encode(int n_heads, int head_dim, int loop_steps, int n_loops, int group,
                int cb_bf16, const void *codebook,
                const uint16_t *x, int64_t n_tokens,
                int64_t sx_tok, int64_t sx_head, int64_t sx_step,
                uint8_t *index, int64_t batch, int64_t t_max, int64_t seq, int64_t first_token,
                int n_threads)
{
    if (check_shape(n_heads, head_dim, loop_steps, group)) return -1;
    if (n_loops < loop_steps || n_loops % loop_steps != 0) return -1;
    if (seq < 0 || seq >= batch) return -1;
    if (!codebook || !x || !index || n_tokens < 0) return -1;
    if (group > 1024) return -1;
    if (first_token < 0 || first_token + n_tokens > t_max) return -1;
    const int H = n_heads, Tc = loop_steps, G = group, NG = n_loops / loop_steps;
    const int cg = G / Tc, S = head_dim / cg;
    if (n_threads < 1) n_threads = 1;

#pragma omp parallel for schedule(static) num_threads(n_threads)
    for (int64_t n = 0; n < n_tokens; ++n) {
        float xv[1024];
        for (int g = 0; g < NG; ++g)
        for (int h = 0; h < H; ++h) {
            for (int j = 0; j < S; ++j) {
                for (int t = 0; t < Tc; ++t)
                    for (int c = 0; c < cg; ++c)
                        xv[t * cg + c] = bf16_bits_to_float(
                            x[n * sx_tok + h * sx_head + (g * Tc + t) * sx_step + j * cg + c]);
                int best = 0;
                float best_d = 0.0f;
                for (int k = 0; k < LVQO_CODES; ++k) {
                    float dist = 0.0f;
                    for (int i = 0; i < G; ++i) {
                        float e = xv[i] - codeword_entry(codebook, cb_bf16, H, S, cg, Tc, g, h, j, k, i);
                        float sq = e * e;
                        dist = dist + sq;
                    }
                    if (k == 0 || dist < best_d) {
                        best = k;
                        best_d = dist;
                    }
                }
                index[((((size_t)g * batch + seq) * H + h) * t_max + first_token + n) * S + j] = (uint8_t)best;
            }
        }
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * Dense attention of one query over L keys/values (fp64):
 *   s_n = scale * sum_ch q[ch] K[n][ch]       (ch ascending)
 *   p_n = exp(s_n - max s) / sum_n' exp(s_n' - max s)
 *   out[ch] = sum_n p_n V[n][ch]              (n ascending)
 * p may be NULL.  L == 0 gives out = 0.
 * ------------------------------------------------------------------------- */
void lvqo_attend(int64_t L, int d, const double *q, const double *K, const double *V,
                 double scale, double *out, double *p)
{
    for (int ch = 0; ch < d; ++ch) out[ch] = 0.0;
    if (L <= 0) return;
    double *s = (double *)malloc((size_t)L * sizeof(double));
    double m = -INFINITY;
    for (int64_t n = 0; n < L; ++n) {
        double acc = 0.0;
        for (int ch = 0; ch < d; ++ch) acc += q[ch] * K[n * d + ch];
        s[n] = scale * acc;
        if (s[n] > m) m = s[n];
    }
    double z = 0.0;
    for (int64_t n = 0; n < L; ++n) {
        s[n] = exp(s[n] - m);
        z += s[n];
    }
    for (int64_t n = 0; n < L; ++n) {
        double pn = s[n] / z;
        if (p) p[n] = pn;
        for (int ch = 0; ch < d; ++ch) out[ch] += pn * V[n * d + ch];
    }
    free(s);
}

/* ---------------------------------------------------------------------------
 * Decode attention of loop step r (0 <= r < R) over the LoopVQ cache; its
 * index rows are those of group g = r / Tc and t = r % Tc below.
 *   D1  windows for a context of L tokens (L counts the current token):
 *       sink = [0, n_s), n_s = min(L, n_sink); VQ = [n_s, n_s + n_v) with
 *       n_v = vq_len[b] when given, else max(0, L - n_sink - n_recent);
 *       recent = [n_s + n_v, L).
 *   D2  dequantise VQ token n: Khat[n][j*cg + c] = codeword(h, j,
 *       idxK[b][h][n][j]) entry t*cg + c; likewise Vhat.  Sink and recent
 *       tokens come from the bf16 window buffers of loop step t.
 *   D3-D5  dense fp64 attention over all L tokens (lvqo_attend).
 * Grouped-query attention: n_heads query heads, n_kv_heads heads in the index
 * caches, codebooks and windows (n_kv_heads divides n_heads); query head h
 * attends over the tokens of KV head h / (n_heads / n_kv_heads).  Equal
 * counts are multi-head attention.
 * out: fp64 [B][H][d]; p_out (optional): fp64 [B][H][t_max], probability of
 * every position < L (entries >= L untouched).  Query heads [h0, h1) only.
 * Returns -1 on a shape or precondition violation.
 * ------------------------------------------------------------------------- */
int lvqo_decode_attn(int batch, int n_heads, int n_kv_heads, int head_dim, int loop_steps,
                     int n_loops, int group,
                     int n_sink, int n_recent, int64_t t_max, int cb_bf16, int loop_step,
                     const uint16_t *q, const int32_t *ctx_len, const int32_t *vq_len,
                     const uint8_t *k_index, const uint8_t *v_index,
                     const void *k_cb, const void *v_cb,
                     const uint16_t *k_win, const uint16_t *v_win,
                     double sm_scale, double *out, double *p_out,
                     int h0, int h1, int n_threads)
{
    if (check_shape(n_heads, head_dim, loop_steps, group)) return -1;
    if (n_kv_heads < 1 || n_heads % n_kv_heads != 0) return -1;
    if (n_loops < loop_steps || n_loops % loop_steps != 0) return -1;
    if (loop_step < 0 || loop_step >= n_loops) return -1;
    if (n_sink < 0 || n_recent < 1 || batch < 0) return -1;
    if (h0 < 0 || h1 > n_heads || h0 > h1) return -1;
    const int H = n_heads, Hk = n_kv_heads, d = head_dim, Tc = loop_steps, R = n_loops;
    const int g = loop_step / Tc, t = loop_step % Tc;
    const int cg = group / Tc, S = d / cg, W = n_sink + n_recent;

    for (int b = 0; b < batch; ++b) {
        int64_t L = ctx_len[b];
        if (L < 0 || L > t_max) return -1;
        int64_t n_s = L < n_sink ? L : n_sink;
        int64_t n_v = vq_len ? vq_len[b] : (L - n_sink - n_recent > 0 ? L - n_sink - n_recent : 0);
        if (n_v < 0 || n_s + n_v > L || L - n_s - n_v > n_recent) return -1;
    }
    if (n_threads < 1) n_threads = 1;
    const int units = batch * (h1 - h0);
    int status = 0;

#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads)
    for (int u = 0; u < units; ++u) {
        const int b = u / (h1 - h0), h = h0 + u % (h1 - h0);
        const int hk = h / (H / Hk);          /* the KV head this query head reads */
        const int64_t L = ctx_len[b];
        const int64_t n_s = L < n_sink ? L : n_sink;
        const int64_t n_v = vq_len ? vq_len[b]
                                   : (L - n_sink - n_recent > 0 ? L - n_sink - n_recent : 0);
        double *K = (double *)malloc((size_t)(L > 0 ? L : 1) * d * sizeof(double));
        double *V = (double *)malloc((size_t)(L > 0 ? L : 1) * d * sizeof(double));
        double *qd = (double *)malloc((size_t)d * sizeof(double));
        if (!K || !V || !qd) {
#pragma omp atomic write
            status = -2;
            free(K); free(V); free(qd);
            continue;
        }
        for (int ch = 0; ch < d; ++ch)
            qd[ch] = bf16_bits_to_float(q[((size_t)b * H + h) * d + ch]);

        for (int64_t pos = 0; pos < L; ++pos) {
            double *kr = K + pos * d, *vr = V + pos * d;
            if (pos >= n_s && pos < n_s + n_v) {
                const size_t row = ((((size_t)g * batch + b) * Hk + hk) * t_max + pos) * S;
                for (int j = 0; j < S; ++j) {
                    int ck = k_index[row + j], cv = v_index[row + j];
                    for (int c = 0; c < cg; ++c) {
                        kr[j * cg + c] = codeword_entry(k_cb, cb_bf16, Hk, S, cg, Tc, g, hk, j, ck, t * cg + c);
                        vr[j * cg + c] = codeword_entry(v_cb, cb_bf16, Hk, S, cg, Tc, g, hk, j, cv, t * cg + c);
                    }
                }
            } else {
                int64_t slot = pos < n_sink ? pos : n_sink + (pos - n_sink) % n_recent;
                const size_t base = ((((size_t)b * R + loop_step) * Hk + hk) * W + slot) * d;
                for (int ch = 0; ch < d; ++ch) {
                    kr[ch] = bf16_bits_to_float(k_win[base + ch]);
                    vr[ch] = bf16_bits_to_float(v_win[base + ch]);
                }
            }
        }
        lvqo_attend(L, d, qd, K, V, sm_scale, out + ((size_t)b * H + h) * d,
                    p_out ? p_out + ((size_t)b * H + h) * t_max : NULL);
        free(K); free(V); free(qd);
    }
    return status;
}

int lvqo_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
