/*
 * moe_oracle.c -- CPU oracle of one MoE feed-forward layer pass.
 *
 * TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the CPU
 * baseline leg of the benchmark call it; the library's compute path never
 * does, and this file shares no code, header or table with the HIP kernels.
 *
 * Plain loops, one token and one expert at a time, float64 accumulation.
 * Inputs are fp32 or bf16 bit patterns; bf16 is decoded exactly (its 16 bits
 * are the top half of an fp32).  Weights may also be FP8 E4M3 codes (the OCP
 * 8-bit float: 1 sign, 4 exponent bits with bias 7, 3 mantissa bits, no
 * infinities, S.1111.111 = NaN) with one fp32 scale per matrix row, the
 * weight being code value * row scale -- weight quantization, the decode-phase
 * remedy of the notes ("量子化").  Where the pages leave a step open the reading
 * taken is stated at the function.
 *
 * What it computes, and where the pages define it:
 *  - routing and top-K selection: named as auxiliary kernels in the talk notes
 *    on "Demystifying the Mixture of Experts Serving Tax" (Table 1, auxiliary
 *    kernels row; finding 5, Fig. 5).  The gating function is not given there;
 *    the reading is softmax over all E logits, the K largest, renormalised to
 *    sum to one.
 *  - alignment with block-wise padding: same notes, "Padding model (Section
 *    5.1)": each expert's token count N_i is rounded up to a multiple of the
 *    block B, P = sum_i ceil(N_i / B) * B.
 *  - expert FFN: the notes give only the "MoE intermediate size" (Table 2);
 *    the reading is a bias-free SwiGLU, y = W2 (silu(W1 x) * (W3 x)).
 *  - combine ("local sum", finding 5): out_t = sum_k w[t,k] y[t,k] (+ shared).
 *  - DenseFA (section "定義"): the same SwiGLU with the intermediate size
 *    scaled by top-K (plus the shared width), applied to every token.
 *  - per-token routing budget: the MoE-Prism page treats the routing top-k
 *    as a runtime knob chosen per request, so one batch mixes budgets.  The
 *    reading: token t routes exactly as above with K = k_t (its request's
 *    budget, 0 <= k_t <= Kmax), its unused slots k_t..Kmax-1 hold no expert
 *    (id -1, weight 0) and are left out of the alignment and the combine.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_FP8 = 2 };

static size_t elem_size(int dt) { return dt == ORC_F32 ? 4 : dt == ORC_BF16 ? 2 : 1; }

/* Value of an FP8 E4M3 code, from the format's definition. */
double orc_fp8_e4m3(uint8_t b)
{
    const int sgn = b >> 7, e = (b >> 3) & 15, m = b & 7;
    double v;
    if (e == 15 && m == 7)
        v = NAN;
    else if (e == 0)
        v = ldexp((double)m, -9);           /* subnormal: m/8 * 2^-6 */
    else
        v = ldexp((double)(8 + m), e - 10); /* (1 + m/8) * 2^(e-7) */
    return sgn ? -v : v;
}

/* Element i of an fp32, bf16 or FP8 array, as a double (exact in every case). */
static double elem(const void *p, int dt, int64_t i)
{
    if (dt == ORC_F32)
        return (double)((const float *)p)[i];
    if (dt == ORC_FP8)
        return orc_fp8_e4m3(((const uint8_t *)p)[i]);
    uint32_t bits = (uint32_t)((const uint16_t *)p)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* Row `row` (length n) of a row-major matrix, decoded to doubles; with a
 * per-row scale (quantized weights) each element is code value * scale[row]. */
static void decode_row(const void *m, int dt, int64_t row, int64_t n, double *dst,
                       const float *scale)
{
    const double sc = scale ? (double)scale[row] : 1.0;
    for (int64_t c = 0; c < n; ++c)
        dst[c] = elem(m, dt, row * n + c) * sc;
}

/* out[j] = sum_c M[row0 + j][c] * v[c] over c ascending, for j < nrows. */
static void matvec(const void *m, int dt, const float *scale, int64_t row0, int64_t nrows,
                   int64_t ncols, const double *v, double *rowbuf, double *out)
{
    for (int64_t j = 0; j < nrows; ++j) {
        decode_row(m, dt, row0 + j, ncols, rowbuf, scale);
        double s = 0.0;
        for (int64_t c = 0; c < ncols; ++c)
            s += rowbuf[c] * v[c];
        out[j] = s;
    }
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

/*
 * One SwiGLU expert applied to one token vector xv[H]:
 *   g_i = sum_h W1[i][h] x[h],  u_i = sum_h W3[i][h] x[h]   (W1 = rows 0..I-1
 *   of w13, W3 = rows I..2I-1), a_i = silu(g_i) * u_i,
 *   y_h = sum_i W2[h][i] a_i   (w2 is [H][I], out x in, row-major).
 * w13/w2 point at this expert's matrices; s13 [2I] / s2 [H] are their row
 * scales (NULL for fp32/bf16 weights).  scratch holds 3*I + max(H,I) doubles.
 */
static void swiglu_token(const double *xv, int H, int I, const void *w13, const void *w2, int wdt,
                         const float *s13, const float *s2, double *scratch, double *y)
{
    double *g = scratch, *u = scratch + I, *a = scratch + 2 * (int64_t)I;
    double *rowbuf = scratch + 3 * (int64_t)I;
    matvec(w13, wdt, s13, 0, I, H, xv, rowbuf, g);
    matvec(w13, wdt, s13, I, I, H, xv, rowbuf, u);
    for (int i = 0; i < I; ++i)
        a[i] = silu(g[i]) * u[i];
    matvec(w2, wdt, s2, 0, H, I, a, rowbuf, y);
}

static size_t swiglu_scratch(int H, int I) { return 3 * (size_t)I + (size_t)(H > I ? H : I); }

void orc_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int orc_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Routing of T tokens over E experts, K per token.
 *   p_e = exp(l_e - max l) / sum_e exp(l_e - max l)        (softmax, e ascending)
 *   the K selected experts are the K largest by the key (l_e descending, e
 *   ascending); slot j holds the j-th of them in that order;
 *   w_j = p_{e_j} / sum_{i<K} p_{e_i}                       (renormalised)
 * The selection compares the fp32 logits themselves: softmax is increasing,
 * so the K largest logits are the K largest probabilities, and ties between
 * equal logits go to the lower expert id (IEEE comparison, -0 == +0).
 * Returns 0, -1 if K is outside [1, E], -3 if out of host memory.
 */
int orc_route(const float *logits, int64_t T, int E, int K, int32_t *ids, double *w);

/*
 * Routing with a per-token budget: token t takes k_t = k_tok[t], clamped to
 * [0, Kmax], experts, selected and renormalised as by orc_route with K = k_t;
 * slots k_t .. Kmax-1 of its row hold id -1 and weight 0.  ids and w are
 * [T][Kmax].  Returns 0, -1 if Kmax is outside [1, E], -3 if out of host
 * memory.
 */
int orc_route_var(const float *logits, int64_t T, int E, int Kmax, const int32_t *k_tok,
                  int32_t *ids, double *w)
{
    if (E < 1 || Kmax < 1 || Kmax > E || T < 0)
        return -1;
    for (int64_t t = 0; t < T; ++t) {
        int k = k_tok[t] < 0 ? 0 : (k_tok[t] > Kmax ? Kmax : k_tok[t]);
        if (k > 0 && orc_route(logits + t * E, 1, E, k, ids + t * Kmax, w + t * Kmax) != 0)
            return -3;
        for (int j = k; j < Kmax; ++j) {
            ids[t * Kmax + j] = -1;
            w[t * Kmax + j] = 0.0;
        }
    }
    return 0;
}

int orc_route(const float *logits, int64_t T, int E, int K, int32_t *ids, double *w)
{
    if (E < 1 || K < 1 || K > E || T < 0)
        return -1;
    double *p = malloc(sizeof(double) * (size_t)E);
    unsigned char *taken = malloc((size_t)E);
    if (!p || !taken) {
        free(p);
        free(taken);
        return -3;
    }
    for (int64_t t = 0; t < T; ++t) {
        const float *l = logits + t * E;
        double m = l[0];
        for (int e = 1; e < E; ++e)
            if (l[e] > m)
                m = l[e];
        double z = 0.0;
        for (int e = 0; e < E; ++e) {
            p[e] = exp((double)l[e] - m);
            z += p[e];
        }
        for (int e = 0; e < E; ++e)
            p[e] /= z;

        memset(taken, 0, (size_t)E);
        double s = 0.0;
        for (int j = 0; j < K; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e)           /* strict '>' keeps the lowest id among equals */
                if (!taken[e] && (best < 0 || l[e] > l[best]))
                    best = e;
            taken[best] = 1;
            ids[t * K + j] = best;
            s += p[best];
        }
        for (int j = 0; j < K; ++j)
            w[t * K + j] = p[ids[t * K + j]] / s;
    }
    free(p);
    free(taken);
    return 0;
}

/*
 * Alignment of the T*K (token, slot) pairs p = t*K + k into expert buckets,
 * padded as in the padding model of the Serving-tax notes (Section 5.1):
 *   N_e = #{p : ids[p] = e};
 *   block-wise (mode 0): P_e = ceil(N_e / B) * B;
 *   max (mode 1):        P_e = ceil(max_i N_i / B) * B for every expert, so
 *                        the total is E * ceil(max_i N_i / B) * B;
 *   offsets[0] = 0, offsets[e+1] = offsets[e] + P_e, num_padded = offsets[E];
 *   bucket e holds its pairs in ascending p at rows offsets[e] ..
 *   offsets[e] + N_e - 1; every other row below cap holds the sentinel T*K;
 *   block_expert[b] = e for the blocks of bucket e and -1 past num_padded;
 *   inv_pos[p] = the row that holds p.
 * A pair with a negative id is an unused slot (per-token budget): it is in no
 * bucket and inv_pos[p] = -1.
 * cap must be a multiple of B.  Returns 0, -1 on bad arguments (an id >= E
 * among them), -2 if the padded total exceeds cap, -3 if out of host memory.
 */
int orc_align_mode(const int32_t *ids, int64_t T, int K, int E, int B, int64_t cap, int mode,
                   int32_t *counts, int32_t *offsets, int32_t *sorted_ids,
                   int32_t *block_expert, int32_t *inv_pos)
{
    if (T < 0 || K < 1 || E < 1 || B < 1 || cap < 0 || cap % B != 0 || mode < 0 || mode > 1)
        return -1;
    const int64_t TK = T * K;
    for (int e = 0; e < E; ++e)
        counts[e] = 0;
    for (int64_t p = 0; p < TK; ++p) {
        if (ids[p] >= E)
            return -1;
        if (ids[p] >= 0)
            counts[ids[p]] += 1;
    }
    int32_t maxn = 0;
    for (int e = 0; e < E; ++e)
        if (counts[e] > maxn)
            maxn = counts[e];
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) {
        int64_t padded = (int64_t)((mode == 1 ? maxn : counts[e]) + B - 1) / B * B;
        if (offsets[e] + padded > cap)
            return -2;
        offsets[e + 1] = (int32_t)(offsets[e] + padded);
    }
    for (int64_t r = 0; r < cap; ++r)
        sorted_ids[r] = (int32_t)TK;
    int32_t *fill = calloc((size_t)E, sizeof(int32_t));
    if (!fill)
        return -3;
    for (int64_t p = 0; p < TK; ++p) {
        int e = ids[p];
        if (e < 0) {
            inv_pos[p] = -1;
            continue;
        }
        int64_t r = offsets[e] + fill[e];
        fill[e] += 1;
        sorted_ids[r] = (int32_t)p;
        inv_pos[p] = (int32_t)r;
    }
    free(fill);
    for (int64_t b = 0; b < cap / B; ++b)
        block_expert[b] = -1;
    for (int e = 0; e < E; ++e)
        for (int64_t b = offsets[e] / B; b < offsets[e + 1] / B; ++b)
            block_expert[b] = e;
    return 0;
}

int orc_align(const int32_t *ids, int64_t T, int K, int E, int B, int64_t cap, int32_t *counts,
              int32_t *offsets, int32_t *sorted_ids, int32_t *block_expert, int32_t *inv_pos)
{
    return orc_align_mode(ids, T, K, E, B, cap, 0, counts, offsets, sorted_ids, block_expert,
                          inv_pos);
}

/*
 * y[r][:] = SwiGLU(x[r][:]) for n rows with one set of weights
 * (w13 [2I][H] gate rows then up rows, w2 [H][I]).  Serves a single expert,
 * the shared experts and DenseFA.  Parallel over rows.  Returns 0, or -3 if
 * a thread's buffers could not be allocated (y is then incomplete).
 */
int orc_swiglu_s(const void *x, int xdt, int64_t n, int H, int I, const void *w13,
                 const void *w2, int wdt, const float *s13, const float *s2, double *y)
{
    int rc = 0;
#pragma omp parallel
    {
        double *xv = malloc(sizeof(double) * (size_t)H);
        double *scratch = malloc(sizeof(double) * swiglu_scratch(H, I));
        if (!xv || !scratch) {
#pragma omp atomic write
            rc = -3;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < n; ++r) {
            if (!xv || !scratch)
                continue;
            decode_row(x, xdt, r, H, xv, NULL);
            swiglu_token(xv, H, I, w13, w2, wdt, s13, s2, scratch, y + r * H);
        }
        free(xv);
        free(scratch);
    }
    return rc;
}

int orc_swiglu(const void *x, int xdt, int64_t n, int H, int I, const void *w13, const void *w2,
               int wdt, double *y)
{
    return orc_swiglu_s(x, xdt, n, H, I, w13, w2, wdt, NULL, NULL, y);
}

/*
 * out[t][h] = sum_{k ascending} w[t][k] * y[t*K + k][h]  (+ s[t][h] if s);
 * slots of weight 0 (unused slots of a per-token budget) are skipped, their
 * rows of y never read.
 */
void orc_combine(const double *y, const double *w, const double *s, int64_t T, int K, int H,
                 double *out)
{
    for (int64_t t = 0; t < T; ++t)
        for (int h = 0; h < H; ++h) {
            double acc = 0.0;
            for (int k = 0; k < K; ++k)
                if (w[t * K + k] != 0.0)
                    acc += w[t * K + k] * y[(t * K + k) * H + h];
            out[t * H + h] = acc + (s ? s[t * H + h] : 0.0);
        }
}

/*
 * The whole layer for T tokens, one token at a time: route the token, run
 * each of its K experts on it, add the shared experts (weight 1, width Is;
 * Is = 0 for none), and combine.  w13 is [E][2I][H], w2 is [E][H][I]; for FP8
 * weights s13 [E][2I], s2 [E][H], ss13 [2Is], ss2 [H] are the row scales
 * (NULL otherwise).  ids_out/w_out (nullable) receive the routing.  Returns 0,
 * -1 on bad arguments, -3 if out of host memory (out is then incomplete).
 */
int orc_moe_layer_k(const void *x, int xdt, const float *logits, const int32_t *k_tok, int64_t T,
                    int H, int I, int E, int K, const void *w13, const void *w2, int wdt,
                    const float *s13, const float *s2, int Is, const void *ws13, const void *ws2,
                    const float *ss13, const float *ss2, int32_t *ids_out, double *w_out,
                    double *out);

int orc_moe_layer_s(const void *x, int xdt, const float *logits, int64_t T, int H, int I, int E,
                    int K, const void *w13, const void *w2, int wdt, const float *s13,
                    const float *s2, int Is, const void *ws13, const void *ws2, const float *ss13,
                    const float *ss2, int32_t *ids_out, double *w_out, double *out)
{
    return orc_moe_layer_k(x, xdt, logits, NULL, T, H, I, E, K, w13, w2, wdt, s13, s2, Is, ws13,
                           ws2, ss13, ss2, ids_out, w_out, out);
}

/*
 * orc_moe_layer_s with a per-token budget k_tok [T] (NULL: K for every
 * token): token t is routed with orc_route_var (K = Kmax) and combines only
 * its k_t experts; ids_out / w_out rows carry -1 / 0 in the unused slots.
 */
int orc_moe_layer_k(const void *x, int xdt, const float *logits, const int32_t *k_tok, int64_t T,
                    int H, int I, int E, int K, const void *w13, const void *w2, int wdt,
                    const float *s13, const float *s2, int Is, const void *ws13, const void *ws2,
                    const float *ss13, const float *ss2, int32_t *ids_out, double *w_out,
                    double *out)
{
    if (E < 1 || K < 1 || K > E || T < 0)
        return -1;
    const size_t esize = elem_size(wdt);
    int rc = 0;  /* written by any thread that fails, with an atomic write */
#pragma omp parallel
    {
        double *xv = malloc(sizeof(double) * (size_t)H);
        int Imax = I > Is ? I : Is;
        double *scratch = malloc(sizeof(double) * swiglu_scratch(H, Imax));
        double *y = malloc(sizeof(double) * (size_t)H * (size_t)(K + 1));
        int32_t *ids = malloc(sizeof(int32_t) * (size_t)K);
        double *w = malloc(sizeof(double) * (size_t)K);
        const int have = xv && scratch && y && ids && w;
        if (!have) {
#pragma omp atomic write
            rc = -3;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < T; ++t) {
            if (!have)
                continue;
            const int32_t kt = k_tok ? k_tok[t] : K;
            const int rr = orc_route_var(logits + t * E, 1, E, K, &kt, ids, w);
            if (rr != 0) {
#pragma omp atomic write
                rc = rr;
                continue;
            }
            decode_row(x, xdt, t, H, xv, NULL);
            for (int k = 0; k < K; ++k) {
                if (ids[k] < 0)
                    continue;   /* an unused slot of the token's budget */
                const char *e13 = (const char *)w13 + (size_t)ids[k] * 2 * I * H * esize;
                const char *e2 = (const char *)w2 + (size_t)ids[k] * H * I * esize;
                const float *es13 = s13 ? s13 + (size_t)ids[k] * 2 * I : NULL;
                const float *es2 = s2 ? s2 + (size_t)ids[k] * H : NULL;
                swiglu_token(xv, H, I, e13, e2, wdt, es13, es2, scratch, y + (size_t)k * H);
            }
            double *s = NULL;
            if (Is > 0) {
                s = y + (size_t)K * H;
                swiglu_token(xv, H, Is, ws13, ws2, wdt, ss13, ss2, scratch, s);
            }
            orc_combine(y, w, s, 1, K, H, out + t * H);
            if (ids_out)
                memcpy(ids_out + t * K, ids, sizeof(int32_t) * (size_t)K);
            if (w_out)
                memcpy(w_out + t * K, w, sizeof(double) * (size_t)K);
        }
        free(xv);
        free(scratch);
        free(y);
        free(ids);
        free(w);
    }
    return rc;
}

int orc_moe_layer(const void *x, int xdt, const float *logits, int64_t T, int H, int I, int E,
                  int K, const void *w13, const void *w2, int wdt, int Is, const void *ws13,
                  const void *ws2, int32_t *ids_out, double *w_out, double *out)
{
    return orc_moe_layer_s(x, xdt, logits, T, H, I, E, K, w13, w2, wdt, NULL, NULL, Is, ws13, ws2,
                           NULL, NULL, ids_out, w_out, out);
}
