/*
 * moe_oracle.c -- plain, slow CPU reference of one quantized routed-expert MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call this
 * file: it exists so that tests, the smoke check and the bench's CPU-baseline leg can
 * compare the HIP kernels against an independent evaluation of the same definition.
 * It shares no code, header, table or constant generator with the GPU library.
 *
 * What the layer computes (sources are the five web pages on Qwen3.8-Flash-Next):
 *   - every layer holds 512 routed experts; each token activates 10 of them plus one
 *     shared expert that is always on
 *       [Strata 与 Qwen3.8-Flash-Next (telli.sh), section 稀疏架构创造了机会];
 *   - a router on the GPU picks the experts
 *       [本地部署Qwen3.8-Flash-Next模型的两条路线 (blog.cycleuser.org), section 硬件形态决定了各自的走法];
 *   - expert weights are stored at 4 bit, some mixed layers at 6 bit, a dense projection
 *     at 8 bit [same blog page, section 精度和内存占用].
 * The pages give no formula for the router, the weight normalisation, the group size or
 * the scale format.  The readings taken here (plainest ones the pages support):
 *   router      logit[t][e] = sum_c x[t][c] * Wr[e][c] (+ b[e]), fp32, in the fixed
 *               summation order described at router_dot
 *   selection   the k largest fp32 logits, equal values -> lower expert index first;
 *               slot 0 holds the largest
 *   weights     softmax over the k selected logits (equal to the full softmax renormalised
 *               over the selected experts), evaluated in fp64
 *   grouping    pairs p = t*k + j stably sorted by (expert id, p)
 *   expert      y = Wd * (silu(Wg x) .* (Wu x)), weights dequantised exactly, fp64 math
 *   combine     out[t] = y_shared[t] + sum_j w[t][j] * y(t, slot j), fp64
 *   residual    (stacked-layer sweep) x_next = bf16(x + bf16(out))
 *
 * Formats (element c of row n, K = row length, groups of 32 along K):
 *   INT4_G32  byte n*K/2 + c/2; low nibble = even c, high nibble = odd c; code u in
 *             [0,15], value = s[n][c/32] * (u - 8); s is IEEE fp16
 *   INT6_G32  each group of 32 codes is a 24-byte little-endian bit string, code i of a
 *             group at bits [6i, 6i+6); value = s * (u - 32)
 *   INT3_G32  the same with 3-bit codes: 12 bytes per group, code i at bits [3i, 3i+3);
 *             value = s * (u - 4)
 *   INT2_G32  2-bit codes: 8 bytes per group, code i at bits [2i, 2i+2); value = s * (u - 2)
 *   INT8_ROW  int8 two's complement q, value = s[n] * q (s fp16, one per row)
 *   FP32      plain IEEE binary32
 * All arithmetic is plain IEEE double unless stated otherwise.  Build with
 * -O2 -fno-fast-math -ffp-contract=off so no fused or reordered arithmetic sneaks in.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OFMT_FP32 = 0, OFMT_INT8_ROW = 1, OFMT_INT4_G32 = 2, OFMT_INT6_G32 = 3,
       OFMT_INT3_G32 = 4, OFMT_INT2_G32 = 5 };

typedef struct {
    int32_t fmt;        /* OFMT_FP32 or OFMT_INT8_ROW */
    int32_t n_experts;  /* E */
    int32_t d_model;    /* d */
    int32_t pad_;
    const void* w;      /* fp32 [E][d] or int8 [E][d] */
    const uint16_t* scale; /* fp16 [E] for INT8_ROW, else unused */
    const float* bias;  /* [E] or NULL */
} oracle_router;

typedef struct {
    int32_t fmt;        /* OFMT_INT4_G32, OFMT_INT6_G32, OFMT_INT3_G32 or OFMT_INT2_G32 */
    int32_t n_experts;
    int32_t d_model;
    int32_t d_ff;
    const uint8_t* w_gate;  /* [E][d_ff][d_model packed] */
    const uint8_t* w_up;    /* [E][d_ff][d_model packed] */
    const uint8_t* w_down;  /* [E][d_model][d_ff packed] */
    const uint16_t* s_gate; /* fp16 [E][d_ff][d_model/32] */
    const uint16_t* s_up;   /* fp16 [E][d_ff][d_model/32] */
    const uint16_t* s_down; /* fp16 [E][d_model][d_ff/32] */
} oracle_experts;

/* ------------------------------------------------------------------ number formats */

/* IEEE 754 binary16 -> double, straight from the definition of the encoding. */
double oracle_half_to_double(uint16_t h)
{
    int sign = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);              /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);  /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16 is the upper half of an IEEE binary32. */
static float bf16_to_float(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Real number (given as a double) -> bfloat16 bits, round to nearest, ties to even:
 * keep 8 significant bits (the exponent range is that of binary32; below 2^-126 the
 * spacing is 2^-133).  Finite inputs only. */
uint16_t oracle_double_to_bf16(double v)
{
    double q;
    if (v == 0.0) {
        q = v;
    } else if (fabs(v) < ldexp(1.0, -126)) {
        q = rint(ldexp(v, 133)) * ldexp(1.0, -133);
    } else {
        int e;
        double m = frexp(v, &e);                 /* v = m * 2^e, 0.5 <= |m| < 1 */
        q = ldexp(rint(ldexp(m, 8)), e - 8);     /* rint: nearest, ties to even */
    }
    float f = (float)q;                           /* exact: q has <= 8 significant bits */
    if (fabs(q) >= ldexp(1.0, 128)) f = (q > 0) ? INFINITY : -INFINITY;
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

/* The same rounding over an array (n values). */
void oracle_double_to_bf16_n(const double* v, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_double_to_bf16(v[i]);
}

/* ------------------------------------------------------------------ weight codes */

/* Signed code of element c of one packed row. */
int oracle_code(int fmt, const uint8_t* row, int c)
{
    if (fmt == OFMT_INT4_G32) {
        uint8_t b = row[c / 2];
        int u = (c % 2 == 0) ? (b & 15) : (b >> 4);
        return u - 8;
    }
    if (fmt == OFMT_INT6_G32) {
        const uint8_t* g = row + (size_t)(c / 32) * 24;
        int bit = 6 * (c % 32);
        unsigned v = g[bit / 8];
        if (bit % 8 + 6 > 8)
            v |= (unsigned)g[bit / 8 + 1] << 8;
        int u = (int)((v >> (bit % 8)) & 63u);
        return u - 32;
    }
    if (fmt == OFMT_INT3_G32 || fmt == OFMT_INT2_G32) {
        /* bit by bit from the group's little-endian bit string */
        const int b = (fmt == OFMT_INT3_G32) ? 3 : 2;
        const uint8_t* g = row + (size_t)(c / 32) * (size_t)(4 * b);
        int u = 0;
        for (int j = 0; j < b; ++j) {
            int bit = b * (c % 32) + j;
            u |= ((g[bit / 8] >> (bit % 8)) & 1) << j;
        }
        return u - (1 << (b - 1));
    }
    if (fmt == OFMT_INT8_ROW)
        return (int)(int8_t)row[c];
    return 0;
}

/* Bytes of one packed row of K codes. */
static size_t row_bytes(int fmt, int K)
{
    if (fmt == OFMT_INT4_G32) return (size_t)K / 2;
    if (fmt == OFMT_INT6_G32) return (size_t)K * 3 / 4;
    if (fmt == OFMT_INT3_G32) return (size_t)K * 3 / 8;
    if (fmt == OFMT_INT2_G32) return (size_t)K / 4;
    return (size_t)K;
}

/* Dequantise row n of a grouped matrix [N][K] exactly into out[K]. */
void oracle_dequant_row(int fmt, const uint8_t* w, const uint16_t* s, int K, int64_t n,
                        double* out)
{
    const uint8_t* row = w + (size_t)n * row_bytes(fmt, K);
    const uint16_t* srow = s + (size_t)n * (K / 32);
    for (int c = 0; c < K; ++c)
        out[c] = oracle_half_to_double(srow[c / 32]) * (double)oracle_code(fmt, row, c);
}

/* ------------------------------------------------------------------ router */

/*
 * Router logits in the fixed fp32 order.  The pages place a router in front of the
 * experts but fix no summation order; because the selection compares fp32 logits, the
 * order is part of the definition here so that expert ids are reproducible bit for bit.
 *
 * The row of d weights is cut into 16-byte vectors (4 fp32 weights, or 16 int8 codes).
 * Vector v belongs to lane (v mod 64); lane l walks its vectors v = l, l+64, l+128, ...
 * in ascending order and, inside a vector, its elements in ascending order, keeping one
 * fp32 accumulator that starts at +0 and is updated with a single-rounding fused
 * multiply-add acc = fma(x_c, w_c, acc).  The 64 lane sums are then combined by a
 * butterfly: for offsets 1, 2, 4, 8, 16, 32 every lane l replaces its value by
 * a_l + a_(l xor offset).  All lanes end with the same value (addition commutes), which
 * is the dot product.  fp32: logit = dot + b.  int8: logit = fl(fl(dot * s_e) + b).
 */
static float router_dot(int fmt, const void* wrow_v, const uint16_t* x, int d)
{
    float lane[64], nxt[64];
    int per_vec = (fmt == OFMT_INT8_ROW) ? 16 : 4;
    int nvec = d / per_vec;
    for (int l = 0; l < 64; ++l) {
        float acc = 0.0f;
        for (int v = l; v < nvec; v += 64) {
            for (int i = 0; i < per_vec; ++i) {
                int c = v * per_vec + i;
                float wv = (fmt == OFMT_INT8_ROW)
                               ? (float)((const int8_t*)wrow_v)[c]
                               : ((const float*)wrow_v)[c];
                acc = fmaf(bf16_to_float(x[c]), wv, acc);
            }
        }
        lane[l] = acc;
    }
    for (int off = 1; off < 64; off *= 2) {
        for (int l = 0; l < 64; ++l)
            nxt[l] = lane[l] + lane[l ^ off];
        memcpy(lane, nxt, sizeof lane);
    }
    return lane[0];
}

void oracle_router_logits(const oracle_router* r, const uint16_t* x, int64_t T, float* logits)
{
    const int E = r->n_experts, d = r->d_model;
    const size_t wrow = (r->fmt == OFMT_INT8_ROW) ? (size_t)d : (size_t)d * 4;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int e = 0; e < E; ++e) {
            const void* w = (const char*)r->w + (size_t)e * wrow;
            float dot = router_dot(r->fmt, w, x + (size_t)t * d, d);
            float logit;
            if (r->fmt == OFMT_INT8_ROW) {
                float se = (float)oracle_half_to_double(r->scale[e]);
                logit = dot * se;
                if (r->bias) logit = logit + r->bias[e];
            } else {
                logit = dot;
                if (r->bias) logit = logit + r->bias[e];
            }
            logits[(size_t)t * E + e] = logit;
        }
    }
}

/* Same affine map evaluated in double (an audit copy: how far the fp32 value is from
 * the real-number dot product). */
void oracle_router_logits_fp64(const oracle_router* r, const uint16_t* x, int64_t T,
                               double* logits)
{
    const int E = r->n_experts, d = r->d_model;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int c = 0; c < d; ++c) {
                double wv = (r->fmt == OFMT_INT8_ROW)
                                ? (double)((const int8_t*)r->w)[(size_t)e * d + c]
                                : (double)((const float*)r->w)[(size_t)e * d + c];
                acc += (double)bf16_to_float(x[(size_t)t * d + c]) * wv;
            }
            if (r->fmt == OFMT_INT8_ROW) acc *= oracle_half_to_double(r->scale[e]);
            if (r->bias) acc += (double)r->bias[e];
            logits[(size_t)t * E + e] = acc;
        }
    }
}

/* ------------------------------------------------------------------ pre-MoE norm */

/*
 * The pages put a gated residual on the GPU next to the router and the shared expert
 * [本地部署Qwen3.8-Flash-Next模型的两条路线 (blog.cycleuser.org), section 硬件形态决定了各自的走法]
 * but give no formula for it or for the normalisation in front of the layer.  Reading: the
 * MoE layer runs on xn = RMSNorm(x), and its output joins the residual stream through a
 * per-token sigmoid gate (see oracle_gated_residual).  The norm, in fp32 with a fixed
 * order so that the routing that follows is reproducible bit for bit:
 *   ss  = sum_c x_c^2: the row cut into chunks of 4 elements, chunk v belongs to lane
 *         (v mod 64), each lane runs acc = fma(x_c, x_c, acc) over its chunks in ascending
 *         order (elements ascending), then the butterfly over lanes with offsets 1..32
 *         (the router's tree);
 *   r   = fl(1 / fl(sqrt(fl(fl(ss / d) + eps))))  (IEEE division and square root);
 *   xn_c = bf16(fl(fl(x_c * r) * gamma_c)).
 */
float oracle_rms_sumsq(const uint16_t* x, int d)
{
    float lane[64], nxt[64];
    int nchunk = d / 4;
    for (int l = 0; l < 64; ++l) {
        float acc = 0.0f;
        for (int v = l; v < nchunk; v += 64)
            for (int i = 0; i < 4; ++i) {
                float xv = bf16_to_float(x[v * 4 + i]);
                acc = fmaf(xv, xv, acc);
            }
        lane[l] = acc;
    }
    for (int off = 1; off < 64; off *= 2) {
        for (int l = 0; l < 64; ++l)
            nxt[l] = lane[l] + lane[l ^ off];
        memcpy(lane, nxt, sizeof lane);
    }
    return lane[0];
}

/* xn [T][d] (bf16 bits) and the scale r [T] (may be NULL) of T rows. */
void oracle_rmsnorm(const uint16_t* x, int64_t T, int d, const float* gamma, float eps,
                    uint16_t* xn, float* r_out)
{
    for (int64_t t = 0; t < T; ++t) {
        const uint16_t* xr = x + (size_t)t * d;
        float ss = oracle_rms_sumsq(xr, d);
        float ms = ss / (float)d;
        float den = sqrtf(ms + eps);
        float r = 1.0f / den;
        if (r_out) r_out[t] = r;
        for (int c = 0; c < d; ++c) {
            float a = bf16_to_float(xr[c]) * r;
            float b = a * gamma[c];
            xn[(size_t)t * d + c] = oracle_double_to_bf16((double)b);
        }
    }
}

/* Gated residual: x_next = bf16(x + bf16(g_t * out)), g_t = 1 / (1 + exp(-z_t)) in double
 * (z = gate logits [T], or NULL for g = 1, the plain residual).  x + bf16(...) is exact in
 * double (two bf16 values), so one rounding remains. */
void oracle_gated_residual(const uint16_t* x, const double* out, const float* z, int64_t T,
                           int d, uint16_t* x_next)
{
    for (int64_t t = 0; t < T; ++t) {
        double g = z ? 1.0 / (1.0 + exp(-(double)z[t])) : 1.0;
        for (int c = 0; c < d; ++c) {
            size_t i = (size_t)t * d + c;
            double o = (double)bf16_to_float(oracle_double_to_bf16(g * out[i]));
            x_next[i] = oracle_double_to_bf16((double)bf16_to_float(x[i]) + o);
        }
    }
}

/* ------------------------------------------------------------------ selection */

/* "a ranks before b": larger logit first; equal logits (+0 and -0 are equal) -> lower id. */
static int ranks_before(float la, int a, float lb, int b)
{
    if (la > lb) return 1;
    if (la < lb) return 0;
    return a < b;
}

/* ids[t][j]: k distinct experts, slot 0 the best, chosen by k rounds of "best remaining". */
void oracle_select_topk(const float* logits, int64_t T, int E, int k, int32_t* ids)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const float* l = logits + (size_t)t * E;
        char* taken = (char*)calloc((size_t)E, 1);
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || ranks_before(l[e], e, l[best], best)) best = e;
            }
            taken[best] = 1;
            ids[(size_t)t * k + j] = best;
        }
        free(taken);
    }
}

/* Gate weights of the selected experts: softmax over the k selected logits, in double,
 * shifted by the largest (slot 0).  Equal in exact arithmetic to the softmax over all E
 * logits renormalised over the selected ones. */
void oracle_topk_weights(const float* logits, const int32_t* ids, int64_t T, int E, int k,
                         double* w)
{
    for (int64_t t = 0; t < T; ++t) {
        const float* l = logits + (size_t)t * E;
        double lmax = (double)l[ids[(size_t)t * k]];
        double den = 0.0;
        for (int j = 0; j < k; ++j)
            den += exp((double)l[ids[(size_t)t * k + j]] - lmax);
        for (int j = 0; j < k; ++j)
            w[(size_t)t * k + j] = exp((double)l[ids[(size_t)t * k + j]] - lmax) / den;
    }
}

/* ------------------------------------------------------------------ grouping */

/* Stable grouping of the T*k (token, slot) pairs by expert: sorted_pairs lists, expert by
 * expert in increasing id, the pairs p = t*k + j routed to it in increasing p;
 * offsets[e] .. offsets[e+1] is expert e's segment; pair_pos[p] is where p landed.
 * Returns the number of ids outside [0, E) (those pairs are left out). */
int64_t oracle_permute(const int32_t* ids, int64_t T, int k, int E, int32_t* offsets,
                       int32_t* sorted_pairs, int32_t* pair_pos)
{
    int64_t P = T * k, pos = 0, bad = 0;
    for (int64_t p = 0; p < P; ++p) {
        pair_pos[p] = -1;
        if (ids[p] < 0 || ids[p] >= E) ++bad;
    }
    for (int e = 0; e < E; ++e) {
        offsets[e] = (int32_t)pos;
        for (int64_t p = 0; p < P; ++p) {
            if (ids[p] == e) {
                sorted_pairs[pos] = (int32_t)p;
                pair_pos[p] = (int32_t)pos;
                ++pos;
            }
        }
    }
    offsets[E] = (int32_t)pos;
    return bad;
}

/* ------------------------------------------------------------------ expert FFN */

/* One token through expert e: g = Wg x, u = Wu x, h = silu(g) * u, y = Wd h (double). */
void oracle_expert_ffn(const oracle_experts* ex, int e, const uint16_t* x_row, double* y)
{
    const int d = ex->d_model, F = ex->d_ff, fmt = ex->fmt;
    const size_t gate_rows = (size_t)e * F, down_rows = (size_t)e * d;
    double* xr = (double*)malloc(sizeof(double) * d);
    double* h = (double*)malloc(sizeof(double) * F);
    double* wrow = (double*)malloc(sizeof(double) * (d > F ? d : F));
    for (int c = 0; c < d; ++c) xr[c] = (double)bf16_to_float(x_row[c]);
    for (int f = 0; f < F; ++f) {
        double g = 0.0, u = 0.0;
        oracle_dequant_row(fmt, ex->w_gate, ex->s_gate, d, (int64_t)(gate_rows + f), wrow);
        for (int c = 0; c < d; ++c) g += wrow[c] * xr[c];
        oracle_dequant_row(fmt, ex->w_up, ex->s_up, d, (int64_t)(gate_rows + f), wrow);
        for (int c = 0; c < d; ++c) u += wrow[c] * xr[c];
        h[f] = g / (1.0 + exp(-g)) * u;            /* silu(g) = g * sigmoid(g) */
    }
    for (int n = 0; n < d; ++n) {
        double acc = 0.0;
        oracle_dequant_row(fmt, ex->w_down, ex->s_down, F, (int64_t)(down_rows + n), wrow);
        for (int f = 0; f < F; ++f) acc += wrow[f] * h[f];
        y[n] = acc;
    }
    free(xr);
    free(h);
    free(wrow);
}

/* ------------------------------------------------------------------ combine */

/* out[t] = y_shared[t] + sum_j w[t][j] * y_pairs[pair_pos[t*k+j]] in double.
 * y_shared may be NULL (no shared expert). */
void oracle_combine(const double* y_pairs, const int32_t* pair_pos, const double* w,
                    const double* y_shared, int64_t T, int k, int d, double* out)
{
    for (int64_t t = 0; t < T; ++t) {
        for (int n = 0; n < d; ++n) {
            double acc = 0.0;
            for (int j = 0; j < k; ++j) {
                int64_t q = pair_pos[t * k + j];
                acc += w[t * k + j] * y_pairs[(size_t)q * d + n];
            }
            if (y_shared) acc += y_shared[(size_t)t * d + n];
            out[(size_t)t * d + n] = acc;
        }
    }
}

/* ------------------------------------------------------------------ whole layer */

/*
 * Output rows of the listed tokens: routing for those tokens (router, selection,
 * weights), every selected expert and the shared expert in double, then the combine.
 * Routing of a token does not depend on other tokens, so a subset is exact.
 *   tokens[n_tok]  token indices into x[T][d]
 *   ids_out[n_tok][k], w_out[n_tok][k], y_sel_out[n_tok][k][d] (slot order, may be NULL),
 *   y_shared_out[n_tok][d] (may be NULL), out[n_tok][d]
 * shared may be NULL (no shared expert).
 */
void oracle_layer_tokens(const oracle_router* r, const oracle_experts* routed,
                         const oracle_experts* shared, const uint16_t* x,
                         const int32_t* tokens, int64_t n_tok, int k, int32_t* ids_out,
                         double* w_out, double* y_sel_out, double* y_shared_out, double* out)
{
    const int E = r->n_experts, d = r->d_model;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < n_tok; ++i) {
        const uint16_t* xr = x + (size_t)tokens[i] * d;
        float* logits = (float*)malloc(sizeof(float) * E);
        double* y = (double*)malloc(sizeof(double) * d);
        oracle_router_logits(r, xr, 1, logits);
        oracle_select_topk(logits, 1, E, k, ids_out + i * k);
        oracle_topk_weights(logits, ids_out + i * k, 1, E, k, w_out + i * k);
        double* o = out + (size_t)i * d;
        for (int n = 0; n < d; ++n) o[n] = 0.0;
        for (int j = 0; j < k; ++j) {
            oracle_expert_ffn(routed, ids_out[i * k + j], xr, y);
            if (y_sel_out) memcpy(y_sel_out + ((size_t)i * k + j) * d, y, sizeof(double) * d);
            for (int n = 0; n < d; ++n) o[n] += w_out[i * k + j] * y[n];
        }
        if (shared) {
            oracle_expert_ffn(shared, 0, xr, y);
            if (y_shared_out) memcpy(y_shared_out + (size_t)i * d, y, sizeof(double) * d);
            for (int n = 0; n < d; ++n) o[n] += y[n];
        }
        free(logits);
        free(y);
    }
}

/* Same as oracle_expert_ffn for a list of (token, expert) pairs, in parallel. */
void oracle_expert_ffn_pairs(const oracle_experts* ex, const uint16_t* x, const int32_t* tok,
                             const int32_t* expert, int64_t n, double* y)
{
    const int d = ex->d_model;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < n; ++i)
        oracle_expert_ffn(ex, expert[i], x + (size_t)tok[i] * d, y + (size_t)i * d);
}

/* Stacked-layer residual: x_next = bf16(x + bf16(out)); the sum of two bf16 numbers is
 * exact in double, so one rounding to bf16 remains. */
void oracle_residual(const uint16_t* x, const double* out, int64_t n, uint16_t* x_next)
{
    for (int64_t i = 0; i < n; ++i) {
        double o = (double)bf16_to_float(oracle_double_to_bf16(out[i]));
        double s = (double)bf16_to_float(x[i]) + o;   /* exact: two bf16 values */
        x_next[i] = oracle_double_to_bf16(s);
    }
}

/* Threads the OpenMP loops above use from now on (n >= 1). */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
