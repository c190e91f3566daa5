/*
 * CPU oracle of the routed top-k mixture-of-experts layer.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this library. The GPU library shares
 * no code, header, table or constant with it.
 *
 * What the layer computes (the first page, the FlyDSL-in-JAX talk summary,
 * sections 5:56 "Optimierung gerouteter MoE-GEMMs" and 8:14 "End-to-End-Integration
 * in MaxText"): every token is routed to its top-2 experts; each selected expert
 * applies a SwiGLU feed-forward block (gate and up projections, SwiGLU, down
 * projection; glossary entry "SwiGLU"); the k expert outputs are scattered back
 * to the token and combined with the routing weights. The pages name the pieces
 * (gather, group GEMM, SwiGLU, scatter, top-2, load-time preshuffle) but write
 * out no formula; the definitions below are the plainest reading, with the
 * shapes x[T,H], W_r[E,H], W1/W3[E,I,H], W2[E,H,I] of the Mixtral 8x7B layer.
 *
 * Arithmetic: fp64 everywhere, except where a floating-point result decides an
 * integer that must match the GPU bit for bit. Those decisions are taken in the
 * GPU's precision, fp32:
 *   - router logits (they decide the top-k ids), summed in one fixed order;
 *   - per-token activation quantisation to e4m3fn (fp32 divide, then RNE).
 * Storage roundings that the method itself prescribes are applied: the bf16
 * SwiGLU intermediate on the bf16 path, the per-row e4m3fn requantisation of the
 * intermediate on the fp8 path, and the bf16 output.
 *
 * MXFP8 path (the second page, the PyTorch FlyDSL backend news item, section
 * "Grenzen und Folgen für Anwender": E4M3 operands with one E8M0 scale per 32
 * values along the reduction, K a multiple of 128). The pages fix only the format; how a block's
 * scale is chosen is the OCP Microscaling specification's conversion, the
 * plainest reading: scale = 2^(floor(log2 max|v|) - 8), 8 being the exponent of
 * E4M3's largest normal, elements rounded to nearest even and saturated at 448.
 * Weights arrive quantised (that page measures from quantised operands); the
 * token rows are block-quantised on the path, and the SwiGLU intermediate is
 * stored in bf16 and block-quantised again for the down projection.
 *
 * MXFP4 path (same page and section: "packed FP4-E2M1 operands" with the same
 * E8M0 scale per 32 values): the expert weights are E2M1 codes, two per byte
 * (value 2i in the low nibble of byte i), with E8M0 block scales; tokens and
 * the intermediate are MXFP8 exactly as above.
 *
 * Each function is plain loops; OpenMP only splits independent output rows.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_BF16 = 0, ORACLE_FP8 = 1, ORACLE_MXFP8 = 2, ORACLE_MXFP4 = 3 };

enum { MX_BLOCK = 32 }; /* values per E8M0 scale along the reduction */

/* ------------------------------------------------------------------------ */
/* Number formats                                                            */

/* bf16 is the upper half of an IEEE binary32. */
double oracle_bf16_to_f64(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Round a binary32 to bf16, to nearest with ties to even; NaN stays NaN. */
uint16_t oracle_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7fffu + lsb;
    return (uint16_t)(u >> 16);
}

/* OCP 8-bit float E4M3 ("fn": finite, no infinities): 1 sign bit, 4 exponent
 * bits with bias 7, 3 mantissa bits. Exponent field 0 is subnormal
 * (m * 2^-9); S.1111.111 is NaN; the largest finite magnitude is 448. */
double oracle_e4m3fn_to_f64(uint8_t q)
{
    int s = q >> 7, e = (q >> 3) & 15, m = q & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + m / 8.0, e - 7);
    return s ? -v : v;
}

/* Nearest e4m3fn code to v, ties to the even code; |v| beyond 448 saturates
 * to +-448. Positive codes 0x00..0x7E increase with their value, so the two
 * neighbours of |v| are found by a search over that ordered table. */
uint8_t oracle_f32_to_e4m3fn(float v)
{
    if (isnan(v))
        return 0x7f;
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs((double)v);
    if (a >= 448.0)
        return sign | 0x7e;
    int lo = 0, hi = 0x7e; /* value(lo) <= a < value(hi) */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (oracle_e4m3fn_to_f64((uint8_t)mid) <= a)
            lo = mid;
        else
            hi = mid;
    }
    double dl = a - oracle_e4m3fn_to_f64((uint8_t)lo);
    double dh = oracle_e4m3fn_to_f64((uint8_t)hi) - a;
    int c;
    if (dl < dh)
        c = lo;
    else if (dh < dl)
        c = hi;
    else
        c = (lo & 1) ? hi : lo;
    return sign | (uint8_t)c;
}

/* OCP E8M0 shared scale: eight exponent bits, no sign, no mantissa; code b
 * is 2^(b - 127) and 0xFF is NaN. */
double oracle_e8m0_to_f64(uint8_t b)
{
    if (b == 0xFF)
        return NAN;
    return ldexp(1.0, (int)b - 127);
}

/* One MX block of n values: returns the E8M0 code of the shared scale and
 * writes the n e4m3fn codes. The shared exponent is floor(log2 amax) - 8,
 * clamped to E8M0's [-127, 127]; an all-zero block gets exponent 0 (scale 1).
 * Elements: e4m3fn(clamp(v / 2^x, -448, 448)); dividing by a power of two is
 * exact, so the only rounding is the encoder's. */
static uint8_t mx_block(const float* v, int n, uint8_t* q)
{
    double amax = 0.0;
    for (int i = 0; i < n; ++i)
        if (fabs((double)v[i]) > amax)
            amax = fabs((double)v[i]);
    int x = 0;
    if (amax > 0.0) {
        int ex;
        frexp(amax, &ex); /* amax = m * 2^ex, 0.5 <= m < 1: floor(log2 amax) = ex - 1 */
        x = ex - 1 - 8;
        if (x < -127)
            x = -127;
        if (x > 127)
            x = 127;
    }
    for (int i = 0; i < n; ++i) {
        double r = ldexp((double)v[i], -x);
        if (r > 448.0)
            r = 448.0;
        if (r < -448.0)
            r = -448.0;
        q[i] = oracle_f32_to_e4m3fn((float)r);
    }
    return (uint8_t)(x + 127);
}

/* OCP 4-bit float E2M1: 1 sign bit, 2 exponent bits with bias 1, 1 mantissa
 * bit; exponent field 0 is subnormal (m * 0.5). Magnitudes 0, 0.5, 1, 1.5, 2,
 * 3, 4, 6; no infinity or NaN. Only the low 4 bits of q are read. */
double oracle_e2m1_to_f64(uint8_t q)
{
    int s = (q >> 3) & 1, e = (q >> 1) & 3, m = q & 1;
    double v = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -v : v;
}

/* Nearest E2M1 code to v, ties to the even code; |v| beyond 6 saturates. */
uint8_t oracle_f32_to_e2m1(float v)
{
    uint8_t sign = signbit(v) ? 0x8 : 0x0;
    double a = fabs((double)v);
    if (isnan(v) || a >= 6.0)
        return sign | 0x7;
    int best = 0;
    double bd = a;
    for (int c = 1; c < 8; ++c) {
        double d = fabs(a - oracle_e2m1_to_f64((uint8_t)c));
        if (d < bd || (d == bd && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            bd = d;
        }
    }
    return sign | (uint8_t)best;
}

static double wval(int dtype, const void* w, size_t idx)
{
    if (dtype == ORACLE_BF16)
        return oracle_bf16_to_f64(((const uint16_t*)w)[idx]);
    if (dtype == ORACLE_MXFP4)
        return oracle_e2m1_to_f64((uint8_t)(((const uint8_t*)w)[idx / 2] >> (4 * (idx % 2))));
    return oracle_e4m3fn_to_f64(((const uint8_t*)w)[idx]);
}

/* Dequantisation factor of weight element (row, col) of a matrix with K
 * columns: per output row (fp32 scale) on the fp8 path, per row and 32-column
 * block (E8M0 code) on the MXFP8 path, 1 for bf16. */
static double wscale(int dtype, const void* s, size_t row, int col, int K)
{
    if (dtype == ORACLE_FP8)
        return (double)((const float*)s)[row];
    if (dtype == ORACLE_MXFP8 || dtype == ORACLE_MXFP4)
        return oracle_e8m0_to_f64(((const uint8_t*)s)[row * (size_t)(K / MX_BLOCK) + col / MX_BLOCK]);
    return 1.0;
}

/* ------------------------------------------------------------------------ */
/* Router: logits, top-k, renormalised weights                               */

/* Router logit of token row x against expert row w, in fp32, in the fixed
 * summation order that is part of this layer's contract:
 *   - the H products are split over 64 partial sums ("lanes"): element h goes
 *     to lane (h / 8) mod 64, i.e. lanes own 8-element chunks round robin;
 *   - each lane adds its products in ascending h, acc = acc + x*w;
 *   - the 64 partials are then folded pairwise: for off = 32,16,8,4,2,1,
 *     p[l] = p[l] + p[l+off] for l < off; the logit is p[0].
 * A bf16*bf16 product has at most 16 significant bits, so it is exact in
 * fp32 and a fused multiply-add gives the same sums. */
float oracle_logit(const uint16_t* x, const uint16_t* w, int H)
{
    float p[64];
    for (int l = 0; l < 64; ++l)
        p[l] = 0.0f;
    for (int h = 0; h < H; ++h) {
        int lane = (h / 8) % 64;
        float prod = (float)oracle_bf16_to_f64(x[h]) * (float)oracle_bf16_to_f64(w[h]);
        p[lane] = p[lane] + prod;
    }
    for (int off = 32; off >= 1; off /= 2)
        for (int l = 0; l < off; ++l)
            p[l] = p[l] + p[l + off];
    return p[0];
}

/* Top-k of one token's E logits: rank j is the largest logit not yet taken,
 * ties going to the lower expert index (IEEE comparison: -0 == +0). The
 * routing weights are the softmax over the k selected logits, which equals the
 * full softmax renormalised over the selected experts. */
static void topk_one(const float* l, int E, int k, int32_t* ids, float* w)
{
    int taken[64] = {0};
    for (int j = 0; j < k; ++j) {
        int best = -1;
        for (int e = 0; e < E; ++e) {
            if (taken[e])
                continue;
            if (best < 0 || l[e] > l[best])
                best = e;
        }
        taken[best] = 1;
        ids[j] = best;
    }
    double den = 0.0, num[64];
    for (int j = 0; j < k; ++j) {
        num[j] = exp((double)l[ids[j]] - (double)l[ids[0]]);
        den += num[j];
    }
    for (int j = 0; j < k; ++j)
        w[j] = (float)(num[j] / den);
}

/* ids[T,k], w[T,k]; logits[T,E] when non-NULL. bias[E] (fp32, may be NULL) is
 * added to each logit as one fp32 addition before selection. */
void oracle_route(const uint16_t* x, const uint16_t* w_router, const float* bias,
                  int T, int H, int E, int k, int32_t* ids, float* w, float* logits)
{
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        float l[64];
        for (int e = 0; e < E; ++e) {
            l[e] = oracle_logit(x + (size_t)t * H, w_router + (size_t)e * H, H);
            if (bias)
                l[e] = l[e] + bias[e];
            if (logits)
                logits[(size_t)t * E + e] = l[e];
        }
        topk_one(l, E, k, ids + (size_t)t * k, w + (size_t)t * k);
    }
}

/* Top-k and weights from given logits (used to tell apart summation-order
 * differences from selection differences). */
void oracle_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w)
{
    for (int t = 0; t < T; ++t)
        topk_one(logits + (size_t)t * E, E, k, ids + (size_t)t * k, w + (size_t)t * k);
}

/* ------------------------------------------------------------------------ */
/* Dynamic per-token activation quantisation (fp8 path)                      */

/* scale s_t = amax_t / 448 in fp32 (1 when the row is all zero);
 * code = e4m3fn(clamp(x / s_t, -448, 448)), the divide in fp32. */
void oracle_quant_tokens(const uint16_t* x, int T, int H, uint8_t* xq, float* xs)
{
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        const uint16_t* r = x + (size_t)t * H;
        float amax = 0.0f;
        for (int h = 0; h < H; ++h) {
            float a = fabsf((float)oracle_bf16_to_f64(r[h]));
            if (a > amax)
                amax = a;
        }
        float s = amax > 0.0f ? amax / 448.0f : 1.0f;
        xs[t] = s;
        for (int h = 0; h < H; ++h) {
            float v = (float)oracle_bf16_to_f64(r[h]) / s;
            if (v > 448.0f)
                v = 448.0f;
            if (v < -448.0f)
                v = -448.0f;
            xq[(size_t)t * H + h] = oracle_f32_to_e4m3fn(v);
        }
    }
}

/* MX block quantisation of token rows (MXFP8 path): for each token and each
 * block of 32 consecutive hidden values, one E8M0 scale code xs[t, h/32] and
 * the e4m3fn codes xq[t, h] (mx_block). H must be a multiple of 32. */
void oracle_quant_tokens_mx(const uint16_t* x, int T, int H, uint8_t* xq, uint8_t* xs)
{
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        float v[MX_BLOCK];
        for (int b = 0; b < H / MX_BLOCK; ++b) {
            for (int i = 0; i < MX_BLOCK; ++i)
                v[i] = (float)oracle_bf16_to_f64(x[(size_t)t * H + b * MX_BLOCK + i]);
            xs[(size_t)t * (H / MX_BLOCK) + b] =
                mx_block(v, MX_BLOCK, xq + (size_t)t * H + b * MX_BLOCK);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Grouping token-slots by expert, padded to the M-tile                      */

/* Slot s = t*k + j is the j-th expert choice of token t. For e = 0..E-1 the
 * group of expert e lists, in ascending s, every slot routed to e, and is then
 * padded with the sentinel T*k up to a multiple of bm. tile_expert holds the
 * expert of each bm-row tile. Returns 0, or -1 when an id is out of range. */
int oracle_align(const int32_t* ids, int T, int k, int E, int bm, int32_t* sorted_slot,
                 int32_t* tile_expert, int32_t* count, int32_t* offset, int32_t* total)
{
    int S = T * k, pos = 0;
    for (int s = 0; s < S; ++s)
        if (ids[s] < 0 || ids[s] >= E)
            return -1;
    for (int e = 0; e < E; ++e) {
        offset[e] = pos;
        int c = 0;
        for (int s = 0; s < S; ++s)
            if (ids[s] == e)
                sorted_slot[pos + c++] = s;
        count[e] = c;
        int padded = (c + bm - 1) / bm * bm;
        for (int p = c; p < padded; ++p)
            sorted_slot[pos + p] = S;
        for (int tl = 0; tl < padded / bm; ++tl)
            tile_expert[pos / bm + tl] = e;
        pos += padded;
    }
    offset[E] = pos;
    *total = pos;
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Expert feed-forward (SwiGLU) and the weighted combine                     */

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* Input row x_hat of token t in fp64: the bf16 value; on the fp8 path the
 * dequantised code of the per-token quantisation; on the MXFP8 path the
 * dequantised code of the per-block quantisation (code * 2^(scale - 127)). */
static void token_row(int dtype, const uint16_t* x, int t, int H, double* xh)
{
    const uint16_t* r = x + (size_t)t * H;
    if (dtype == ORACLE_BF16) {
        for (int h = 0; h < H; ++h)
            xh[h] = oracle_bf16_to_f64(r[h]);
        return;
    }
    uint8_t* q = (uint8_t*)malloc((size_t)H);
    if (dtype == ORACLE_MXFP8 || dtype == ORACLE_MXFP4) {
        uint8_t* sb = (uint8_t*)malloc((size_t)H / MX_BLOCK);
        oracle_quant_tokens_mx(r, 1, H, q, sb);
        for (int h = 0; h < H; ++h)
            xh[h] = oracle_e4m3fn_to_f64(q[h]) * oracle_e8m0_to_f64(sb[h / MX_BLOCK]);
        free(sb);
        free(q);
        return;
    }
    float s;
    oracle_quant_tokens(r, 1, H, q, &s);
    for (int h = 0; h < H; ++h)
        xh[h] = oracle_e4m3fn_to_f64(q[h]) * (double)s;
    free(q);
}

/* SwiGLU intermediate of one (token, expert) pair, before storage rounding:
 * a_i = silu(g_i) * u_i, g = W1[e] x_hat, u = W3[e] x_hat, with dequantised
 * weights: code * s[e,i] on the fp8 path, code * 2^(s[e,i,h/32] - 127) on the
 * MXFP8 path (wscale). */
static void swiglu_row(int dtype, const double* xh, const void* w1, const void* w3,
                       const void* s1, const void* s3, int e, int H, int I, double* a)
{
#pragma omp parallel for schedule(static)
    for (int i = 0; i < I; ++i) {
        size_t r = (size_t)e * I + i, row = r * (size_t)H;
        double g = 0.0, u = 0.0;
        for (int h = 0; h < H; ++h) {
            g += xh[h] * (wval(dtype, w1, row + h) * wscale(dtype, s1, r, h, H));
            u += xh[h] * (wval(dtype, w3, row + h) * wscale(dtype, s3, r, h, H));
        }
        a[i] = silu(g) * u;
    }
}

/* The intermediate as stage two reads it: bf16 storage on the bf16 path
 * (fp32, then bf16, both round-to-nearest-even); on the fp8 path a per-row
 * requantisation, scale = max|a| / 448 (1 if zero), code = e4m3fn(a / scale),
 * value = code * scale; on the MXFP8 path bf16 storage, then the MX block
 * quantisation of each 32 consecutive values (mx_block), value = code * 2^x. */
static void store_intermediate(int dtype, double* a, int I)
{
    if (dtype == ORACLE_BF16) {
        for (int i = 0; i < I; ++i)
            a[i] = oracle_bf16_to_f64(oracle_f32_to_bf16((float)a[i]));
        return;
    }
    if (dtype == ORACLE_MXFP8 || dtype == ORACLE_MXFP4) {
        float v[MX_BLOCK];
        uint8_t q[MX_BLOCK];
        for (int b = 0; b < I / MX_BLOCK; ++b) {
            for (int i = 0; i < MX_BLOCK; ++i)
                v[i] = (float)oracle_bf16_to_f64(oracle_f32_to_bf16((float)a[b * MX_BLOCK + i]));
            double sc = oracle_e8m0_to_f64(mx_block(v, MX_BLOCK, q));
            for (int i = 0; i < MX_BLOCK; ++i)
                a[b * MX_BLOCK + i] = oracle_e4m3fn_to_f64(q[i]) * sc;
        }
        return;
    }
    double amax = 0.0;
    for (int i = 0; i < I; ++i)
        if (fabs(a[i]) > amax)
            amax = fabs(a[i]);
    double s = amax > 0.0 ? amax / 448.0 : 1.0;
    for (int i = 0; i < I; ++i) {
        double v = a[i] / s;
        if (v > 448.0)
            v = 448.0;
        if (v < -448.0)
            v = -448.0;
        a[i] = oracle_e4m3fn_to_f64(oracle_f32_to_e4m3fn((float)v)) * s;
    }
}

/* Down projection y_h = sum_i a_i * W2[e,h,i] (weights dequantised as in
 * swiglu_row, the reduction running over i). */
static void down_row(int dtype, const double* a, const void* w2, const void* s2, int e,
                     int H, int I, double* y)
{
#pragma omp parallel for schedule(static)
    for (int h = 0; h < H; ++h) {
        size_t r = (size_t)e * H + h, row = r * (size_t)I;
        double acc = 0.0;
        for (int i = 0; i < I; ++i)
            acc += a[i] * (wval(dtype, w2, row + i) * wscale(dtype, s2, r, i, I));
        y[h] = acc;
    }
}

/* SwiGLU intermediate rows for given (token, expert) pairs, before storage
 * rounding (stage-one parity). act[n, I] in fp64. */
void oracle_swiglu(int dtype, const uint16_t* x, const void* w1, const void* w3,
                   const void* s1, const void* s3, int T, int H, int I,
                   const int32_t* tokens, const int32_t* experts, int n, double* act)
{
    double* xh = (double*)malloc(sizeof(double) * (size_t)H);
    for (int r = 0; r < n; ++r) {
        (void)T;
        token_row(dtype, x, tokens[r], H, xh);
        swiglu_row(dtype, xh, w1, w3, s1, s3, experts[r], H, I, act + (size_t)r * I);
    }
    free(xh);
}

/* Down projection of given intermediate rows (already in the value they are
 * stored at) through given experts: y[n, H] in fp64 (stage-two parity). */
void oracle_down(int dtype, const double* act, const void* w2, const void* s2,
                 int H, int I, const int32_t* experts, int n, double* y)
{
    for (int r = 0; r < n; ++r)
        down_row(dtype, act + (size_t)r * I, w2, s2, experts[r], H, I, y + (size_t)r * H);
}

/* The whole layer for the listed tokens: route, (quantise), for j in 0..k-1
 * the selected expert's SwiGLU block, then out = bf16(sum_j w_j * y_j) with the
 * sum taken in ascending j. out_bf16[n,H]; out_f64[n,H] (the value before the
 * final rounding) when non-NULL. */
void oracle_forward(int dtype, const uint16_t* x, const uint16_t* w_router, const float* bias,
                    const void* w1, const void* w3, const void* w2, const void* s1,
                    const void* s3, const void* s2, int T, int H, int I, int E, int k,
                    const int32_t* tokens, int n, uint16_t* out_bf16, double* out_f64)
{
    double* xh = (double*)malloc(sizeof(double) * (size_t)H);
    double* a = (double*)malloc(sizeof(double) * (size_t)I);
    double* y = (double*)malloc(sizeof(double) * (size_t)H);
    double* o = (double*)malloc(sizeof(double) * (size_t)H);
    int32_t ids[64];
    float w[64];
    for (int r = 0; r < n; ++r) {
        int t = tokens[r];
        (void)T;
        oracle_route(x + (size_t)t * H, w_router, bias, 1, H, E, k, ids, w, NULL);
        token_row(dtype, x, t, H, xh);
        for (int h = 0; h < H; ++h)
            o[h] = 0.0;
        for (int j = 0; j < k; ++j) {
            swiglu_row(dtype, xh, w1, w3, s1, s3, ids[j], H, I, a);
            store_intermediate(dtype, a, I);
            down_row(dtype, a, w2, s2, ids[j], H, I, y);
            for (int h = 0; h < H; ++h)
                o[h] = o[h] + (double)w[j] * y[h];
        }
        for (int h = 0; h < H; ++h) {
            if (out_f64)
                out_f64[(size_t)r * H + h] = o[h];
            out_bf16[(size_t)r * H + h] = oracle_f32_to_bf16((float)o[h]);
        }
    }
    free(xh);
    free(a);
    free(y);
    free(o);
}

/* Apply the intermediate storage rounding to n rows of I values in place. */
void oracle_store_intermediate(int dtype, double* act, int n, int I)
{
    for (int r = 0; r < n; ++r)
        store_intermediate(dtype, act + (size_t)r * I, I);
}

/* ------------------------------------------------------------------------ */
/* One-time weight preshuffle into MFMA operand order                        */

/* The layout the GPU library stores expert weights in (load time only, not
 * arithmetic). A weight matrix with R rows (output features) and a reduction
 * of K_bytes bytes per row is cut into fragments of 32 rows x 64 bytes (64
 * e4m3fn or 32 bf16 values), stored row-block major, then reduction block.
 * A fragment is two 1 KB pieces; in piece pc, the 16 bytes of lane l = 0..63
 * (at l*16) are row l mod 32, bytes (l / 32)*32 + pc*16 .. +15 of the 64.
 * For the gate/up pair, the rows of one expert are taken in blocks of 32
 * alternating W1, W3: composite row c is W1 row (c/64)*32 + c%32 when (c/32)
 * is even, W3 row of the same index when it is odd. */
static void shuffle_matrix(const uint8_t* const* rows, int R, size_t K_bytes, uint8_t* out)
{
    size_t kblocks = K_bytes / 64;
    for (int rb = 0; rb < R / 32; ++rb)
        for (size_t kb = 0; kb < kblocks; ++kb)
            for (int pc = 0; pc < 2; ++pc)
                for (int l = 0; l < 64; ++l) {
                    const uint8_t* src = rows[rb * 32 + l % 32] + kb * 64 + (size_t)(l / 32) * 32 +
                                         (size_t)pc * 16;
                    uint8_t* dst = out + (((size_t)rb * kblocks + kb) * 2 + pc) * 1024 + l * 16;
                    memcpy(dst, src, 16);
                }
}

void oracle_preshuffle_w13(int dtype, int E, int H, int I, const void* w1, const void* w3,
                           void* out)
{
    size_t es = dtype == ORACLE_BF16 ? 2 : 1;
    size_t rowbytes = (size_t)H * es, per = (size_t)I * rowbytes;
    const uint8_t** rows = (const uint8_t**)malloc(sizeof(uint8_t*) * 2 * (size_t)I);
    for (int e = 0; e < E; ++e) {
        for (int c = 0; c < 2 * I; ++c) {
            const uint8_t* base = (const uint8_t*)(((c / 32) % 2 == 0) ? w1 : w3) + e * per;
            rows[c] = base + (size_t)((c / 64) * 32 + c % 32) * rowbytes;
        }
        shuffle_matrix(rows, 2 * I, rowbytes, (uint8_t*)out + 2 * e * per);
    }
    free(rows);
}

void oracle_preshuffle_w2(int dtype, int E, int H, int I, const void* w2, void* out)
{
    size_t es = dtype == ORACLE_BF16 ? 2 : 1;
    size_t rowbytes = (size_t)I * es, per = (size_t)H * rowbytes;
    const uint8_t** rows = (const uint8_t**)malloc(sizeof(uint8_t*) * (size_t)H);
    for (int e = 0; e < E; ++e) {
        for (int h = 0; h < H; ++h)
            rows[h] = (const uint8_t*)w2 + e * per + (size_t)h * rowbytes;
        shuffle_matrix(rows, H, rowbytes, (uint8_t*)out + e * per);
    }
    free(rows);
}

int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Array forms of the format conversions (same definitions, element by element). */
void oracle_e2m1_to_f64_n(const uint8_t* q, long n, double* v)
{
    for (long i = 0; i < n; ++i)
        v[i] = oracle_e2m1_to_f64(q[i]);
}

void oracle_f32_to_e2m1_n(const float* v, long n, uint8_t* q)
{
    for (long i = 0; i < n; ++i)
        q[i] = oracle_f32_to_e2m1(v[i]);
}

void oracle_e8m0_to_f64_n(const uint8_t* b, long n, double* v)
{
    for (long i = 0; i < n; ++i)
        v[i] = oracle_e8m0_to_f64(b[i]);
}

void oracle_f32_to_e4m3fn_n(const float* v, long n, uint8_t* q)
{
    for (long i = 0; i < n; ++i)
        q[i] = oracle_f32_to_e4m3fn(v[i]);
}

void oracle_e4m3fn_to_f64_n(const uint8_t* q, long n, double* v)
{
    for (long i = 0; i < n; ++i)
        v[i] = oracle_e4m3fn_to_f64(q[i]);
}

void oracle_f32_to_bf16_n(const float* v, long n, uint16_t* b)
{
    for (long i = 0; i < n; ++i)
        b[i] = oracle_f32_to_bf16(v[i]);
}

void oracle_bf16_to_f64_n(const uint16_t* b, long n, double* v)
{
    for (long i = 0; i < n; ++i)
        v[i] = oracle_bf16_to_f64(b[i]);
}

/* ------------------------------------------------------------------------ */
/* Backward pass of the bf16 layer (the custom VJP the FlyDSL-in-JAX talk     */
/* summary lists as its next step, "Ausblick und Roadmap" 10:07; "broader    */
/* backward coverage" in the glance summary's "What's Next?")                 */
/*                                                                            */
/* The pages give no formula. The plainest reading, adopted here: the exact   */
/* gradient of the layer function                                             */
/*   out_t = sum_j w_tj * W2[e_j] (silu(W1[e_j] x_t) * W3[e_j] x_t),          */
/*   w_t = softmax over the k selected logits l_tj = W_r[e_j] . x_t (+ b),    */
/* with the selection e_tj held fixed (top-k is piecewise constant), taken in */
/* fp64 on the bf16 input values, for a given output gradient dout. Storage   */
/* roundings of the forward (the bf16 intermediate and output) are not part of*/
/* the function being differentiated.                                         */

/* fp64 forward of that function for given (perturbable) fp64 parameters and a
 * fixed selection ids[T,k]: out[T,H]. Used to pin the gradients by finite
 * differences. */
void oracle_forward_f64(const double* x, const double* wr, const double* bias,
                        const double* w1, const double* w3, const double* w2,
                        const int32_t* ids, int T, int H, int I, int E, int k, double* out)
{
    (void)E;
    for (int t = 0; t < T; ++t) {
        const double* xt = x + (size_t)t * H;
        double l[64], w[64], m = -INFINITY, den = 0.0;
        for (int j = 0; j < k; ++j) {
            int e = ids[(size_t)t * k + j];
            double s = bias ? bias[e] : 0.0;
            for (int h = 0; h < H; ++h)
                s += wr[(size_t)e * H + h] * xt[h];
            l[j] = s;
            if (s > m)
                m = s;
        }
        for (int j = 0; j < k; ++j) {
            w[j] = exp(l[j] - m);
            den += w[j];
        }
        double* o = out + (size_t)t * H;
        for (int h = 0; h < H; ++h)
            o[h] = 0.0;
        double* a = (double*)malloc(sizeof(double) * (size_t)I);
        for (int j = 0; j < k; ++j) {
            int e = ids[(size_t)t * k + j];
            double wj = w[j] / den;
#pragma omp parallel for schedule(static)
            for (int i = 0; i < I; ++i) {
                size_t r = ((size_t)e * I + i) * H;
                double g = 0.0, u = 0.0;
                for (int c = 0; c < H; ++c) {
                    g += w1[r + c] * xt[c];
                    u += w3[r + c] * xt[c];
                }
                a[i] = silu(g) * u;
            }
#pragma omp parallel for schedule(static)
            for (int h = 0; h < H; ++h) {
                double y = 0.0;
                for (int i = 0; i < I; ++i)
                    y += w2[((size_t)e * H + h) * I + i] * a[i];
                o[h] += wj * y;
            }
        }
        free(a);
    }
}

/* Gradients of sum_t <dout_t, out_t> with respect to x, W1, W3, W2, W_r and the
 * bias, for the bf16 layer (inputs as bf16 bit patterns, dout bf16 [T,H]).
 * The selection is the forward's (fixed-order fp32 logits, oracle_route); the
 * routing weights and everything else are fp64. Per token and selected expert
 * e (rank j):
 *   g = W1 x, u = W3 x, a = silu(g) u, y = W2 a        (the forward values)
 *   dw_j = <dout, y>                                   (gradient of w_j)
 *   z = W2^T dout, da = w_j z                          (gradient of a)
 *   dg = da u silu'(g), du = da silu(g),  silu'(g) = s (1 + g (1 - s)), s = sigmoid(g)
 *   dW2[e] += (w_j dout) a^T,  dW1[e] += dg x^T,  dW3[e] += du x^T
 *   dx += W1^T dg + W3^T du
 * then the softmax over the selected logits: dl_j = w_j (dw_j - sum_i w_i dw_i),
 *   dW_r[e_j] += dl_j x,  db[e_j] += dl_j,  dx += sum_j dl_j W_r[e_j].
 * Outputs are fp64 and overwritten: dx [T,H], dw1 and dw3 [E,I,H], dw2 [E,H,I],
 * dwr [E,H], dbias [E] (may be NULL). Tokens are taken one after another (the
 * weight gradients accumulate in token order); OpenMP splits rows inside. */
void oracle_backward(const uint16_t* x, const uint16_t* w_router, const float* bias,
                     const uint16_t* w1, const uint16_t* w3, const uint16_t* w2, int T, int H,
                     int I, int E, int k, const uint16_t* dout, double* dx, double* dw1,
                     double* dw3, double* dw2, double* dwr, double* dbias)
{
    memset(dx, 0, sizeof(double) * (size_t)T * H);
    memset(dw1, 0, sizeof(double) * (size_t)E * I * H);
    memset(dw3, 0, sizeof(double) * (size_t)E * I * H);
    memset(dw2, 0, sizeof(double) * (size_t)E * H * I);
    memset(dwr, 0, sizeof(double) * (size_t)E * H);
    if (dbias)
        memset(dbias, 0, sizeof(double) * (size_t)E);
    double* xt = (double*)malloc(sizeof(double) * (size_t)H);
    double* dy = (double*)malloc(sizeof(double) * (size_t)H);
    double* g = (double*)malloc(sizeof(double) * (size_t)I);
    double* u = (double*)malloc(sizeof(double) * (size_t)I);
    double* a = (double*)malloc(sizeof(double) * (size_t)I);
    double* z = (double*)malloc(sizeof(double) * (size_t)I);
    double* dg = (double*)malloc(sizeof(double) * (size_t)I);
    double* du = (double*)malloc(sizeof(double) * (size_t)I);
    for (int t = 0; t < T; ++t) {
        int32_t ids[64];
        float wf[64];
        oracle_route(x + (size_t)t * H, w_router, bias, 1, H, E, k, ids, wf, NULL);
        for (int h = 0; h < H; ++h) {
            xt[h] = oracle_bf16_to_f64(x[(size_t)t * H + h]);
            dy[h] = oracle_bf16_to_f64(dout[(size_t)t * H + h]);
        }
        /* routing weights in fp64 from fp64 logits */
        double l[64], w[64], m = -INFINITY, den = 0.0, dwj[64];
        for (int j = 0; j < k; ++j) {
            double s = bias ? (double)bias[ids[j]] : 0.0;
            for (int h = 0; h < H; ++h)
                s += oracle_bf16_to_f64(w_router[(size_t)ids[j] * H + h]) * xt[h];
            l[j] = s;
            if (s > m)
                m = s;
        }
        for (int j = 0; j < k; ++j) {
            w[j] = exp(l[j] - m);
            den += w[j];
        }
        for (int j = 0; j < k; ++j)
            w[j] /= den;
        for (int j = 0; j < k; ++j) {
            const int e = ids[j];
#pragma omp parallel for schedule(static)
            for (int i = 0; i < I; ++i) {
                size_t r = ((size_t)e * I + i) * H;
                double gg = 0.0, uu = 0.0;
                for (int h = 0; h < H; ++h) {
                    gg += oracle_bf16_to_f64(w1[r + h]) * xt[h];
                    uu += oracle_bf16_to_f64(w3[r + h]) * xt[h];
                }
                g[i] = gg;
                u[i] = uu;
                a[i] = silu(gg) * uu;
            }
            /* z = W2^T dout and dw_j = <dout, W2 a> = <z, a> */
#pragma omp parallel for schedule(static)
            for (int i = 0; i < I; ++i) {
                double s = 0.0;
                for (int h = 0; h < H; ++h)
                    s += oracle_bf16_to_f64(w2[((size_t)e * H + h) * I + i]) * dy[h];
                z[i] = s;
            }
            double d = 0.0;
            for (int i = 0; i < I; ++i)
                d += z[i] * a[i];
            dwj[j] = d;
            for (int i = 0; i < I; ++i) {
                double sg = 1.0 / (1.0 + exp(-g[i]));
                double da = w[j] * z[i];
                dg[i] = da * u[i] * sg * (1.0 + g[i] * (1.0 - sg));
                du[i] = da * g[i] * sg;
            }
#pragma omp parallel for schedule(static)
            for (int h = 0; h < H; ++h) {
                double* row = dw2 + ((size_t)e * H + h) * I;
                for (int i = 0; i < I; ++i)
                    row[i] += w[j] * dy[h] * a[i];
            }
#pragma omp parallel for schedule(static)
            for (int i = 0; i < I; ++i) {
                double* r1 = dw1 + ((size_t)e * I + i) * H;
                double* r3 = dw3 + ((size_t)e * I + i) * H;
                for (int h = 0; h < H; ++h) {
                    r1[h] += dg[i] * xt[h];
                    r3[h] += du[i] * xt[h];
                }
            }
#pragma omp parallel for schedule(static)
            for (int h = 0; h < H; ++h) {
                double s = 0.0;
                for (int i = 0; i < I; ++i) {
                    size_t r = ((size_t)e * I + i) * H + h;
                    s += oracle_bf16_to_f64(w1[r]) * dg[i] + oracle_bf16_to_f64(w3[r]) * du[i];
                }
                dx[(size_t)t * H + h] += s;
            }
        }
        double sw = 0.0;
        for (int j = 0; j < k; ++j)
            sw += w[j] * dwj[j];
        for (int j = 0; j < k; ++j) {
            const int e = ids[j];
            const double dl = w[j] * (dwj[j] - sw);
            for (int h = 0; h < H; ++h) {
                dwr[(size_t)e * H + h] += dl * xt[h];
                dx[(size_t)t * H + h] += dl * oracle_bf16_to_f64(w_router[(size_t)e * H + h]);
            }
            if (dbias)
                dbias[e] += dl;
        }
    }
    free(xt);
    free(dy);
    free(g);
    free(u);
    free(a);
    free(z);
    free(dg);
    free(du);
}
