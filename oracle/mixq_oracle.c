/*
 * CPU oracle for the MixQ-style mixed-precision linear layer  Y = X . W^T.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously-correct
 * definition that the GPU path is checked against.  Only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg load it; the product path
 * (the HIP library and its Python binding) never includes, links or calls it,
 * and it shares no code, header or table with that path.
 *
 * Sources (the method is described in prose only; no code was printed):
 *   [MixQ]   news article on MixQ, "一键部署LLM混合精度推理，端到端吞吐比AWQ
 *            最大提升6倍！": section "研究背景：已有量化技术总结" (Fig. 5, the
 *            mixed-precision split) and section "MixQ的解决方案" (Fig. 9 outlier
 *            locality, the amax-vs-threshold paragraph, Fig. 10 equivalent graph
 *            transform, Fig. 11 order-preserving outlier matrix, Fig. 12 fused
 *            dequantize/scale/add).
 *   [FP6]    explainer "DeepSpeed FP6以 FP6 量化与 TC-FPx 全栈 GPU Kernel 为核心的
 *            LLM 推理服务加速", section 3 (per-output-channel scale = max|x| over
 *            the range, a zero scale replaced by 1, round to nearest).
 *
 * Readings taken where the pages are silent (each is listed in the design
 * notes of the repository):
 *   - an activation channel is an outlier when some token in the call has
 *     |x| strictly greater than the threshold ("大于" in [MixQ]);
 *   - the gate looks at the amax over channels not already cached, and a
 *     firing gate adds the newly detected channels to the cached set (union);
 *   - per-token scale over the non-outlier channels, symmetric codes in
 *     [-(2^(b-1)-1), 2^(b-1)-1], one reciprocal per row, round half to even;
 *   - outlier columns in ascending channel order, zero padded;
 *   - the final output is computed in double precision here (the GPU writes
 *     fp32; the two are compared within a tolerance).
 *
 * Floating point: every float operation is a single IEEE binary32 operation
 * with round-to-nearest-even (build with -ffp-contract=off, no fast-math).
 * Parity unpinned: none (every function is pinned by the CPU test suite).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* IEEE binary16 bit pattern -> float, decoded from the format definition. */
float orc_half_to_float(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 31;
    int mant = h & 1023;
    float v;
    if (expo == 0)
        v = ldexpf((float)mant, -24);               /* subnormal: m * 2^-24 */
    else if (expo == 31)
        v = mant ? NAN : INFINITY;
    else
        v = ldexpf((float)(mant + 1024), expo - 25); /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* Largest code of a symmetric b-bit integer: 127 for INT8, 7 for INT4. */
static int qmax_for_bits(int bits)
{
    return (1 << (bits - 1)) - 1;
}

/* Scale and reciprocal from an amax, with the zero-scale rule of [FP6] s3. */
static void scale_from_amax(float amax, int qmax, float *scale, float *recip)
{
    if (amax == 0.0f) {
        *scale = 1.0f;
        *recip = 1.0f;
    } else {
        *scale = amax / (float)qmax;
        *recip = (float)qmax / amax;
    }
}

/* Round half to even, then clamp to the symmetric code range. */
static int8_t quantize_value(float x, float recip, int qmax)
{
    float y = nearbyintf(x * recip);
    if (y > (float)qmax) y = (float)qmax;
    if (y < (float)-qmax) y = (float)-qmax;
    return (int8_t)y;
}

/*
 * Gate + re-detection + union.  [MixQ] "MixQ的解决方案": outliers recur in
 * fixed channels across decode steps (Fig. 9), so the set is cached; the amax
 * that quantization needs anyway tells whether any outlier exists (amax above
 * the threshold), and only then is detection needed (Fig. 10).
 *
 *   in_set [K]  in: cached set (0/1); out: the set after this call.
 *   flag        out: 0 = gate closed, set unchanged;
 *                    1 = gate fired, newly detected channels added;
 *                    2 = gate fired but the union would exceed k_cap; the set
 *                        is left unchanged.
 *   returns the size of the set after the call.
 */
int32_t orc_update_outlier_set(const uint16_t *X, int64_t M, int64_t K, int64_t ldx,
                               float tau, int32_t k_cap, uint8_t *in_set,
                               int32_t *flag)
{
    int64_t m, k;
    int fired = 0;
    int32_t before = 0, after = 0;
    uint8_t *cand;

    for (k = 0; k < K; ++k)
        before += in_set[k] ? 1 : 0;

    /* gate: amax over the channels not already cached, compared strictly */
    for (m = 0; m < M && !fired; ++m) {
        float g = 0.0f;
        for (k = 0; k < K; ++k) {
            if (in_set[k]) continue;
            float a = fabsf(orc_half_to_float(X[m * ldx + k]));
            if (a > g) g = a;
        }
        if (g > tau) fired = 1;
    }
    if (!fired) {
        *flag = 0;
        return before;
    }

    /* detection: a channel is an outlier if any token exceeds the threshold */
    cand = (uint8_t *)malloc((size_t)K);
    for (k = 0; k < K; ++k) {
        int hit = in_set[k] ? 1 : 0;
        for (m = 0; m < M && !hit; ++m)
            if (fabsf(orc_half_to_float(X[m * ldx + k])) > tau) hit = 1;
        cand[k] = (uint8_t)hit;
        after += hit;
    }
    if (after > k_cap) {
        *flag = 2;
        free(cand);
        return before;
    }
    memcpy(in_set, cand, (size_t)K);
    free(cand);
    *flag = 1;
    return after;
}

/* Ascending list of the set's channels (the order-preserving concatenation
 * order of [MixQ] Fig. 11).  Returns its length. */
int32_t orc_outlier_list(const uint8_t *in_set, int64_t K, int32_t *idx)
{
    int32_t n = 0;
    int64_t k;
    for (k = 0; k < K; ++k)
        if (in_set[k]) idx[n++] = (int32_t)k;
    return n;
}

/*
 * Per-token activation quantization with outliers split out.
 * [MixQ] Fig. 5: most of the activations go to low bit, outliers stay in FP16;
 * Fig. 11: the outlier channels are concatenated, in order, into a new matrix.
 *
 *   Xq    [M, K] int8: code of every non-outlier element, 0 on outlier channels
 *   s_x   [M]        : per-token scale = amax over non-outlier channels / 127
 *   X_out [M, ldo]   : X at the outlier channels in ascending order, then zeros
 */
void orc_quantize_act(const uint16_t *X, int64_t M, int64_t K, int64_t ldx,
                      const uint8_t *in_set, int8_t *Xq, float *s_x,
                      uint16_t *X_out, int64_t ldo)
{
    int64_t m;
    const int qmax = 127;
#pragma omp parallel for schedule(static)
    for (m = 0; m < M; ++m) {
        const uint16_t *row = X + m * ldx;
        float amax = 0.0f, scale, recip;
        int64_t k, j;
        for (k = 0; k < K; ++k) {
            if (in_set[k]) continue;
            float a = fabsf(orc_half_to_float(row[k]));
            if (a > amax) amax = a;
        }
        scale_from_amax(amax, qmax, &scale, &recip);
        s_x[m] = scale;
        for (k = 0; k < K; ++k)
            Xq[m * K + k] = in_set[k] ? 0
                                      : quantize_value(orc_half_to_float(row[k]), recip, qmax);
        j = 0;
        for (k = 0; k < K; ++k)
            if (in_set[k] && j < ldo) X_out[m * ldo + j++] = row[k];
        for (; j < ldo; ++j)
            X_out[m * ldo + j] = 0;
    }
}

/*
 * Per-output-channel symmetric weight quantization ([FP6] s3: scale is the
 * row's max |w| over the code range, a zero scale becomes 1).  The amax runs
 * over all K input channels; the code at an outlier channel never contributes
 * because the matching activation code is 0.
 *   Wq [N, K] int8 (unpacked codes, also for bits = 4), s_w [N].
 */
void orc_quantize_weight(const uint16_t *W, int64_t N, int64_t K, int bits,
                         int8_t *Wq, float *s_w)
{
    int64_t n;
    const int qmax = qmax_for_bits(bits);
#pragma omp parallel for schedule(static)
    for (n = 0; n < N; ++n) {
        const uint16_t *row = W + n * K;
        float amax = 0.0f, scale, recip;
        int64_t k;
        for (k = 0; k < K; ++k) {
            float a = fabsf(orc_half_to_float(row[k]));
            if (a > amax) amax = a;
        }
        scale_from_amax(amax, qmax, &scale, &recip);
        s_w[n] = scale;
        for (k = 0; k < K; ++k)
            Wq[n * K + k] = quantize_value(orc_half_to_float(row[k]), recip, qmax);
    }
}

/* FP16 weight columns at the outlier channels, ascending, then zeros.
 * W_out[n, j] = W[n, I[j]].  [MixQ] Fig. 11. */
void orc_gather_weight_cols(const uint16_t *W, int64_t N, int64_t K,
                            const uint8_t *in_set, uint16_t *W_out, int64_t ldo)
{
    int64_t n;
#pragma omp parallel for schedule(static)
    for (n = 0; n < N; ++n) {
        int64_t k, j = 0;
        for (k = 0; k < K; ++k)
            if (in_set[k] && j < ldo) W_out[n * ldo + j++] = W[n * K + k];
        for (; j < ldo; ++j)
            W_out[n * ldo + j] = 0;
    }
}

/*
 * Low-precision product: acc[m, n] = sum_k Xq[m, k] * Wq[n, k], summed in
 * 64-bit integers.  Returns 0, or -1 if some sum does not fit in int32.
 */
int orc_int_gemm(const int8_t *Xq, const int8_t *Wq, int64_t M, int64_t N,
                 int64_t K, int32_t *acc)
{
    int64_t m;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (m = 0; m < M; ++m) {
        int64_t n, k;
        for (n = 0; n < N; ++n) {
            int64_t s = 0;
            for (k = 0; k < K; ++k)
                s += (int64_t)Xq[m * K + k] * (int64_t)Wq[n * K + k];
            if (s > INT32_MAX || s < INT32_MIN) bad = 1;
            acc[m * N + n] = (int32_t)s;
        }
    }
    return bad ? -1 : 0;
}

/*
 * Output: the low-precision result dequantized and scaled, plus the FP16
 * outlier product ([MixQ] Fig. 12).  In double precision:
 *   Y[m, n] = acc[m, n] * s_x[m] * s_w[n] + sum_{j<k} X_out[m, j] * W_out[n, j]
 */
void orc_output(const int32_t *acc, const float *s_x, const float *s_w,
                const uint16_t *X_out, int64_t ldxo, const uint16_t *W_out,
                int64_t ldwo, int64_t M, int64_t N, int64_t k, double *Y)
{
    int64_t m;
#pragma omp parallel for schedule(static)
    for (m = 0; m < M; ++m) {
        int64_t n, j;
        for (n = 0; n < N; ++n) {
            double y = (double)acc[m * N + n] * (double)s_x[m] * (double)s_w[n];
            for (j = 0; j < k; ++j)
                y += (double)orc_half_to_float(X_out[m * ldxo + j]) *
                     (double)orc_half_to_float(W_out[n * ldwo + j]);
            Y[m * N + n] = y;
        }
    }
}

/*
 * The same two steps for chosen (row, col) pairs only, for shapes where the
 * full product is too slow on a CPU.  Xq is [*, K], Wq is [*, K].
 */
int orc_sampled_output(const int8_t *Xq, const int8_t *Wq, int64_t K,
                       const float *s_x, const float *s_w,
                       const uint16_t *X_out, int64_t ldxo,
                       const uint16_t *W_out, int64_t ldwo, int64_t k,
                       const int64_t *rows, const int64_t *cols, int64_t S,
                       int32_t *acc, double *Y)
{
    int64_t i;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (i = 0; i < S; ++i) {
        int64_t m = rows[i], n = cols[i], kk, j;
        int64_t s = 0;
        double y;
        for (kk = 0; kk < K; ++kk)
            s += (int64_t)Xq[m * K + kk] * (int64_t)Wq[n * K + kk];
        if (s > INT32_MAX || s < INT32_MIN) bad = 1;
        acc[i] = (int32_t)s;
        y = (double)(int32_t)s * (double)s_x[m] * (double)s_w[n];
        for (j = 0; j < k; ++j)
            y += (double)orc_half_to_float(X_out[m * ldxo + j]) *
                 (double)orc_half_to_float(W_out[n * ldwo + j]);
        Y[i] = y;
    }
    return bad ? -1 : 0;
}
