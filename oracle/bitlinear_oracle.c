/*
 * bitlinear_oracle.c -- CPU oracle for the BitNet b1.58 BitLinear forward
 * (W1.58A8).  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the
 * benchmark's CPU-baseline leg call it; the product path never does.
 *
 * Plain, single-threaded, slow on purpose.  Every function follows one step
 * of the method as the pages state it, in the order they state it; nothing is
 * blocked, fused or reordered.  It shares no code, header, table or constant
 * generator with the HIP library.
 *
 * Build: gcc -std=c11 -O2 -ffp-contract=off -fno-fast-math -shared -fPIC
 * (no FMA contraction, default rounding, no flush-to-zero).
 *
 * Sources (page title, then the section on it):
 *  [Q]  "BitNet", Transformers quantization guide (Portuguese edition),
 *       numbered list of the three quantization steps.
 *  [T]  "Transformers 实战 BitNet 1.58 位量化：BitLinear 原理、量化流程与推理加载全指南",
 *       sections "BitLinear 的三步量化" (steps 1-3) and
 *       "推理侧 BitLinear：打包权重、解包与缩放" (pack / unpack / forward),
 *       and the subln paragraph that follows it.
 *  [M]  "BitNet" model documentation (Chinese and Portuguese editions),
 *       "模型详情" / "Detalhes do Modelo" (ReLU squared, subln, no bias,
 *       W1.58A8) and "BitNetConfig" (rms_norm_eps = 1e-5, shapes).
 *
 * Readings where the pages are open (each also listed in the design notes):
 *  - weight codes divide by the absmean scale ([Q] step 2 divides; [T] step 2
 *    multiplies by its reciprocal): we divide, in fp32;
 *  - the mean is accumulated in fp64 in index order, rounded to fp32, then
 *    floored at 1e-5;
 *  - activation absmax is per token (per row), the floor applies to the max;
 *  - rounding is half-to-even (nearbyint), as torch's round() does;
 *  - packing is plane order: field i (bits 2i..2i+1) of packed row r holds
 *    weight row i*N/4 + r;
 *  - rescale: y = float(A) * (w_mean / a), fp32;
 *  - RMSNorm: x * 1/sqrt(mean(x^2) + eps), sum in fp64, then times the gain.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORA_EPS_SCALE 1e-5f

/* ---------------------------------------------------------------------------
 * Weight scale.  [Q] step 1, [T] "三步量化" step 1: the scale of a weight
 * tensor is the mean of |W| over the whole tensor (symmetric, per tensor),
 * floored at 1e-5 so an all-zero tensor does not divide by zero.
 * Returns w_mean = max(float(sum|W| / count), 1e-5).
 * ------------------------------------------------------------------------ */
float ora_weight_mean(const float *W, int64_t count)
{
    double s = 0.0;
    for (int64_t i = 0; i < count; ++i)
        s += fabs((double)W[i]);
    double m = s / (double)count;
    float mf = (float)m;
    return mf < ORA_EPS_SCALE ? ORA_EPS_SCALE : mf;
}

/* ---------------------------------------------------------------------------
 * Ternary codes.  [Q] step 2, [T] "三步量化" step 2: divide the weights by the
 * scale, round to the nearest integer, clip to [-1, 1].  Codes in {-1,0,1}.
 * ------------------------------------------------------------------------ */
void ora_ternarize(const float *W, int64_t count, float w_mean, int8_t *codes)
{
    for (int64_t i = 0; i < count; ++i) {
        float t = W[i] / w_mean;          /* fp32 IEEE division          */
        float r = nearbyintf(t);          /* round half to even          */
        if (r > 1.0f) r = 1.0f;
        if (r < -1.0f) r = -1.0f;
        codes[i] = (int8_t)r;
    }
}

/* QAT fake-quant weight: codes mapped back to the full-precision range
 * ([T] "三步量化" step 2, the final division by the reciprocal scale). */
void ora_fake_quant_weight(const int8_t *codes, int64_t count, float w_mean, float *out)
{
    for (int64_t i = 0; i < count; ++i)
        out[i] = (float)codes[i] * w_mean;
}

/* ---------------------------------------------------------------------------
 * Packing.  [T] "推理侧 BitLinear", pack bullet: each code is shifted by +1 to
 * {0,1,2}, and four 2-bit values share one uint8, so the packed tensor has a
 * quarter of the rows.  Unpack bullet: field i is selected by the mask 3<<2i
 * and 1 is subtracted.
 * Reading: plane order.  Packed row r, field i holds code row i*N/4 + r.
 * codes: [N,K] row-major; packed: [N/4,K] row-major.  N % 4 == 0.
 * ------------------------------------------------------------------------ */
void ora_pack(const int8_t *codes, int N, int K, uint8_t *packed)
{
    int R = N / 4;
    for (int r = 0; r < R; ++r)
        for (int k = 0; k < K; ++k) {
            unsigned byte = 0;
            for (int i = 0; i < 4; ++i) {
                int n = i * R + r;
                unsigned v = (unsigned)(codes[(int64_t)n * K + k] + 1);
                byte |= v << (2 * i);
            }
            packed[(int64_t)r * K + k] = (uint8_t)byte;
        }
}

/* Inverse of ora_pack.  Returns the number of fields holding the unused
 * value 3 (those decode to 2 and are reported, never produced by packing). */
int64_t ora_unpack(const uint8_t *packed, int N, int K, int8_t *codes)
{
    int R = N / 4;
    int64_t bad = 0;
    for (int r = 0; r < R; ++r)
        for (int k = 0; k < K; ++k) {
            unsigned byte = packed[(int64_t)r * K + k];
            for (int i = 0; i < 4; ++i) {
                unsigned v = (byte & (3u << (2 * i))) >> (2 * i);
                if (v == 3) ++bad;
                codes[(int64_t)(i * R + r) * K + k] = (int8_t)((int)v - 1);
            }
        }
    return bad;
}

/* ---------------------------------------------------------------------------
 * Activation quantization.  [Q] step 3, [T] "三步量化" step 3, [M] "模型详情":
 * absmax to 8 bits per token.  For each row m:
 *   a_m = 127 / max(max_k |x[m,k]|, 1e-5)        (fp32 division)
 *   q   = clip(round(x * a_m), -128, 127)       (fp32 multiply, half-even)
 * x: [M,K] fp32 (bf16 inputs are widened exactly by the caller).
 * ------------------------------------------------------------------------ */
void ora_quant_act(const float *x, int M, int K, int8_t *q, float *a)
{
    for (int m = 0; m < M; ++m) {
        const float *row = x + (int64_t)m * K;
        float amax = 0.0f;
        for (int k = 0; k < K; ++k) {
            float v = fabsf(row[k]);
            if (v > amax) amax = v;
        }
        if (amax < ORA_EPS_SCALE) amax = ORA_EPS_SCALE;
        float s = 127.0f / amax;
        a[m] = s;
        for (int k = 0; k < K; ++k) {
            float t = row[k] * s;
            float r = nearbyintf(t);
            if (r > 127.0f) r = 127.0f;
            if (r < -128.0f) r = -128.0f;
            q[(int64_t)m * K + k] = (int8_t)r;
        }
    }
}

/* ---------------------------------------------------------------------------
 * Contraction.  [T] "推理侧 BitLinear", forward bullet: the linear product of
 * the int8 activations with the unpacked ternary weights.  Integer result:
 *   A[m,n] = sum_k q[m,k] * c[n,k]     (int64 accumulate, stored as int32)
 * Returns the number of results that do not fit in int32 (always 0 for
 * |q| <= 128 and K < 2^23).
 * ------------------------------------------------------------------------ */
int64_t ora_contract(const int8_t *q, int M, int K, const int8_t *codes, int N, int32_t *A)
{
    int64_t overflow = 0;
    for (int m = 0; m < M; ++m)
        for (int n = 0; n < N; ++n) {
            int64_t s = 0;
            for (int k = 0; k < K; ++k)
                s += (int64_t)q[(int64_t)m * K + k] * (int64_t)codes[(int64_t)n * K + k];
            if (s > INT32_MAX || s < INT32_MIN) ++overflow;
            A[(int64_t)m * N + n] = (int32_t)s;
        }
    return overflow;
}

/* ---------------------------------------------------------------------------
 * Rescale.  [T] "推理侧 BitLinear", forward bullet (post_quant_process): the
 * output is brought back to its range by the activation scale and the weight
 * scale.  With a_m = 127/absmax and w_mean the absmean, that is
 *   y[m,n] = float(A[m,n]) * (w_mean_s / a_m)     (fp32, s = segment of n)
 * Segments: n_seg tensors concatenated along N, widths seg_n[], each with
 * its own w_mean.
 * ------------------------------------------------------------------------ */
void ora_rescale(const int32_t *A, int M, int N, const float *a,
                 int n_seg, const int *seg_n, const float *w_mean, float *y)
{
    for (int m = 0; m < M; ++m) {
        int n0 = 0;
        for (int s = 0; s < n_seg; ++s) {
            float sc = w_mean[s] / a[m];
            for (int n = n0; n < n0 + seg_n[s]; ++n)
                y[(int64_t)m * N + n] = (float)A[(int64_t)m * N + n] * sc;
            n0 += seg_n[s];
        }
    }
}

/* fp32 -> bf16 (round to nearest even on the bit pattern; finite input). */
void ora_to_bf16(const float *y, int64_t count, uint16_t *out)
{
    for (int64_t i = 0; i < count; ++i) {
        uint32_t u;
        memcpy(&u, &y[i], 4);
        uint32_t lsb = (u >> 16) & 1u;
        out[i] = (uint16_t)((u + 0x7FFFu + lsb) >> 16);
    }
}

/* ---------------------------------------------------------------------------
 * Independent cross-check of contraction + rescale: the dequantized product
 *   y[m,n] = sum_k (q[m,k] / a_m) * (c[n,k] * w_mean_s)      in fp64.
 * ------------------------------------------------------------------------ */
void ora_dequant_f64(const int8_t *q, const float *a, int M, int K,
                     const int8_t *codes, int N, int n_seg, const int *seg_n,
                     const float *w_mean, double *y)
{
    for (int m = 0; m < M; ++m) {
        int n0 = 0;
        for (int s = 0; s < n_seg; ++s) {
            for (int n = n0; n < n0 + seg_n[s]; ++n) {
                double acc = 0.0;
                for (int k = 0; k < K; ++k)
                    acc += ((double)q[(int64_t)m * K + k] / (double)a[m]) *
                           ((double)codes[(int64_t)n * K + k] * (double)w_mean[s]);
                y[(int64_t)m * N + n] = acc;
            }
            n0 += seg_n[s];
        }
    }
}

/* ---------------------------------------------------------------------------
 * RMSNorm (subln).  [T] subln paragraph after "推理侧 BitLinear": the attention
 * output and the MLP activation are normalized before the next projection;
 * [M] "BitNetConfig": rms_norm_eps = 1e-5, no bias.  The pages print no
 * formula; reading: the textbook RMSNorm with eps inside the root,
 *   r = float(1 / sqrt(sum_k h^2 / K + eps))   (fp64),
 *   out = (h * r) * g                          (fp32, g omitted when NULL).
 * ------------------------------------------------------------------------ */
void ora_rmsnorm(const float *h, int M, int K, const float *g, float eps, float *out)
{
    for (int m = 0; m < M; ++m) {
        const float *row = h + (int64_t)m * K;
        double ss = 0.0;
        for (int k = 0; k < K; ++k)
            ss += (double)row[k] * (double)row[k];
        float r = (float)(1.0 / sqrt(ss / (double)K + (double)eps));
        for (int k = 0; k < K; ++k) {
            float v = row[k] * r;
            if (g) v = v * g[k];
            out[(int64_t)m * K + k] = v;
        }
    }
}

/* ---------------------------------------------------------------------------
 * FFN activation.  [M] "模型详情" and "BitNetConfig" (hidden_act relu2): the
 * gate branch goes through squared ReLU and multiplies the up branch.
 *   p = (max(g,0) * max(g,0)) * u     (fp32, two roundings, no FMA)
 * ------------------------------------------------------------------------ */
void ora_relu2_mul(const float *gate, const float *up, int64_t count, float *p)
{
    for (int64_t i = 0; i < count; ++i) {
        float gp = gate[i] > 0.0f ? gate[i] : 0.0f;
        float sq = gp * gp;
        p[i] = sq * up[i];
    }
}

/* ---------------------------------------------------------------------------
 * One BitLinear forward on already-quantized weights:
 * quantize x (per token) -> integer product -> rescale.
 * codes: [N,K] stacked segments.  Outputs q [M,K], a [M], A [M,N], y [M,N].
 * ------------------------------------------------------------------------ */
void ora_bitlinear(const float *x, int M, int K, const int8_t *codes, int N,
                   int n_seg, const int *seg_n, const float *w_mean,
                   int8_t *q, float *a, int32_t *A, float *y)
{
    ora_quant_act(x, M, K, q, a);
    ora_contract(q, M, K, codes, N, A);
    ora_rescale(A, M, N, a, n_seg, seg_n, w_mean, y);
}

/* ---------------------------------------------------------------------------
 * FFN chain of one layer ([T] subln paragraph; [M] "模型详情"):
 *   subln RMSNorm(h) -> quantize -> gate|up (two segments) -> ReLU^2(gate)*up
 *   -> ffn_sub_norm RMSNorm -> quantize -> down.
 * h: [M,H]; codes_gu: [2I,H] (gate rows then up rows); codes_down: [H,I].
 * Stage outputs (all required): q1 [M,H], a1 [M], p [M,I], q2 [M,I], a2 [M];
 * y [M,H].  g_subln / g_ffn may be NULL (unit gain).
 * ------------------------------------------------------------------------ */
void ora_ffn_chain(const float *h, int M, int H, int I,
                   const float *g_subln, const float *g_ffn, float eps,
                   const int8_t *codes_gu, const float *w_mean_gu,
                   const int8_t *codes_down, const float *w_mean_down,
                   int8_t *q1, float *a1, float *p, int8_t *q2, float *a2, float *y)
{
    float *hn = (float *)malloc(sizeof(float) * (size_t)M * H);
    int32_t *Agu = (int32_t *)malloc(sizeof(int32_t) * (size_t)M * 2 * I);
    float *ygu = (float *)malloc(sizeof(float) * (size_t)M * 2 * I);
    float *gate = (float *)malloc(sizeof(float) * (size_t)M * I);
    float *up = (float *)malloc(sizeof(float) * (size_t)M * I);
    float *pn = (float *)malloc(sizeof(float) * (size_t)M * I);
    int32_t *Ad = (int32_t *)malloc(sizeof(int32_t) * (size_t)M * H);
    int seg_gu[2] = {I, I};
    int seg_d[1] = {H};

    ora_rmsnorm(h, M, H, g_subln, eps, hn);
    ora_bitlinear(hn, M, H, codes_gu, 2 * I, 2, seg_gu, w_mean_gu, q1, a1, Agu, ygu);
    for (int m = 0; m < M; ++m)
        for (int j = 0; j < I; ++j) {
            gate[(int64_t)m * I + j] = ygu[(int64_t)m * 2 * I + j];
            up[(int64_t)m * I + j] = ygu[(int64_t)m * 2 * I + I + j];
        }
    ora_relu2_mul(gate, up, (int64_t)M * I, p);
    ora_rmsnorm(p, M, I, g_ffn, eps, pn);
    ora_bitlinear(pn, M, I, codes_down, H, 1, seg_d, w_mean_down, q2, a2, Ad, y);

    free(hn); free(Agu); free(ygu); free(gate); free(up); free(pn); free(Ad);
}

/* ===========================================================================
 * Attention side of a decoder layer, one new token (decode).
 *  [M] "BitNet" model documentation, "模型详情": the architecture uses rotary
 *      position embeddings (RoPE); "BitNetConfig": 20 attention heads, 5
 *      key/value heads (grouped-query attention: each key/value head serves an
 *      equal group of consecutive query heads), hidden size 2560 (so a head
 *      has 2560 / 20 = 128 dimensions), at most 2048 positions; the RoPE base
 *      (rope_theta) is a parameter whose value the pages do not print.
 * Readings (also in the design notes): the rotation pairs dimension i with
 * i + D/2 of a head (the split-half convention), at angle
 * pos * base^(-2i/D); the new token attends to every cached position and to
 * itself (positions 0 .. pos); scores are scaled by 1/sqrt(D); softmax with
 * the maximum subtracted.  Everything here is fp64; inputs and the cached
 * keys/values are fp32.
 * ------------------------------------------------------------------------ */

/* RoPE of nh heads of D dims at position pos, fp64 in, fp64 out. */
void ora_rope_f64(const double *x, int nh, int D, int pos, double base, double *y)
{
    const int h2 = D / 2;
    for (int h = 0; h < nh; ++h)
        for (int i = 0; i < h2; ++i) {
            const double ang = (double)pos * pow(base, -2.0 * (double)i / (double)D);
            const double c = cos(ang), s = sin(ang);
            const double a = x[(int64_t)h * D + i], b = x[(int64_t)h * D + h2 + i];
            y[(int64_t)h * D + i] = a * c - b * s;
            y[(int64_t)h * D + h2 + i] = b * c + a * s;
        }
}

/* Decode attention for one token.
 *   q [H*D], k_new [KVH*D], v_new [KVH*D]: the new token's projections (fp32,
 *     before RoPE);
 *   k_cache, v_cache [KVH][max_seq][D] fp32: positions 0 .. pos-1 hold the
 *     earlier tokens' rotated keys and their values (position pos is the new
 *     token's, taken from k_new / v_new here);
 *   out [H*D] fp64: softmax(q' k'^T / sqrt(D)) v per query head h, with key /
 *     value head h / (H / KVH). */
void ora_attn_decode(const float *q, const float *k_new, const float *v_new, int pos,
                     int H, int KVH, int D, const float *k_cache, const float *v_cache,
                     int max_seq, double base, double *out)
{
    const int G = H / KVH;
    double *qd = (double *)malloc(sizeof(double) * (size_t)H * D);
    double *qr = (double *)malloc(sizeof(double) * (size_t)H * D);
    double *kd = (double *)malloc(sizeof(double) * (size_t)KVH * D);
    double *kr = (double *)malloc(sizeof(double) * (size_t)KVH * D);
    double *sc = (double *)malloc(sizeof(double) * (size_t)(pos + 1));
    for (int64_t i = 0; i < (int64_t)H * D; ++i) qd[i] = (double)q[i];
    for (int64_t i = 0; i < (int64_t)KVH * D; ++i) kd[i] = (double)k_new[i];
    ora_rope_f64(qd, H, D, pos, base, qr);
    ora_rope_f64(kd, KVH, D, pos, base, kr);
    const double scale = 1.0 / sqrt((double)D);
    for (int h = 0; h < H; ++h) {
        const int g = h / G;
        double mx = -INFINITY;
        for (int j = 0; j <= pos; ++j) {
            double s = 0.0;
            for (int d = 0; d < D; ++d) {
                const double kv = j < pos ? (double)k_cache[((int64_t)g * max_seq + j) * D + d] : kr[(int64_t)g * D + d];
                s += qr[(int64_t)h * D + d] * kv;
            }
            sc[j] = s * scale;
            if (sc[j] > mx) mx = sc[j];
        }
        double l = 0.0;
        for (int j = 0; j <= pos; ++j) {
            sc[j] = exp(sc[j] - mx);
            l += sc[j];
        }
        for (int d = 0; d < D; ++d) {
            double o = 0.0;
            for (int j = 0; j <= pos; ++j) {
                const double vv = j < pos ? (double)v_cache[((int64_t)g * max_seq + j) * D + d] : (double)v_new[(int64_t)g * D + d];
                o += sc[j] * vv;
            }
            out[(int64_t)h * D + d] = o / l;
        }
    }
    free(qd); free(qr); free(kd); free(kr); free(sc);
}

/* ===========================================================================
 * Attention side of a decoder layer over a prompt (prefill): the tokens sit
 * at positions 0 .. M-1 and token p attends to positions 0 .. p (causal).
 * Same pages and readings as ora_attn_decode: RoPE with dimension i paired
 * with i + D/2 at angle pos * base^(-2i/D) on queries and keys, scores scaled
 * by 1/sqrt(D), softmax with the maximum subtracted, query head h reading
 * key/value head h / (H / KVH).  The plain definition in fp64 throughout: the
 * rotated queries and keys are never rounded, the values are the fp32 inputs.
 *   q [M][H*D], k [M][KVH*D], v [M][KVH*D] fp32 (before RoPE), contiguous;
 *   rows[nrows]: the token positions whose outputs are wanted;
 *   out [nrows][H*D] fp64.
 * ------------------------------------------------------------------------ */
void ora_attn_prefill_f64(const float *q, const float *k, const float *v, int M, int H, int KVH, int D,
                          double base, const int *rows, int nrows, double *out)
{
    const int G = H / KVH;
    int pmax = 0;
    for (int r = 0; r < nrows; ++r)
        if (rows[r] > pmax) pmax = rows[r];
    if (pmax >= M) pmax = M - 1;
    const int64_t kw = (int64_t)KVH * D;
    double *kd = (double *)malloc(sizeof(double) * (size_t)kw);
    double *kr = (double *)malloc(sizeof(double) * (size_t)(pmax + 1) * kw);
    double *qd = (double *)malloc(sizeof(double) * (size_t)H * D);
    double *qr = (double *)malloc(sizeof(double) * (size_t)H * D);
    double *sc = (double *)malloc(sizeof(double) * (size_t)(pmax + 1));
    for (int j = 0; j <= pmax; ++j) {
        for (int64_t i = 0; i < kw; ++i) kd[i] = (double)k[(int64_t)j * kw + i];
        ora_rope_f64(kd, KVH, D, j, base, kr + (int64_t)j * kw);
    }
    const double scale = 1.0 / sqrt((double)D);
    for (int r = 0; r < nrows; ++r) {
        const int p = rows[r];
        for (int64_t i = 0; i < (int64_t)H * D; ++i) qd[i] = (double)q[(int64_t)p * H * D + i];
        ora_rope_f64(qd, H, D, p, base, qr);
        for (int h = 0; h < H; ++h) {
            const int g = h / G;
            double mx = -INFINITY;
            for (int j = 0; j <= p; ++j) {
                double s = 0.0;
                for (int d = 0; d < D; ++d)
                    s += qr[(int64_t)h * D + d] * kr[(int64_t)j * kw + (int64_t)g * D + d];
                sc[j] = s * scale;
                if (sc[j] > mx) mx = sc[j];
            }
            double l = 0.0;
            for (int j = 0; j <= p; ++j) {
                sc[j] = exp(sc[j] - mx);
                l += sc[j];
            }
            for (int d = 0; d < D; ++d) {
                double o = 0.0;
                for (int j = 0; j <= p; ++j)
                    o += sc[j] * (double)v[(int64_t)j * kw + (int64_t)g * D + d];
                out[(int64_t)r * H * D + (int64_t)h * D + d] = o / l;
            }
        }
    }
    free(kd); free(kr); free(qd); free(qr); free(sc);
}

/* ===========================================================================
 * Backward of BitLinear in quantization-aware training.  [T] "BitLinear 的三步
 * 量化": in training both quantizers hand the incoming gradient through
 * unchanged (straight-through estimator), so the layer's gradients are those
 * of a plain linear layer evaluated at the fake-quantized tensors
 *   W~ = codes * w_mean           (the ternary weight mapped back to its range)
 *   x~ = q / a                    (the int8 activation mapped back)
 *   dX = dY . W~,   dW = dY^T . x~.
 * The plain definitions in fp64; dy is the fp32 output gradient.  Only the
 * requested rows are formed (whole products are large).
 * ------------------------------------------------------------------------ */

/* dx[r][k] = sum_n dy[m][n] * (codes[n][k] * w_mean), m = rows[r].
 * dy [M][N] fp32; codes [N][K] int8; dx [nrows][K] fp64. */
void ora_ste_grad_input_rows(const float *dy, int M, int N, const int8_t *codes, int K, float w_mean,
                             const int *rows, int nrows, double *dx)
{
    (void)M;
    for (int r = 0; r < nrows; ++r) {
        const int m = rows[r];
        double *o = dx + (int64_t)r * K;
        for (int kk = 0; kk < K; ++kk) o[kk] = 0.0;
        for (int n = 0; n < N; ++n) {
            const double g = (double)dy[(int64_t)m * N + n];
            const int8_t *c = codes + (int64_t)n * K;
            for (int kk = 0; kk < K; ++kk)
                o[kk] += g * ((double)c[kk] * (double)w_mean);
        }
    }
}

/* dw[r][k] = sum_m dy[m][n] * (q[m][k] / a[m]), n = rows[r].
 * dy [M][N] fp32; q [M][K] int8; a [M] fp32; dw [nrows][K] fp64. */
void ora_ste_grad_weight_rows(const float *dy, int M, int N, const int8_t *q, const float *a, int K,
                              const int *rows, int nrows, double *dw)
{
    for (int r = 0; r < nrows; ++r) {
        const int n = rows[r];
        double *o = dw + (int64_t)r * K;
        for (int kk = 0; kk < K; ++kk) o[kk] = 0.0;
        for (int m = 0; m < M; ++m) {
            const double g = (double)dy[(int64_t)m * N + n];
            const int8_t *qm = q + (int64_t)m * K;
            for (int kk = 0; kk < K; ++kk)
                o[kk] += g * ((double)qm[kk] / (double)a[m]);
        }
    }
}

/* ===========================================================================
 * The 1-bit BitLinear (binarized weights).
 *  [S] project summary of a PyTorch "BitNet" implementation of 1-bit
 *      Transformers, section "How It Works": the BitLinear that replaces a
 *      linear layer quantizes its weights to one bit by binarization, and
 *      its input through layer normalization followed by absolute-maximum
 *      quantization.
 * The page prints no formula.  Readings (also in the design notes):
 *  - weight: sign(W), negative -> -1, anything else (zero included) -> +1;
 *    one scale per tensor, the mean of |W| as for the ternary scale
 *    (ora_weight_mean: fp64 sum in index order, fp32, floor 1e-5);
 *  - packing: one bit per weight, plane order: bit i of packed row r holds
 *    weight row i*N/8 + r (1 for +1, 0 for -1); N % 8 == 0;
 *  - layer normalization per token over K, with optional gain and bias:
 *      mu  = sum_k x / K                    (fp64, index order)
 *      var = sum_k (x - mu)^2 / K           (fp64, index order)
 *      r   = float(1 / sqrt(var + eps))     (fp64, then fp32)
 *      out = (float(x - mu) * r) * gamma + beta   (fp32, no FMA)
 *  - activations: the per-token absmax int8 quantization of the ternary
 *    path (ora_quant_act);
 *  - output: y = float(A) * (w_scale / a), A = sum_k q * sign (ora_rescale).
 * ------------------------------------------------------------------------ */

/* Binarization ([S] "How It Works"): -1 where W < 0, else +1. */
void ora_binarize(const float *W, int64_t count, int8_t *signs)
{
    for (int64_t i = 0; i < count; ++i)
        signs[i] = W[i] < 0.0f ? (int8_t)-1 : (int8_t)1;
}

/* One bit per weight, plane order (reading above).  signs: [N,K] in {-1,+1};
 * packed: [N/8,K]. */
void ora_pack_bits(const int8_t *signs, int N, int K, uint8_t *packed)
{
    int R = N / 8;
    for (int r = 0; r < R; ++r)
        for (int k = 0; k < K; ++k) {
            unsigned byte = 0;
            for (int i = 0; i < 8; ++i)
                if (signs[(int64_t)(i * R + r) * K + k] > 0)
                    byte |= 1u << i;
            packed[(int64_t)r * K + k] = (uint8_t)byte;
        }
}

/* Inverse of ora_pack_bits. */
void ora_unpack_bits(const uint8_t *packed, int N, int K, int8_t *signs)
{
    int R = N / 8;
    for (int r = 0; r < R; ++r)
        for (int k = 0; k < K; ++k) {
            unsigned byte = packed[(int64_t)r * K + k];
            for (int i = 0; i < 8; ++i)
                signs[(int64_t)(i * R + r) * K + k] = ((byte >> i) & 1u) ? (int8_t)1 : (int8_t)-1;
        }
}

/* Layer normalization ([S] "How It Works"; formula as read above).
 * gamma / beta may be NULL (1 and 0). */
void ora_layernorm(const float *x, int M, int K, const float *gamma, const float *beta, float eps, float *out)
{
    for (int m = 0; m < M; ++m) {
        const float *row = x + (int64_t)m * K;
        double s = 0.0;
        for (int k = 0; k < K; ++k)
            s += (double)row[k];
        double mu = s / (double)K;
        double ss = 0.0;
        for (int k = 0; k < K; ++k) {
            double d = (double)row[k] - mu;
            ss += d * d;
        }
        float r = (float)(1.0 / sqrt(ss / (double)K + (double)eps));
        for (int k = 0; k < K; ++k) {
            float v = (float)((double)row[k] - mu) * r;
            if (gamma) v = v * gamma[k];
            if (beta) v = v + beta[k];
            out[(int64_t)m * K + k] = v;
        }
    }
}

/* One 1-bit BitLinear forward ([S] "How It Works", steps in the order the
 * page names them): layer norm -> absmax int8 -> product with the signs ->
 * rescale by the weight scale and the activation scale.
 * Outputs q [M,K], a [M], A [M,N], y [M,N]. */
void ora_bitlinear_w1(const float *x, int M, int K, const float *gamma, const float *beta, float eps,
                      const int8_t *signs, int N, float w_scale, int8_t *q, float *a, int32_t *A, float *y)
{
    float *xn = (float *)malloc(sizeof(float) * (size_t)M * K);
    int seg[1] = {N};
    ora_layernorm(x, M, K, gamma, beta, eps, xn);
    ora_quant_act(xn, M, K, q, a);
    ora_contract(q, M, K, signs, N, A);
    ora_rescale(A, M, N, a, 1, seg, &w_scale, y);
    free(xn);
}
