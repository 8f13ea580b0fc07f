/* Driver for the sanitizer build of the oracle (test infrastructure): calls
 * every exported oracle function on small ragged shapes with buffers of
 * exactly the documented sizes, so that AddressSanitizer sees any access past
 * an end and UndefinedBehaviorSanitizer any overflow or bad shift.  Prints a
 * checksum of the outputs and returns 0. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

float ora_weight_mean(const float *W, int64_t count);
void ora_ternarize(const float *W, int64_t count, float w_mean, int8_t *codes);
void ora_fake_quant_weight(const int8_t *codes, int64_t count, float w_mean, float *out);
void ora_pack(const int8_t *codes, int N, int K, uint8_t *packed);
int64_t ora_unpack(const uint8_t *packed, int N, int K, int8_t *codes);
void ora_quant_act(const float *x, int M, int K, int8_t *q, float *a);
int64_t ora_contract(const int8_t *q, int M, int K, const int8_t *codes, int N, int32_t *A);
void ora_rescale(const int32_t *A, int M, int N, const float *a, int n_seg, const int *seg_n, const float *w_mean,
                 float *y);
void ora_to_bf16(const float *y, int64_t count, uint16_t *out);
void ora_dequant_f64(const int8_t *q, const float *a, int M, int K, const int8_t *codes, int N, int n_seg,
                     const int *seg_n, const float *w_mean, double *y);
void ora_rmsnorm(const float *h, int M, int K, const float *g, float eps, float *out);
void ora_relu2_mul(const float *gate, const float *up, int64_t count, float *p);
void ora_bitlinear(const float *x, int M, int K, const int8_t *codes, int N, int n_seg, const int *seg_n,
                   const float *w_mean, int8_t *q, float *a, int32_t *A, float *y);
void ora_ffn_chain(const float *h, int M, int H, int I, const float *g_subln, const float *g_ffn, float eps,
                   const int8_t *codes_gu, const float *w_mean_gu, const int8_t *codes_down, const float *w_mean_down,
                   int8_t *q1, float *a1, float *p, int8_t *q2, float *a2, float *y);
void ora_rope_f64(const double *x, int nh, int D, int pos, double base, double *y);
void ora_attn_decode(const float *q, const float *k_new, const float *v_new, int pos, int H, int KVH, int D,
                     const float *k_cache, const float *v_cache, int max_seq, double base, double *out);
void ora_attn_prefill_f64(const float *q, const float *k, const float *v, int M, int H, int KVH, int D, double base,
                          const int *rows, int nrows, double *out);
void ora_ste_grad_input_rows(const float *dy, int M, int N, const int8_t *codes, int K, float w_mean,
                             const int *rows, int nrows, double *dx);
void ora_ste_grad_weight_rows(const float *dy, int M, int N, const int8_t *q, const float *a, int K, const int *rows,
                              int nrows, double *dw);
void ora_binarize(const float *W, int64_t count, int8_t *signs);
void ora_pack_bits(const int8_t *signs, int N, int K, uint8_t *packed);
void ora_unpack_bits(const uint8_t *packed, int N, int K, int8_t *signs);
void ora_layernorm(const float *x, int M, int K, const float *gamma, const float *beta, float eps, float *out);
void ora_bitlinear_w1(const float *x, int M, int K, const float *gamma, const float *beta, float eps,
                      const int8_t *signs, int N, float w_scale, int8_t *q, float *a, int32_t *A, float *y);

static uint64_t st = 88172645463325252ull;
static double unif(void) { /* xorshift64, in [-1, 1) */
    st ^= st << 13;
    st ^= st >> 7;
    st ^= st << 17;
    return (double)(st >> 11) / (double)(1ull << 52) - 1.0;
}
static float *fbuf(size_t n, double scale) {
    float *p = (float *)malloc(sizeof(float) * (n ? n : 1));
    for (size_t i = 0; i < n; ++i) p[i] = (float)(scale * unif());
    return p;
}
static double sum_f(const float *p, size_t n) {
    double s = 0;
    for (size_t i = 0; i < n; ++i) s += p[i];
    return s;
}
static double sum_d(const double *p, size_t n) {
    double s = 0;
    for (size_t i = 0; i < n; ++i) s += p[i];
    return s;
}

int main(void) {
    double chk = 0;
    /* ternary path: ragged M, N (multiple of 4), K */
    const int M = 3, N = 12, K = 37;
    float *W = fbuf((size_t)N * K, 0.05);
    const float wm = ora_weight_mean(W, (int64_t)N * K);
    int8_t *codes = (int8_t *)malloc((size_t)N * K);
    ora_ternarize(W, (int64_t)N * K, wm, codes);
    float *fq = (float *)malloc(sizeof(float) * N * K);
    ora_fake_quant_weight(codes, (int64_t)N * K, wm, fq);
    uint8_t *packed = (uint8_t *)malloc((size_t)(N / 4) * K);
    ora_pack(codes, N, K, packed);
    int8_t *codes2 = (int8_t *)malloc((size_t)N * K);
    chk += (double)ora_unpack(packed, N, K, codes2);
    float *x = fbuf((size_t)M * K, 3.0);
    int8_t *q = (int8_t *)malloc((size_t)M * K);
    float *a = (float *)malloc(sizeof(float) * M);
    ora_quant_act(x, M, K, q, a);
    int32_t *A = (int32_t *)malloc(sizeof(int32_t) * M * N);
    chk += (double)ora_contract(q, M, K, codes, N, A);
    const int seg[2] = {8, 4};
    const float wms[2] = {wm, 2.0f * wm};
    float *y = (float *)malloc(sizeof(float) * M * N);
    ora_rescale(A, M, N, a, 2, seg, wms, y);
    uint16_t *yb = (uint16_t *)malloc(sizeof(uint16_t) * M * N);
    ora_to_bf16(y, (int64_t)M * N, yb);
    double *yd = (double *)malloc(sizeof(double) * M * N);
    ora_dequant_f64(q, a, M, K, codes, N, 2, seg, wms, yd);
    ora_bitlinear(x, M, K, codes, N, 2, seg, wms, q, a, A, y);
    chk += sum_f(y, (size_t)M * N) + sum_d(yd, (size_t)M * N) + sum_f(fq, (size_t)N * K) + yb[0];
    float *g = fbuf(K, 1.0);
    float *hn = (float *)malloc(sizeof(float) * M * K);
    ora_rmsnorm(x, M, K, g, 1e-5f, hn);
    ora_rmsnorm(x, M, K, NULL, 1e-5f, hn);
    float *pr = (float *)malloc(sizeof(float) * M * K);
    ora_relu2_mul(x, hn, (int64_t)M * K, pr);
    chk += sum_f(pr, (size_t)M * K);

    /* FFN chain: H = 20, I = 12 (gate|up: 2I rows of K = H, down: H rows of K = I) */
    const int Hh = 20, Ii = 12;
    float *h = fbuf((size_t)M * Hh, 2.0);
    float *gs = fbuf(Hh, 1.0), *gf = fbuf(Ii, 1.0);
    float *Wgu = fbuf((size_t)2 * Ii * Hh, 0.05), *Wd = fbuf((size_t)Hh * Ii, 0.05);
    int8_t *cgu = (int8_t *)malloc((size_t)2 * Ii * Hh), *cd = (int8_t *)malloc((size_t)Hh * Ii);
    const float wgu[2] = {ora_weight_mean(Wgu, (int64_t)Ii * Hh), ora_weight_mean(Wgu + Ii * Hh, (int64_t)Ii * Hh)};
    ora_ternarize(Wgu, (int64_t)Ii * Hh, wgu[0], cgu);
    ora_ternarize(Wgu + Ii * Hh, (int64_t)Ii * Hh, wgu[1], cgu + Ii * Hh);
    const float wd = ora_weight_mean(Wd, (int64_t)Hh * Ii);
    ora_ternarize(Wd, (int64_t)Hh * Ii, wd, cd);
    int8_t *q1 = (int8_t *)malloc((size_t)M * Hh), *q2 = (int8_t *)malloc((size_t)M * Ii);
    float *a1 = (float *)malloc(sizeof(float) * M), *a2 = (float *)malloc(sizeof(float) * M);
    float *p = (float *)malloc(sizeof(float) * M * Ii), *yf = (float *)malloc(sizeof(float) * M * Hh);
    ora_ffn_chain(h, M, Hh, Ii, gs, gf, 1e-5f, cgu, wgu, cd, &wd, q1, a1, p, q2, a2, yf);
    chk += sum_f(yf, (size_t)M * Hh);

    /* attention: H = 4, KVH = 2, D = 8 */
    const int AH = 4, AKV = 2, D = 8, S = 5, maxs = 7;
    double *xr = (double *)malloc(sizeof(double) * AH * D), *yr = (double *)malloc(sizeof(double) * AH * D);
    for (int i = 0; i < AH * D; ++i) xr[i] = unif();
    ora_rope_f64(xr, AH, D, 3, 10000.0, yr);
    float *qa = fbuf((size_t)AH * D, 1.0), *kn = fbuf((size_t)AKV * D, 1.0), *vn = fbuf((size_t)AKV * D, 1.0);
    float *kc = fbuf((size_t)AKV * maxs * D, 1.0), *vc = fbuf((size_t)AKV * maxs * D, 1.0);
    double *ao = (double *)malloc(sizeof(double) * AH * D);
    ora_attn_decode(qa, kn, vn, S - 1, AH, AKV, D, kc, vc, maxs, 10000.0, ao);
    float *qp = fbuf((size_t)S * AH * D, 1.0), *kp = fbuf((size_t)S * AKV * D, 1.0), *vp = fbuf((size_t)S * AKV * D, 1.0);
    const int rows[3] = {0, 2, S - 1};
    double *po = (double *)malloc(sizeof(double) * 3 * AH * D);
    ora_attn_prefill_f64(qp, kp, vp, S, AH, AKV, D, 10000.0, rows, 3, po);
    chk += sum_d(yr, (size_t)AH * D) + sum_d(ao, (size_t)AH * D) + sum_d(po, (size_t)3 * AH * D);

    /* straight-through gradients: dy [M][N] */
    float *dy = fbuf((size_t)M * N, 1.0);
    const int rk[2] = {0, K - 1}, rn[2] = {1, N - 1}, rm[2] = {0, M - 1};
    double *dx = (double *)malloc(sizeof(double) * 2 * K), *dw = (double *)malloc(sizeof(double) * 2 * K);
    ora_ste_grad_input_rows(dy, M, N, codes, K, wm, rm, 2, dx);
    ora_ste_grad_weight_rows(dy, M, N, q, a, K, rn, 2, dw);
    (void)rk;
    chk += sum_d(dx, (size_t)2 * K) + sum_d(dw, (size_t)2 * K);

    /* 1-bit path: N multiple of 8 */
    const int N1 = 16;
    float *W1 = fbuf((size_t)N1 * K, 0.05);
    int8_t *sg = (int8_t *)malloc((size_t)N1 * K), *sg2 = (int8_t *)malloc((size_t)N1 * K);
    ora_binarize(W1, (int64_t)N1 * K, sg);
    uint8_t *pb = (uint8_t *)malloc((size_t)(N1 / 8) * K);
    ora_pack_bits(sg, N1, K, pb);
    ora_unpack_bits(pb, N1, K, sg2);
    float *ln = (float *)malloc(sizeof(float) * M * K);
    float *beta = fbuf(K, 0.1);
    ora_layernorm(x, M, K, g, beta, 1e-5f, ln);
    ora_layernorm(x, M, K, NULL, NULL, 1e-5f, ln);
    int32_t *A1 = (int32_t *)malloc(sizeof(int32_t) * M * N1);
    float *y1 = (float *)malloc(sizeof(float) * M * N1);
    ora_bitlinear_w1(x, M, K, g, beta, 1e-5f, sg, N1, ora_weight_mean(W1, (int64_t)N1 * K), q, a, A1, y1);
    chk += sum_f(ln, (size_t)M * K) + sum_f(y1, (size_t)M * N1) + (memcmp(sg, sg2, (size_t)N1 * K) == 0);

    printf("checksum %.6e\n", chk);
    free(W); free(codes); free(fq); free(packed); free(codes2); free(x); free(q); free(a); free(A); free(y);
    free(yb); free(yd); free(g); free(hn); free(pr); free(h); free(gs); free(gf); free(Wgu); free(Wd); free(cgu);
    free(cd); free(q1); free(q2); free(a1); free(a2); free(p); free(yf); free(xr); free(yr); free(qa); free(kn);
    free(vn); free(kc); free(vc); free(ao); free(qp); free(kp); free(vp); free(po); free(dy); free(dx); free(dw);
    free(W1); free(sg); free(sg2); free(pb); free(ln); free(beta); free(A1); free(y1);
    return isfinite(chk) ? 0 : 1;
}
