// bl_api.hip -- the C ABI of libbitlinear (declared in include/bitlinear.h):
// argument checks, workspace layout and kernel dispatch.  Every check runs on
// the host before anything is enqueued; nothing here synchronizes.
//
// Dispatch of the contraction:
//   decode (bl_gemv_w2a8*, M <= 64): the batched decode kernel; activations
//     quantized in its prologue when M <= 4 and the rows fit in LDS, else by
//     the row kernel into the workspace first;
//   prefill (bl_gemm_w2a8): the row kernel, then the MFMA GEMM;
//   any K that is not a multiple of 16: the plain kernel.
// The workspace only holds per-call scratch (activation codes and scales,
// intermediate chain tensors); nothing in it survives a call.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "bl_attn.h"
#include "bl_common.h"
#include "bl_ste.h"

namespace {

constexpr int kMaxK = 1 << 19;
constexpr int kMaxGemvM = 64;

thread_local char g_err[512] = "";

int fail(int st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

int check_hip(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(BL_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return BL_OK;
}

size_t quant_scratch(int M, int K) { return align256((size_t)M * K) + align256((size_t)M * sizeof(float)); }

// Decode calls that quantize outside the contraction kernel: codes (token
// rows padded to a multiple of 16 for the tiled layout of the batched
// kernel), scales, then the rows' code sums.
size_t decode_codes(int M, int K) { return align256((size_t)((M + 15) / 16 * 16) * K); }
size_t decode_quant_scratch(int M, int K) {
    return decode_codes(M, K) + align256((size_t)M * sizeof(float)) + align256((size_t)M * sizeof(int));
}

bool fusable(int M, int K) {
    return M <= bl::kFuseMaxM && (size_t)M * K <= (size_t)bl::kFuseMaxBytes && K % 16 == 0;
}

struct ChainScratch {
    size_t q1, a1, p, q2, a2, qs, end;
};

ChainScratch chain_scratch(int M, int H, int I) {
    ChainScratch s;
    s.q1 = 0;
    s.a1 = s.q1 + align256((size_t)M * H);
    s.p = s.a1 + align256((size_t)M * sizeof(float));
    s.q2 = s.p + align256((size_t)M * I * sizeof(float));
    s.a2 = s.q2 + align256((size_t)M * I);
    s.qs = s.a2 + align256((size_t)M * sizeof(float));   // code sums, reused by both contractions
    s.end = s.qs + align256((size_t)M * sizeof(int));
    return s;
}

// Builds the segment table; returns BL_OK or an error status.
int make_segtab(int N, int n_seg, const int *seg_n, bl::SegTab &t) {
    if (n_seg < 1 || n_seg > BL_MAX_SEGMENTS)
        return fail(BL_ERR_SEGMENTS, "n_seg=%d must be in [1,%d]", n_seg, BL_MAX_SEGMENTS);
    if (n_seg > 1 && !seg_n) return fail(BL_ERR_SEGMENTS, "seg_n is NULL with n_seg=%d", n_seg);
    t.n = n_seg;
    int sum = 0;
    t.roff[0] = 0;
    for (int s = 0; s < n_seg; ++s) {
        const int w = seg_n ? seg_n[s] : N;
        if (w < 4 || w % 4 != 0)
            return fail(BL_ERR_SEGMENTS, "segment %d width %d is not a positive multiple of 4", s, w);
        sum += w;
        if (sum > N) break;
        t.roff[s + 1] = sum / 4;
    }
    if (sum != N) return fail(BL_ERR_SEGMENTS, "segment widths sum to %d, N=%d", sum, N);
    for (int s = n_seg + 1; s <= BL_MAX_SEGMENTS; ++s) t.roff[s] = t.roff[n_seg];
    return BL_OK;
}

// Validated view of one contraction call.
struct Call {
    const void *x;
    int x_dt, ldx;
    const float *a;
    int M, K;
    const uint8_t *packed;
    int N;
    bl::SegTab seg;
    const float *w_mean;
    void *y;
    int y_dt;
};

int validate(const char *fn, bool decode, const bl_gemv_problem &pr, Call &c) {
    if (!pr.x || !pr.packed || !pr.w_mean || !pr.y) return fail(BL_ERR_NULL, "%s: NULL pointer argument", fn);
    if (pr.x_dtype != BL_F32 && pr.x_dtype != BL_BF16 && pr.x_dtype != BL_I8)
        return fail(BL_ERR_DTYPE, "%s: x dtype %d not allowed", fn, pr.x_dtype);
    if (pr.x_dtype == BL_I8 && !pr.a) return fail(BL_ERR_NULL, "%s: x is int8 codes but a is NULL", fn);
    if (pr.y_dtype != BL_F32 && pr.y_dtype != BL_BF16 && pr.y_dtype != BL_I32)
        return fail(BL_ERR_DTYPE, "%s: y dtype %d not allowed", fn, pr.y_dtype);
    if (pr.M < 1 || pr.K < 1 || pr.N < 4)
        return fail(BL_ERR_SHAPE, "%s: M=%d K=%d N=%d out of range", fn, pr.M, pr.K, pr.N);
    if (decode && pr.M > kMaxGemvM) return fail(BL_ERR_SHAPE, "%s: M=%d exceeds %d", fn, pr.M, kMaxGemvM);
    if (pr.K >= kMaxK) return fail(BL_ERR_SHAPE, "%s: K=%d must be below %d", fn, pr.K, kMaxK);
    if (pr.N % 4 != 0) return fail(BL_ERR_SHAPE, "%s: N=%d is not a multiple of 4", fn, pr.N);
    const int ldx = pr.ldx == 0 ? pr.K : pr.ldx;
    if (ldx < pr.K) return fail(BL_ERR_SHAPE, "%s: ldx=%d < K=%d", fn, ldx, pr.K);
    if (!aligned(pr.x, 16) || !aligned(pr.packed, 16) || !aligned(pr.y, 16) || !aligned(pr.w_mean, 4) ||
        (pr.a && !aligned(pr.a, 4)))
        return fail(BL_ERR_ALIGN, "%s: misaligned pointer", fn);
    if (int st = make_segtab(pr.N, pr.n_seg, pr.seg_n, c.seg)) return st;
    c.x = pr.x;
    c.x_dt = pr.x_dtype;
    c.ldx = ldx;
    c.a = pr.a;
    c.M = pr.M;
    c.K = pr.K;
    c.packed = pr.packed;
    c.N = pr.N;
    c.w_mean = pr.w_mean;
    c.y = pr.y;
    c.y_dt = pr.y_dtype;
    return BL_OK;
}

bool is_fast(const Call &c) { return c.K % 16 == 0; }

// Decode calls are quantized inside the contraction kernel (fused prologue)
// when every fast call of the launch has raw activations that fit;
// otherwise the raw ones are quantized by one batched row-kernel launch into
// the workspace.  Calls with K % 16 != 0 use the plain kernel.
bool decode_all_fused(int n, const Call *calls) {
    bool any = false;
    for (int i = 0; i < n; ++i) {
        if (!is_fast(calls[i])) continue;
        if (calls[i].x_dt == BL_I8 || !fusable(calls[i].M, calls[i].K)) return false;
        any = true;
    }
    return any;
}

size_t decode_scratch(int n, const Call *calls) {
    const bool fused = decode_all_fused(n, calls);
    size_t need = 0;
    for (int i = 0; i < n; ++i) {
        const Call &c = calls[i];
        if (c.x_dt == BL_I8) continue;
        if (is_fast(c) && fused) continue;
        need += decode_quant_scratch(c.M, c.K);
    }
    return need;
}

// Prefill scratch: the codes and scales when x is not int8, then the rows'
// code sums (M ints) that the large-tile GEMM reads.
size_t prefill_scratch(const Call &c) {
    return (c.x_dt == BL_I8 ? 0 : quant_scratch(c.M, c.K)) + align256((size_t)c.M * sizeof(int));
}

bl::Contract contract_of(const Call &c, const int8_t *q, int ldq, const float *a) {
    bl::Contract k;
    k.q = q;
    k.ldq = ldq;
    k.a = a;
    k.M = c.M;
    k.K = c.K;
    k.P = c.packed;
    k.seg = c.seg;
    k.R = c.N / 4;
    k.w_mean = c.w_mean;
    k.y = c.y;
    k.y_dt = c.y_dt;
    k.ldy = c.N;
    k.pair = false;
    return k;
}

bl::GemvProblem gemv_of(const Call &c, int mode, const void *x, int ldx, const float *a) {
    bl::GemvProblem p;
    memset(&p, 0, sizeof(p));
    p.x = x;
    p.a = a;
    p.P = c.packed;
    p.w_mean = c.w_mean;
    p.y = c.y;
    p.seg = c.seg;
    p.x_dt = c.x_dt;
    p.ldx = ldx;
    p.M = c.M;
    p.K = c.K;
    p.R = c.N / 4;
    p.y_dt = c.y_dt;
    p.ldy = c.N;
    p.mode = mode;
    return p;
}

// Enqueues a set of validated decode calls (n <= kMaxProblems).
int run_decode(const char *fn, int n, const Call *calls, char *ws, hipStream_t s) {
    const bool fused = decode_all_fused(n, calls);
    bl::GemvBatch b;
    b.n = 0;
    bl::QuantBatch qb;
    qb.n = 0;
    size_t off = 0;
    // codes / scales of every call that is not quantized in a fused prologue
    const int8_t *qv[BL_MAX_PROBLEMS];
    const float *av[BL_MAX_PROBLEMS];
    const int *sv[BL_MAX_PROBLEMS];
    int ldq[BL_MAX_PROBLEMS];
    // The batched streaming kernel takes every call when all are quantized
    // here and fit it; its codes are written tiled (code_offset).
    bool mt = !fused;
    int Ms[BL_MAX_PROBLEMS], Ks[BL_MAX_PROBLEMS];
    for (int i = 0; i < n; ++i) {
        const Call &c = calls[i];
        mt = mt && c.x_dt != BL_I8 && is_fast(c) && aligned(c.packed, 16);
        Ms[i] = c.M;
        Ks[i] = c.K;
    }
    mt = mt && bl::gemv_mt_plan_ok(n, Ms, Ks);
    for (int i = 0; i < n; ++i) {
        const Call &c = calls[i];
        qv[i] = (const int8_t *)c.x;
        av[i] = c.a;
        sv[i] = nullptr;
        ldq[i] = c.ldx;
        if (c.x_dt != BL_I8 && !(is_fast(c) && fused)) {
            int8_t *qw = (int8_t *)(ws + off);
            float *aw = (float *)(ws + off + decode_codes(c.M, c.K));
            int *sw = (int *)(ws + off + decode_codes(c.M, c.K) + align256((size_t)c.M * sizeof(float)));
            off += decode_quant_scratch(c.M, c.K);
            bl::QuantProblem &qp = qb.p[qb.n++];
            qp = bl::QuantProblem{};
            qp.x = c.x; qp.q = qw; qp.a = aw; qp.qsum = sw; qp.x_dt = c.x_dt; qp.M = c.M; qp.K = c.K; qp.ldx = c.ldx;
            qp.tile_m = mt ? (c.M + 15) / 16 * 16 : 0;
            qv[i] = qw;
            av[i] = aw;
            sv[i] = sw;
            ldq[i] = c.K;
        }
    }
    if (qb.n > 0)
        if (int st = check_hip(bl::launch_quant_batch(qb, s), fn)) return st;
    for (int i = 0; i < n; ++i) {
        const Call &c = calls[i];
        if (!is_fast(c) || ldq[i] % 16 != 0) {
            if (int st = check_hip(bl::launch_generic(contract_of(c, qv[i], ldq[i], av[i]), s), fn)) return st;
        } else if (fused) {
            b.p[b.n++] = gemv_of(c, 1, c.x, c.ldx, nullptr);
        } else {
            bl::GemvProblem p = gemv_of(c, 0, qv[i], ldq[i], av[i]);
            p.x_dt = BL_I8;
            p.qsum = sv[i];
            p.qtile = mt ? (c.M + 15) / 16 * 16 : 0;
            b.p[b.n++] = p;
        }
    }
    if (b.n == 0) return BL_OK;
    return check_hip(bl::launch_gemv_batch(b, s), fn);
}

int check_ws(const char *fn, const void *ws, size_t ws_bytes, size_t need) {
    if (need == 0) return BL_OK;
    if (!ws) return fail(BL_ERR_WORKSPACE, "%s: workspace of %zu bytes required, got NULL", fn, need);
    if (!aligned(ws, 16)) return fail(BL_ERR_ALIGN, "%s: misaligned workspace", fn);
    if (ws_bytes < need) return fail(BL_ERR_WORKSPACE, "%s: workspace %zu bytes < required %zu", fn, ws_bytes, need);
    return BL_OK;
}

bl_gemv_problem as_problem(const void *x, int x_dtype, int ldx, const float *a, int M, int K, const uint8_t *packed,
                           int N, int n_seg, const int *seg_n, const float *w_mean, void *y, int y_dtype) {
    bl_gemv_problem p;
    p.x = x;
    p.x_dtype = x_dtype;
    p.ldx = ldx;
    p.a = a;
    p.M = M;
    p.K = K;
    p.packed = packed;
    p.N = N;
    p.n_seg = n_seg;
    p.seg_n = seg_n;
    p.w_mean = w_mean;
    p.y = y;
    p.y_dtype = y_dtype;
    return p;
}

} // namespace

extern "C" {

int bl_abi_version(void) { return BL_ABI_VERSION; }

int bl_device_errors(unsigned int *expired_waits, int reset) {
    g_err[0] = 0;
    if (!expired_waits) return fail(BL_ERR_NULL, "bl_device_errors: NULL pointer argument");
    if (hipError_t e = hipDeviceSynchronize(); e != hipSuccess) return check_hip(e, "bl_device_errors");
    unsigned int a = 0, b = 0, c = 0;
    if (int st = check_hip(bl::gemv_wait_expired(&a, reset != 0), "bl_device_errors")) return st;
    if (int st = check_hip(bl::chain_wait_expired(&b, reset != 0), "bl_device_errors")) return st;
    if (int st = check_hip(bl::w1_wait_expired(&c, reset != 0), "bl_device_errors")) return st;
    *expired_waits = a + b + c;
    return BL_OK;
}

const char *bl_status_string(int status) {
    switch (status) {
    case BL_OK: return "BL_OK";
    case BL_ERR_NULL: return "BL_ERR_NULL";
    case BL_ERR_SHAPE: return "BL_ERR_SHAPE";
    case BL_ERR_ALIGN: return "BL_ERR_ALIGN";
    case BL_ERR_DTYPE: return "BL_ERR_DTYPE";
    case BL_ERR_SEGMENTS: return "BL_ERR_SEGMENTS";
    case BL_ERR_WORKSPACE: return "BL_ERR_WORKSPACE";
    case BL_ERR_HIP: return "BL_ERR_HIP";
    default: return "BL_ERR_UNKNOWN";
    }
}

const char *bl_last_error(void) { return g_err; }

size_t bl_ternarize_workspace_bytes(int64_t N, int64_t K) {
    if (N < 1 || K < 1) return 256;
    return align256((size_t)bl::absmean_parts(N * K) * sizeof(double));
}

int bl_ternarize_pack(const float *W, int N, int K, uint8_t *packed, float *w_mean, void *ws, size_t ws_bytes,
                      bl_stream stream) {
    g_err[0] = 0;
    if (!W || !packed || !w_mean || !ws) return fail(BL_ERR_NULL, "bl_ternarize_pack: NULL pointer argument");
    if (N < 4 || K < 1 || N % 4 != 0)
        return fail(BL_ERR_SHAPE, "bl_ternarize_pack: N=%d must be a positive multiple of 4, K=%d >= 1", N, K);
    if ((int64_t)N * K >= ((int64_t)1 << 40)) return fail(BL_ERR_SHAPE, "bl_ternarize_pack: N*K too large");
    if (!aligned(W, 16) || !aligned(packed, 16) || !aligned(ws, 16) || !aligned(w_mean, 4))
        return fail(BL_ERR_ALIGN, "bl_ternarize_pack: misaligned pointer");
    const size_t need = bl_ternarize_workspace_bytes(N, K);
    if (ws_bytes < need)
        return fail(BL_ERR_WORKSPACE, "bl_ternarize_pack: workspace %zu bytes < required %zu", ws_bytes, need);
    hipStream_t s = (hipStream_t)stream;
    const int64_t count = (int64_t)N * K;
    if (int st = check_hip(bl::launch_absmean(W, count, (double *)ws, bl::absmean_parts(count), w_mean, s),
                           "bl_ternarize_pack absmean"))
        return st;
    return check_hip(bl::launch_ternarize_pack(W, N, K, w_mean, packed, s), "bl_ternarize_pack pack");
}

int bl_quant_act(const void *x, int x_dtype, int M, int K, int ldx, int8_t *q, float *a, bl_stream stream) {
    g_err[0] = 0;
    if (!x || !q || !a) return fail(BL_ERR_NULL, "bl_quant_act: NULL pointer argument");
    if (x_dtype != BL_F32 && x_dtype != BL_BF16) return fail(BL_ERR_DTYPE, "bl_quant_act: x dtype %d not allowed", x_dtype);
    if (M < 1 || K < 1) return fail(BL_ERR_SHAPE, "bl_quant_act: M=%d K=%d out of range", M, K);
    if (ldx == 0) ldx = K;
    if (ldx < K) return fail(BL_ERR_SHAPE, "bl_quant_act: ldx=%d < K=%d", ldx, K);
    if (!aligned(x, 16) || !aligned(q, 16) || !aligned(a, 4))
        return fail(BL_ERR_ALIGN, "bl_quant_act: misaligned pointer");
    return check_hip(bl::launch_quant_act(x, x_dtype, M, K, ldx, q, a, nullptr, (hipStream_t)stream), "bl_quant_act");
}

int bl_rmsnorm_quant(const void *h, int h_dtype, int M, int K, const float *gain, float eps, int8_t *q, float *a,
                     bl_stream stream) {
    g_err[0] = 0;
    const char *fn = "bl_rmsnorm_quant";
    if (!h || !q || !a) return fail(BL_ERR_NULL, "%s: NULL pointer argument", fn);
    if (h_dtype != BL_F32 && h_dtype != BL_BF16) return fail(BL_ERR_DTYPE, "%s: h dtype %d not allowed", fn, h_dtype);
    if (M < 1 || K < 1) return fail(BL_ERR_SHAPE, "%s: M=%d K=%d out of range", fn, M, K);
    if (!(eps >= 0.0f) || !isfinite(eps)) return fail(BL_ERR_SHAPE, "%s: eps=%g", fn, (double)eps);
    if (!aligned(h, 16) || !aligned(q, 16) || !aligned(a, 4) || (gain && !aligned(gain, 4)))
        return fail(BL_ERR_ALIGN, "%s: misaligned pointer", fn);
    return check_hip(bl::launch_rmsnorm_quant(h, h_dtype, M, K, gain, eps, q, a, nullptr, (hipStream_t)stream), fn);
}

size_t bl_gemv_workspace_bytes(int M, int N, int K) {
    (void)N;
    if (M < 1 || K < 1) return 0;
    return decode_quant_scratch(M, K);
}

size_t bl_gemm_workspace_bytes(int M, int N, int K) {
    (void)N;
    if (M < 1 || K < 1) return 0;
    return quant_scratch(M, K) + align256((size_t)M * sizeof(int));
}

int bl_gemv_w2a8(const void *x, int x_dtype, int ldx, const float *a, int M, int K, const uint8_t *packed, int N,
                 int n_seg, const int *seg_n, const float *w_mean, void *y, int y_dtype, void *ws, size_t ws_bytes,
                 bl_stream stream) {
    g_err[0] = 0;
    const char *fn = "bl_gemv_w2a8";
    const bl_gemv_problem pr = as_problem(x, x_dtype, ldx, a, M, K, packed, N, n_seg, seg_n, w_mean, y, y_dtype);
    Call c;
    if (int st = validate(fn, true, pr, c)) return st;
    if (int st = check_ws(fn, ws, ws_bytes, decode_scratch(1, &c))) return st;
    return run_decode(fn, 1, &c, (char *)ws, (hipStream_t)stream);
}

size_t bl_gemv_batched_workspace_bytes(int n, const bl_gemv_problem *problems) {
    size_t need = 0;
    if (!problems || n < 1) return 0;
    for (int i = 0; i < n && i < BL_MAX_PROBLEMS; ++i)
        if (problems[i].M > 0 && problems[i].K > 0) need += decode_quant_scratch(problems[i].M, problems[i].K);
    return need;
}

int bl_gemv_w2a8_batched(int n, const bl_gemv_problem *problems, void *ws, size_t ws_bytes, bl_stream stream) {
    g_err[0] = 0;
    const char *fn = "bl_gemv_w2a8_batched";
    if (!problems) return fail(BL_ERR_NULL, "%s: problems is NULL", fn);
    if (n < 1 || n > BL_MAX_PROBLEMS) return fail(BL_ERR_SHAPE, "%s: n=%d must be in [1,%d]", fn, n, BL_MAX_PROBLEMS);
    Call calls[BL_MAX_PROBLEMS];
    for (int i = 0; i < n; ++i)
        if (int st = validate(fn, true, problems[i], calls[i])) return st;
    if (int st = check_ws(fn, ws, ws_bytes, decode_scratch(n, calls))) return st;
    return run_decode(fn, n, calls, (char *)ws, (hipStream_t)stream);
}

int bl_gemm_w2a8(const void *x, int x_dtype, int ldx, const float *a, int M, int K, const uint8_t *packed, int N,
                 int n_seg, const int *seg_n, const float *w_mean, void *y, int y_dtype, void *ws, size_t ws_bytes,
                 bl_stream stream) {
    g_err[0] = 0;
    const char *fn = "bl_gemm_w2a8";
    const bl_gemv_problem pr = as_problem(x, x_dtype, ldx, a, M, K, packed, N, n_seg, seg_n, w_mean, y, y_dtype);
    Call c;
    if (int st = validate(fn, false, pr, c)) return st;
    if (int st = check_ws(fn, ws, ws_bytes, prefill_scratch(c))) return st;
    hipStream_t s = (hipStream_t)stream;
    const int8_t *q = (const int8_t *)c.x;
    int ldq = c.ldx;
    const float *aq = c.a;
    int *qsum = (int *)((char *)ws + (c.x_dt == BL_I8 ? 0 : quant_scratch(c.M, c.K)));
    const bool fast = is_fast(c);
    if (c.x_dt != BL_I8) {
        int8_t *qw = (int8_t *)ws;
        float *aw = (float *)((char *)ws + align256((size_t)c.M * c.K));
        if (int st = check_hip(bl::launch_quant_act(c.x, c.x_dt, c.M, c.K, c.ldx, qw, aw, fast ? qsum : nullptr, s), fn))
            return st;
        q = qw;
        ldq = c.K;
        aq = aw;
    }
    bl::Contract k = contract_of(c, q, ldq, aq);
    if (fast && ldq % 16 == 0) {
        // codes quantized here come with their row sums
        if (c.x_dt != BL_I8) k.qsum = qsum;
        return check_hip(bl::launch_gemm(k, qsum, s), fn);
    }
    return check_hip(bl::launch_generic(k, s), fn);
}

size_t bl_subln_gemv_workspace_bytes(int M, int K) {
    if (M < 1 || K < 1) return 0;
    return quant_scratch(M, K) + align256((size_t)M * sizeof(int));
}

int bl_subln_gemv_w2a8(const void *h, int h_dtype, int M, int K, const float *gain, float eps, const uint8_t *packed,
                       int N, const float *w_mean, void *y, int y_dtype, int8_t *q_out, float *a_out, void *ws,
                       size_t ws_bytes, bl_stream stream) {
    g_err[0] = 0;
    const char *fn = "bl_subln_gemv_w2a8";
    if (h_dtype != BL_F32 && h_dtype != BL_BF16) return fail(BL_ERR_DTYPE, "%s: h dtype %d not allowed", fn, h_dtype);
    const bl_gemv_problem pr = as_problem(h, h_dtype, 0, nullptr, M, K, packed, N, 1, nullptr, w_mean, y, y_dtype);
    Call c;
    if (int st = validate(fn, false, pr, c)) return st;
    if (!(eps >= 0.0f) || !isfinite(eps)) return fail(BL_ERR_SHAPE, "%s: eps=%g", fn, (double)eps);
    if ((gain && !aligned(gain, 4)) || (q_out && !aligned(q_out, 16)) || (a_out && !aligned(a_out, 4)))
        return fail(BL_ERR_ALIGN, "%s: misaligned pointer", fn);
    if (int st = check_ws(fn, ws, ws_bytes, bl_subln_gemv_workspace_bytes(M, K))) return st;
    hipStream_t s = (hipStream_t)stream;
    const bool decode = M <= kMaxGemvM;
    const bool fast = is_fast(c);
    if (decode && fast && fusable(M, K)) {
        // one launch: the decode kernel normalizes and quantizes its rows in
        // the prologue (codes and scales also to q_out / a_out when given)
        bl::GemvBatch b;
        memset(&b, 0, sizeof(b));
        b.n = 1;
        b.p[0] = gemv_of(c, 2, h, K, nullptr);
        b.p[0].gain = gain;
        b.p[0].eps = eps;
        b.p[0].dbg_q = q_out;
        b.p[0].dbg_a = a_out;
        return check_hip(bl::launch_gemv_batch(b, s), fn);
    }
    char *wsb = (char *)ws;
    int8_t *q = q_out ? q_out : (int8_t *)wsb;
    float *a = a_out ? a_out : (float *)(wsb + align256((size_t)M * K));
    int *qsum = (int *)(wsb + quant_scratch(M, K));
    if (int st = check_hip(
            bl::launch_rmsnorm_quant(h, h_dtype, M, K, gain, eps, q, a, !decode && fast ? qsum : nullptr, s), fn))
        return st;
    Call ci = c;
    ci.x = q;
    ci.x_dt = BL_I8;
    ci.ldx = K;
    ci.a = a;
    if (decode) return run_decode(fn, 1, &ci, wsb, s);
    bl::Contract k = contract_of(ci, q, K, a);
    if (fast) {
        k.qsum = qsum;
        return check_hip(bl::launch_gemm(k, qsum, s), fn);
    }
    return check_hip(bl::launch_generic(k, s), fn);
}

} // extern "C"

// ---------------------------------------------------------------------------
// The allocation-free variant of bl_ffn_chain: its scratch is this
// file-scope device array (one copy per device, held until the process
// ends).  Host code never passes the array's name to a kernel: it passes the
// device address hipGetSymbolAddress returns for the current device, taken
// once per device and kept.
// ---------------------------------------------------------------------------
namespace {

constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
constexpr int kMaxDevices = 64;

} // namespace

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch array (BL_OK), looked up on the
// device's first call.
int scratch_address(const char *fn, void **out) {
    int dev = 0;
    if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) return check_hip(e, fn);
    if (dev < 0 || dev >= kMaxDevices) return fail(BL_ERR_HIP, "%s: device %d beyond the library's %d", fn, dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)); e != hipSuccess) {
            (void)hipGetLastError();
            return check_hip(e, fn);
        }
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return BL_OK;
}

} // namespace

extern "C" {

size_t bl_ffn_chain_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

int bl_ffn_chain_noalloc(const void *h, int h_dtype, int M, int H, int I, const float *g_subln, const float *g_ffn,
                         float eps, const uint8_t *packed_gu, const float *w_mean_gu, const uint8_t *packed_down,
                         const float *w_mean_down, void *y, int y_dtype, const bl_ffn_debug *dbg, bl_stream stream) {
    g_err[0] = 0;
    const char *fn = "bl_ffn_chain_noalloc";
    if (M < 1 || H < 4 || I < 4 || H % 4 != 0 || I % 4 != 0)
        return fail(BL_ERR_SHAPE, "%s: M=%d H=%d I=%d (H, I must be positive multiples of 4)", fn, M, H, I);
    const size_t need = bl_ffn_chain_workspace_bytes(M, H, I);
    if (need > kNoAllocScratchBytes)
        return fail(BL_ERR_WORKSPACE, "%s: M=%d H=%d I=%d needs %zu bytes of scratch, beyond the fixed %zu", fn, M, H,
                    I, need, kNoAllocScratchBytes);
    void *ws = nullptr;
    if (int st = scratch_address(fn, &ws)) return st;
    return bl_ffn_chain(h, h_dtype, M, H, I, g_subln, g_ffn, eps, packed_gu, w_mean_gu, packed_down, w_mean_down, y,
                        y_dtype, ws, kNoAllocScratchBytes, dbg, stream);
}

size_t bl_ffn_chain_workspace_bytes(int M, int H, int I) {
    if (M < 1 || H < 1 || I < 1) return 0;
    return chain_scratch(M, H, I).end;
}

int bl_ffn_chain(const void *h, int h_dtype, int M, int H, int I, const float *g_subln, const float *g_ffn, float eps,
                 const uint8_t *packed_gu, const float *w_mean_gu, const uint8_t *packed_down,
                 const float *w_mean_down, void *y, int y_dtype, void *ws, size_t ws_bytes, const bl_ffn_debug *dbg,
                 bl_stream stream) {
    g_err[0] = 0;
    const char *fn = "bl_ffn_chain";
    if (!h || !packed_gu || !w_mean_gu || !packed_down || !w_mean_down || !y)
        return fail(BL_ERR_NULL, "%s: NULL pointer argument", fn);
    if (h_dtype != BL_F32 && h_dtype != BL_BF16) return fail(BL_ERR_DTYPE, "%s: h dtype %d not allowed", fn, h_dtype);
    if (y_dtype != BL_F32 && y_dtype != BL_BF16) return fail(BL_ERR_DTYPE, "%s: y dtype %d not allowed", fn, y_dtype);
    if (M < 1 || H < 4 || I < 4 || H % 4 != 0 || I % 4 != 0)
        return fail(BL_ERR_SHAPE, "%s: M=%d H=%d I=%d (H, I must be positive multiples of 4)", fn, M, H, I);
    if (H >= kMaxK || I >= kMaxK) return fail(BL_ERR_SHAPE, "%s: H or I too large", fn);
    if (!(eps >= 0.0f)) return fail(BL_ERR_SHAPE, "%s: eps must be >= 0", fn);
    if (!aligned(h, 16) || !aligned(packed_gu, 16) || !aligned(packed_down, 16) || !aligned(y, 16) ||
        !aligned(w_mean_gu, 4) || !aligned(w_mean_down, 4) || (g_subln && !aligned(g_subln, 4)) ||
        (g_ffn && !aligned(g_ffn, 4)))
        return fail(BL_ERR_ALIGN, "%s: misaligned pointer", fn);
    if (dbg && ((dbg->q1 && !aligned(dbg->q1, 16)) || (dbg->q2 && !aligned(dbg->q2, 16)) ||
                (dbg->p && !aligned(dbg->p, 16)) || (dbg->a1 && !aligned(dbg->a1, 4)) ||
                (dbg->a2 && !aligned(dbg->a2, 4))))
        return fail(BL_ERR_ALIGN, "%s: misaligned debug pointer", fn);
    const ChainScratch sc = chain_scratch(M, H, I);
    if (int st = check_ws(fn, ws, ws_bytes, sc.end)) return st;

    hipStream_t s = (hipStream_t)stream;
    char *wsb = (char *)ws;
    int8_t *q1 = dbg && dbg->q1 ? dbg->q1 : (int8_t *)(wsb + sc.q1);
    float *a1 = dbg && dbg->a1 ? dbg->a1 : (float *)(wsb + sc.a1);
    float *p = dbg && dbg->p ? dbg->p : (float *)(wsb + sc.p);
    int8_t *q2 = dbg && dbg->q2 ? dbg->q2 : (int8_t *)(wsb + sc.q2);
    float *a2 = dbg && dbg->a2 ? dbg->a2 : (float *)(wsb + sc.a2);
    const bool decode = M <= kMaxGemvM;
    const bool fuse = decode && fusable(M, H) && fusable(M, I);

    bl::SegTab seg_i, seg_h;
    make_segtab(I, 1, nullptr, seg_i);
    make_segtab(H, 1, nullptr, seg_h);

    if (fuse) {
        // Two launches: each decode kernel normalizes and quantizes its own
        // input rows in the prologue (stage codes go to the debug buffers).
        bl::GemvBatch b;
        memset(&b, 0, sizeof(b));
        b.n = 1;
        bl::GemvProblem &g = b.p[0];
        g.x = h; g.x_dt = h_dtype; g.ldx = H; g.gain = g_subln; g.eps = eps; g.mode = 2;
        g.M = M; g.K = H; g.R = I / 4; g.P = packed_gu; g.seg = seg_i; g.w_mean = w_mean_gu;
        g.y = p; g.y_dt = BL_F32; g.ldy = I; g.pair = 1;
        g.dbg_q = dbg ? dbg->q1 : nullptr; g.dbg_a = dbg ? dbg->a1 : nullptr;
        if (int st = check_hip(bl::launch_gemv_batch(b, s), "gate|up launch")) return st;
        memset(&b, 0, sizeof(b));
        b.n = 1;
        bl::GemvProblem &d = b.p[0];
        d.x = p; d.x_dt = BL_F32; d.ldx = I; d.gain = g_ffn; d.eps = eps; d.mode = 2;
        d.M = M; d.K = I; d.R = H / 4; d.P = packed_down; d.seg = seg_h; d.w_mean = w_mean_down;
        d.y = y; d.y_dt = y_dtype; d.ldy = H; d.pair = 0;
        d.dbg_q = dbg ? dbg->q2 : nullptr; d.dbg_a = dbg ? dbg->a2 : nullptr;
        return check_hip(bl::launch_gemv_batch(b, s), "down launch");
    }

    // 1. subln RMSNorm + quantize
    int *qs = (int *)(wsb + sc.qs);
    if (int st = check_hip(bl::launch_rmsnorm_quant(h, h_dtype, M, H, g_subln, eps, q1, a1, decode ? nullptr : qs, s),
                           "subln launch"))
        return st;
    // 2. gate|up with ReLU^2(gate)*up
    bl::Contract c;
    c.q = q1; c.ldq = H; c.a = a1; c.M = M; c.K = H; c.P = packed_gu; c.seg = seg_i; c.R = I / 4;
    c.w_mean = w_mean_gu; c.y = p; c.y_dt = BL_F32; c.ldy = I; c.pair = true;
    hipError_t e;
    if (H % 16 != 0) {
        e = bl::launch_generic(c, s);
    } else if (decode) {
        bl::GemvBatch b;
        memset(&b, 0, sizeof(b));
        b.n = 1;
        bl::GemvProblem &g = b.p[0];
        g.x = q1; g.x_dt = BL_I8; g.ldx = H; g.a = a1; g.mode = 0; g.M = M; g.K = H; g.R = I / 4;
        g.P = packed_gu; g.seg = seg_i; g.w_mean = w_mean_gu; g.y = p; g.y_dt = BL_F32; g.ldy = I; g.pair = 1;
        e = bl::launch_gemv_batch(b, s);
    } else {
        c.qsum = qs;
        e = bl::launch_gemm(c, qs, s);
    }
    if (int st = check_hip(e, "gate|up launch")) return st;
    // 3. ffn_sub_norm RMSNorm + quantize
    if (int st = check_hip(bl::launch_rmsnorm_quant(p, BL_F32, M, I, g_ffn, eps, q2, a2, decode ? nullptr : qs, s),
                           "ffn_sub_norm launch"))
        return st;
    // 4. down
    c.q = q2; c.ldq = I; c.a = a2; c.K = I; c.P = packed_down; c.seg = seg_h; c.R = H / 4;
    c.w_mean = w_mean_down; c.y = y; c.y_dt = y_dtype; c.ldy = H; c.pair = false;
    if (I % 16 != 0) {
        e = bl::launch_generic(c, s);
    } else if (decode) {
        bl::GemvBatch b;
        memset(&b, 0, sizeof(b));
        b.n = 1;
        bl::GemvProblem &d = b.p[0];
        d.x = q2; d.x_dt = BL_I8; d.ldx = I; d.a = a2; d.mode = 0; d.M = M; d.K = I; d.R = H / 4;
        d.P = packed_down; d.seg = seg_h; d.w_mean = w_mean_down; d.y = y; d.y_dt = y_dtype; d.ldy = H; d.pair = 0;
        e = bl::launch_gemv_batch(b, s);
    } else {
        c.qsum = qs;
        e = bl::launch_gemm(c, qs, s);
    }
    return check_hip(e, "down launch");
}

int bl_rope_table(int max_pos, int head_dim, double base, float *cos_out, float *sin_out) {
    g_err[0] = 0;
    const char *fn = "bl_rope_table";
    if (!cos_out || !sin_out) return fail(BL_ERR_NULL, "%s: output array is NULL", fn);
    if (max_pos < 1 || head_dim < 2 || head_dim % 2 != 0 || !(base > 0.0))
        return fail(BL_ERR_SHAPE, "%s: max_pos=%d head_dim=%d base=%g", fn, max_pos, head_dim, base);
    const int h2 = head_dim / 2;
    for (int p = 0; p < max_pos; ++p)
        for (int i = 0; i < h2; ++i) {
            const double ang = (double)p * pow(base, -2.0 * (double)i / (double)head_dim);
            cos_out[(size_t)p * h2 + i] = (float)cos(ang);
            sin_out[(size_t)p * h2 + i] = (float)sin(ang);
        }
    return BL_OK;
}

size_t bl_attn_decode_workspace_bytes(int n_heads, int max_seq) {
    if (n_heads < 1 || max_seq < 1) return 0;
    return align256(bl::attn_decode_workspace_bytes(n_heads, max_seq));
}

int bl_attn_decode(const float *q, const float *k_new, const float *v_new, int pos, int n_heads, int n_kv_heads,
                   int head_dim, float *k_cache, float *v_cache, int max_seq, const float *rope_cos,
                   const float *rope_sin, float *out, void *ws, size_t ws_bytes, bl_stream stream) {
    g_err[0] = 0;
    const char *fn = "bl_attn_decode";
    if (!q || !k_new || !v_new || !k_cache || !v_cache || !rope_cos || !rope_sin || !out)
        return fail(BL_ERR_NULL, "%s: a device pointer is NULL", fn);
    if (head_dim != 128) return fail(BL_ERR_SHAPE, "%s: head_dim=%d (only 128 is supported)", fn, head_dim);
    if (n_heads < 1 || n_kv_heads < 1 || n_heads % n_kv_heads != 0 || n_heads / n_kv_heads > 4)
        return fail(BL_ERR_SHAPE, "%s: n_heads=%d n_kv_heads=%d (a multiple, at most 4 per key/value head)", fn,
                    n_heads, n_kv_heads);
    if (max_seq < 1 || max_seq > bl::attn_decode_max_seq() || pos < 0 || pos >= max_seq)
        return fail(BL_ERR_SHAPE, "%s: pos=%d max_seq=%d (max_seq at most %d)", fn, pos, max_seq,
                    bl::attn_decode_max_seq());
    const void *ptrs[] = {q, k_new, v_new, k_cache, v_cache, rope_cos, rope_sin, out};
    for (const void *p : ptrs)
        if (!aligned(p, 16)) return fail(BL_ERR_ALIGN, "%s: misaligned device pointer", fn);
    if (int st = check_ws(fn, ws, ws_bytes, bl_attn_decode_workspace_bytes(n_heads, max_seq))) return st;
    return check_hip(bl::launch_attn_decode(q, k_new, v_new, pos, n_heads, n_kv_heads, k_cache, v_cache, max_seq,
                                            rope_cos, rope_sin, out, ws, (hipStream_t)stream),
                     fn);
}

size_t bl_attn_prefill_workspace_bytes(int M, int n_heads, int n_kv_heads) {
    if (M < 1 || n_heads < 1 || n_kv_heads < 1) return 0;
    return align256(bl::attn_prefill_workspace_bytes(M, n_heads, n_kv_heads));
}

int bl_attn_prefill(const float *q, const float *k, const float *v, int ldx, int M, int n_heads, int n_kv_heads,
                    int head_dim, float *k_cache, float *v_cache, int max_seq, const float *rope_cos,
                    const float *rope_sin, float *out, int ldo, void *ws, size_t ws_bytes, bl_stream stream) {
    g_err[0] = 0;
    const char *fn = "bl_attn_prefill";
    if (!q || !k || !v || !k_cache || !v_cache || !rope_cos || !rope_sin || !out)
        return fail(BL_ERR_NULL, "%s: a device pointer is NULL", fn);
    if (head_dim != 128) return fail(BL_ERR_SHAPE, "%s: head_dim=%d (only 128 is supported)", fn, head_dim);
    if (n_heads < 1 || n_kv_heads < 1 || n_heads % n_kv_heads != 0)
        return fail(BL_ERR_SHAPE, "%s: n_heads=%d n_kv_heads=%d (n_heads a multiple of n_kv_heads)", fn, n_heads,
                    n_kv_heads);
    if (M < 1 || M > max_seq) return fail(BL_ERR_SHAPE, "%s: M=%d max_seq=%d", fn, M, max_seq);
    if (ldx < 128 * n_heads || ldo < 128 * n_heads || ldo % 4 != 0)
        return fail(BL_ERR_SHAPE, "%s: ldx=%d ldo=%d (at least n_heads*128; ldo a multiple of 4)", fn, ldx, ldo);
    const void *p4[] = {q, k, v, k_cache, v_cache, rope_cos, rope_sin};
    for (const void *p : p4)
        if (!aligned(p, 4)) return fail(BL_ERR_ALIGN, "%s: misaligned device pointer", fn);
    if (!aligned(out, 16)) return fail(BL_ERR_ALIGN, "%s: out must be 16-byte aligned", fn);
    if (int st = check_ws(fn, ws, ws_bytes, bl_attn_prefill_workspace_bytes(M, n_heads, n_kv_heads))) return st;
    return check_hip(bl::launch_attn_prefill(q, k, v, ldx, M, n_heads, n_kv_heads, k_cache, v_cache, max_seq,
                                             rope_cos, rope_sin, out, ldo, ws, (hipStream_t)stream),
                     fn);
}

size_t bl_stack_decode_workspace_bytes(int n_layers, int H, int KV, int I) {
    if (n_layers < 1 || H < 1 || KV < 0 || I < 1) return 0;
    return align256((size_t)n_layers * ((size_t)(H + 2 * KV) + H + I + H) * sizeof(float));
}

int bl_stack_decode(const void *x, int x_dtype, int n_layers, const bl_layer *layers, int H, int KV, int I, float eps,
                    float *y, float *stages, void *ws, size_t ws_bytes, bl_stream stream) {
    g_err[0] = 0;
    const char *fn = "bl_stack_decode";
    if (!x || !layers || !y) return fail(BL_ERR_NULL, "%s: NULL pointer argument", fn);
    if (x_dtype != BL_F32 && x_dtype != BL_BF16) return fail(BL_ERR_DTYPE, "%s: x dtype %d not allowed", fn, x_dtype);
    if (n_layers < 1 || n_layers > bl::chain_max_layers())
        return fail(BL_ERR_SHAPE, "%s: n_layers=%d (1..%d per call)", fn, n_layers, bl::chain_max_layers());
    if (!(eps >= 0.0f)) return fail(BL_ERR_SHAPE, "%s: eps must be >= 0", fn);
    const int G = bl::chain_workgroups();
    if (G < 1) return fail(BL_ERR_SHAPE, "%s: the kernel does not fit one workgroup per compute unit here", fn);
    if (!bl::chain_fits(H, KV, I, G))
        return fail(BL_ERR_SHAPE, "%s: H=%d KV=%d I=%d outside the persistent kernel's capacity (H, I multiples of "
                                  "256 up to 8192, KV of 16, the units per workgroup bounded)", fn, H, KV, I);
    for (int l = 0; l < n_layers; ++l) {
        const bl_layer &w = layers[l];
        if (!w.packed_qkv || !w.w_qkv || !w.packed_o || !w.w_o || !w.packed_gu || !w.w_gu || !w.packed_down ||
            !w.w_down)
            return fail(BL_ERR_NULL, "%s: layer %d has a NULL weight pointer", fn, l);
        if (!aligned(w.packed_qkv, 16) || !aligned(w.packed_o, 16) || !aligned(w.packed_gu, 16) ||
            !aligned(w.packed_down, 16) || !aligned(w.w_qkv, 4) || !aligned(w.w_o, 4) || !aligned(w.w_gu, 4) ||
            !aligned(w.w_down, 4) || (w.g_subln && !aligned(w.g_subln, 4)) || (w.g_ffn && !aligned(w.g_ffn, 4)))
            return fail(BL_ERR_ALIGN, "%s: layer %d has a misaligned pointer", fn, l);
    }
    if (!aligned(x, x_dtype == BL_F32 ? 4 : 2) || !aligned(y, 4) || (stages && !aligned(stages, 4)))
        return fail(BL_ERR_ALIGN, "%s: misaligned pointer", fn);
    if (int e = check_ws(fn, ws, ws_bytes, bl_stack_decode_workspace_bytes(n_layers, H, KV, I))) return e;

    bl::ChainLayerPtrs lp[32];
    for (int l = 0; l < n_layers; ++l) {
        const bl_layer &w = layers[l];
        lp[l] = bl::ChainLayerPtrs{w.packed_qkv, w.w_qkv, w.packed_o, w.w_o, w.packed_gu, w.w_gu, w.packed_down,
                                   w.w_down, w.g_subln, w.g_ffn};
    }
    bl::ChainParams p{};
    p.x = x; p.x_dt = x_dtype; p.L = n_layers; p.H = H; p.KV = KV; p.I = I; p.eps = eps;
    p.xch = (float *)ws; p.stages = stages; p.y = y;
    p.G = G; p.layers = lp;
    const int segs[3] = {H, KV, KV};
    if (int e = make_segtab(H + 2 * KV, 3, segs, p.seg_qkv)) return e;
    return check_hip(bl::launch_chain_decode(p, (hipStream_t)stream), fn);
}

int bl_unpack_bf16(const uint8_t *packed, int N, int K, int n_seg, const int *seg_n, void *w_codes,
                   bl_stream stream) {
    g_err[0] = 0;
    const char *fn = "bl_unpack_bf16";
    if (!packed || !w_codes) return fail(BL_ERR_NULL, "%s: NULL pointer argument", fn);
    if (N < 4 || N % 4 != 0 || K < 1) return fail(BL_ERR_SHAPE, "%s: N=%d K=%d (N a positive multiple of 4)", fn, N, K);
    if ((size_t)N * K >= ((size_t)1 << 40)) return fail(BL_ERR_SHAPE, "%s: N*K too large", fn);
    bl::SegTab seg;
    if (int st = make_segtab(N, n_seg, seg_n, seg)) return st;
    if (!aligned(w_codes, 2)) return fail(BL_ERR_ALIGN, "%s: w_codes must be 2-byte aligned", fn);
    return check_hip(bl::launch_unpack_bf16(packed, N, K, seg, w_codes, (hipStream_t)stream), fn);
}

size_t bl_gemm_unpacked_workspace_bytes(int M, int N, int K) {
    if (M < 1 || N < 1 || K < 1) return 0;
    (void)N;
    return quant_scratch(M, K) + align256(bl::unpacked_gemm_ws_bytes(M, K));
}

int bl_gemm_unpacked(const void *x, int x_dtype, int ldx, const float *a, int M, int K, const void *w_codes, int N,
                     int n_seg, const int *seg_n, const float *w_mean, void *y, int y_dtype, void *ws,
                     size_t ws_bytes, bl_stream stream) {
    g_err[0] = 0;
    const char *fn = "bl_gemm_unpacked";
    if (!x || !w_codes || !w_mean || !y) return fail(BL_ERR_NULL, "%s: NULL pointer argument", fn);
    if (x_dtype != BL_F32 && x_dtype != BL_BF16 && x_dtype != BL_I8)
        return fail(BL_ERR_DTYPE, "%s: x dtype %d not allowed", fn, x_dtype);
    if (y_dtype != BL_F32 && y_dtype != BL_BF16 && y_dtype != BL_I32)
        return fail(BL_ERR_DTYPE, "%s: y dtype %d not allowed", fn, y_dtype);
    if (x_dtype == BL_I8 && !a) return fail(BL_ERR_NULL, "%s: a is required with int8 codes", fn);
    if (M < 1 || K < 1 || N < 4 || N % 4 != 0)
        return fail(BL_ERR_SHAPE, "%s: M=%d K=%d N=%d (N a positive multiple of 4)", fn, M, K, N);
    if (ldx == 0) ldx = K;
    if (ldx < K) return fail(BL_ERR_SHAPE, "%s: ldx=%d < K=%d", fn, ldx, K);
    if (x_dtype == BL_I8 && ldx != K) return fail(BL_ERR_SHAPE, "%s: int8 codes must be contiguous rows", fn);
    const bool gemv = M <= 4 && bl::unpacked_gemv_fits(K);
    const bool gemm = bl::unpacked_gemm_fits(M, N, K);
    if (!gemv && !gemm && !bl::unpacked_gemv_fits(K))
        return fail(BL_ERR_SHAPE, "%s: M=%d N=%d K=%d: needs K a multiple of 8 up to 8192, or K a multiple of 64 "
                                  "and N of 128", fn, M, N, K);
    bl::SegTab seg;
    if (int st = make_segtab(N, n_seg, seg_n, seg)) return st;
    if (!aligned(x, x_dtype == BL_F32 ? 4 : (x_dtype == BL_BF16 ? 2 : 4)) || !aligned(w_codes, 16) ||
        !aligned(y, 16) || !aligned(w_mean, 4) || (a && !aligned(a, 4)))
        return fail(BL_ERR_ALIGN, "%s: misaligned pointer", fn);
    if (int st = check_ws(fn, ws, ws_bytes, bl_gemm_unpacked_workspace_bytes(M, N, K))) return st;
    hipStream_t s = (hipStream_t)stream;
    char *wsb = (char *)ws;
    const int8_t *q = (const int8_t *)x;
    const float *av = a;
    if (x_dtype != BL_I8) {
        int8_t *qw = (int8_t *)wsb;
        float *aw = (float *)(wsb + align256((size_t)M * K));
        if (int st = check_hip(bl::launch_quant_act(x, x_dtype, M, K, ldx, qw, aw, nullptr, s), fn)) return st;
        q = qw;
        av = aw;
    }
    bl::GemmEpi e{};
    e.a = av;
    e.w_mean = w_mean;
    e.nseg = seg.n;
    for (int i = 0; i < BL_MAX_SEGMENTS; ++i) e.cend[i] = 4 * seg.roff[i < seg.n ? i + 1 : seg.n];
    e.y_dt = y_dtype;
    if (gemv || !gemm) return check_hip(bl::launch_unpacked_gemv(q, av, M, K, w_codes, N, e, y, s), fn);
    return check_hip(bl::launch_unpacked_gemm(q, av, M, K, (const __bf16 *)w_codes, N, e, y, wsb + quant_scratch(M, K),
                                              s),
                     fn);
}

size_t bl_ste_grad_input_workspace_bytes(int M, int N, int K, int dy_dtype) {
    if (M < 1 || N < 1 || K < 1 || (dy_dtype != BL_BF16 && dy_dtype != BL_F32)) return 0;
    return align256(bl::ste_grad_input_ws_bytes(M, N, K, dy_dtype == BL_BF16));
}

size_t bl_ste_grad_weight_workspace_bytes(int M, int N, int K) {
    if (M < 1 || N < 1 || K < 1) return 0;
    return align256(bl::ste_grad_weight_ws_bytes(M, N, K));
}

static int ste_shape(const char *fn, int M, int N, int K, int dy_dtype) {
    if (M < 1 || N < 1 || K < 1) return fail(BL_ERR_SHAPE, "%s: M=%d N=%d K=%d (each >= 1)", fn, M, N, K);
    if (!bl::ste_dims_fit(M, N, K))
        return fail(BL_ERR_SHAPE, "%s: M=%d N=%d K=%d (each product of two, padded to 128, below 2^31)", fn, M, N,
                    K);
    if (dy_dtype != BL_BF16 && dy_dtype != BL_F32) return fail(BL_ERR_DTYPE, "%s: dy_dtype must be BF16 or F32", fn);
    return BL_OK;
}

int bl_ste_grad_input(const void *dy, int dy_dtype, int M, int N, int K, const uint8_t *packed, const float *w_mean,
                      void *dx, int dx_dtype, void *ws, size_t ws_bytes, bl_stream stream) {
    g_err[0] = 0;
    const char *fn = "bl_ste_grad_input";
    if (!dy || !packed || !w_mean || !dx) return fail(BL_ERR_NULL, "%s: NULL pointer argument", fn);
    if (int st = ste_shape(fn, M, N, K, dy_dtype)) return st;
    if (N % 4) return fail(BL_ERR_SHAPE, "%s: N=%d is not a multiple of 4", fn, N);
    if (dx_dtype != BL_F32 && dx_dtype != BL_BF16) return fail(BL_ERR_DTYPE, "%s: dx_dtype %d", fn, dx_dtype);
    if (!aligned(dy, 16) || !aligned(dx, dx_dtype == BL_BF16 ? 8 : 16) || !aligned(w_mean, 4))
        return fail(BL_ERR_ALIGN, "%s: misaligned pointer", fn);
    if (int st = check_ws(fn, ws, ws_bytes, bl_ste_grad_input_workspace_bytes(M, N, K, dy_dtype))) return st;
    return check_hip(bl::launch_ste_grad_input(dy, dy_dtype == BL_BF16, M, N, K, packed, w_mean, dx,
                                               dx_dtype == BL_BF16, ws, (hipStream_t)stream),
                     fn);
}

int bl_ste_grad_weight(const void *dy, int dy_dtype, const int8_t *q, const float *a, int M, int N, int K, float *dw,
                       void *ws, size_t ws_bytes, bl_stream stream) {
    g_err[0] = 0;
    const char *fn = "bl_ste_grad_weight";
    if (!dy || !q || !a || !dw) return fail(BL_ERR_NULL, "%s: NULL pointer argument", fn);
    if (int st = ste_shape(fn, M, N, K, dy_dtype)) return st;
    if (!aligned(dy, dy_dtype == BL_BF16 ? 2 : 4) || !aligned(dw, 16) || !aligned(a, 4))
        return fail(BL_ERR_ALIGN, "%s: misaligned pointer", fn);
    if (int st = check_ws(fn, ws, ws_bytes, bl_ste_grad_weight_workspace_bytes(M, N, K))) return st;
    return check_hip(bl::launch_ste_grad_weight(dy, dy_dtype == BL_BF16, M, N, K, q, a, dw, ws, (hipStream_t)stream),
                     fn);
}

// ---------------------------------------------------------------------------
// The 1-bit BitLinear.
// ---------------------------------------------------------------------------
size_t bl_binarize_workspace_bytes(int64_t N, int64_t K) { return bl_ternarize_workspace_bytes(N, K); }

int bl_binarize_pack(const float *W, int N, int K, uint8_t *packed, float *w_scale, void *ws, size_t ws_bytes,
                     bl_stream stream) {
    g_err[0] = 0;
    const char *fn = "bl_binarize_pack";
    if (!W || !packed || !w_scale || !ws) return fail(BL_ERR_NULL, "%s: NULL pointer argument", fn);
    if (N < 8 || N % 8 != 0 || K < 4 || K % 4 != 0)
        return fail(BL_ERR_SHAPE, "%s: N=%d (a positive multiple of 8), K=%d (a positive multiple of 4)", fn, N, K);
    if ((int64_t)N * K >= ((int64_t)1 << 40)) return fail(BL_ERR_SHAPE, "%s: N*K too large", fn);
    if (!aligned(W, 16) || !aligned(packed, 16) || !aligned(ws, 16) || !aligned(w_scale, 4))
        return fail(BL_ERR_ALIGN, "%s: misaligned pointer", fn);
    if (int e = check_ws(fn, ws, ws_bytes, bl_binarize_workspace_bytes(N, K))) return e;
    hipStream_t s = (hipStream_t)stream;
    const int64_t count = (int64_t)N * K;
    if (int st = check_hip(bl::launch_absmean(W, count, (double *)ws, bl::absmean_parts(count), w_scale, s), fn))
        return st;
    return check_hip(bl::launch_binarize_pack(W, N, K, packed, s), fn);
}

// Shape and pointer checks of one 1-bit problem; `norm`: x is read (else q).
static int w1_check(const char *fn, int i, const void *x, int x_dtype, int M, int K, int ldx, const float *gamma,
                    const float *beta, const uint8_t *packed, int N, const float *w_scale, const float *y,
                    bool norm, bool gemm) {
    if (M < 1 || K < 4 || K % 4 != 0) return fail(BL_ERR_SHAPE, "%s: problem %d: M=%d K=%d", fn, i, M, K);
    if (norm) {
        if (!x) return fail(BL_ERR_NULL, "%s: problem %d: NULL x", fn, i);
        if (x_dtype != BL_F32 && x_dtype != BL_BF16)
            return fail(BL_ERR_DTYPE, "%s: problem %d: x dtype %d not allowed", fn, i, x_dtype);
        if (K > bl::w1_ln_max_k()) return fail(BL_ERR_SHAPE, "%s: problem %d: K=%d above %d", fn, i, K, bl::w1_ln_max_k());
        if (ldx < K || ldx % 4 != 0) return fail(BL_ERR_SHAPE, "%s: problem %d: ldx=%d", fn, i, ldx);
        if (!aligned(x, 16) || (gamma && !aligned(gamma, 16)) || (beta && !aligned(beta, 16)))
            return fail(BL_ERR_ALIGN, "%s: problem %d: misaligned x, gamma or beta", fn, i);
    }
    if (gemm) {
        if (!packed || !w_scale || !y) return fail(BL_ERR_NULL, "%s: problem %d: NULL pointer", fn, i);
        if (K % 16 != 0 || K < 16 || K > 16384 || N < 8 || N % 8 != 0)
            return fail(BL_ERR_SHAPE, "%s: problem %d: K=%d (16..16384, a multiple of 16), N=%d (a multiple of 8)",
                        fn, i, K, N);
        if ((int64_t)M * N >= ((int64_t)1 << 40)) return fail(BL_ERR_SHAPE, "%s: problem %d: M*N too large", fn, i);
        if (!aligned(packed, 16) || !aligned(w_scale, 4) || !aligned(y, 4))
            return fail(BL_ERR_ALIGN, "%s: problem %d: misaligned packed, w_scale or y", fn, i);
    }
    return 0;
}

int bl_layernorm_quant(const void *x, int x_dtype, int M, int K, int ldx, const float *gamma, const float *beta,
                       float eps, int8_t *q, float *a, bl_stream stream) {
    g_err[0] = 0;
    const char *fn = "bl_layernorm_quant";
    if (!q || !a) return fail(BL_ERR_NULL, "%s: NULL pointer argument", fn);
    if (ldx == 0) ldx = K;
    if (int e = w1_check(fn, 0, x, x_dtype, M, K, ldx, gamma, beta, nullptr, 0, nullptr, nullptr, true, false))
        return e;
    if (!(eps >= 0.0f) || !isfinite(eps)) return fail(BL_ERR_SHAPE, "%s: eps=%g", fn, (double)eps);
    if (!aligned(q, 16) || !aligned(a, 4)) return fail(BL_ERR_ALIGN, "%s: misaligned q or a", fn);
    bl::W1Args w{x, x_dtype, ldx, gamma, beta, M, K, q, a, nullptr, 0, nullptr, nullptr};
    return check_hip(bl::launch_w1_norm(&w, 1, eps, (hipStream_t)stream), fn);
}

int bl_gemm_w1a8(const int8_t *q, const float *a, int M, int K, const uint8_t *packed, int N, const float *w_scale,
                 float *y, bl_stream stream) {
    g_err[0] = 0;
    const char *fn = "bl_gemm_w1a8";
    if (!q || !a) return fail(BL_ERR_NULL, "%s: NULL pointer argument", fn);
    if (int e = w1_check(fn, 0, nullptr, 0, M, K, K, nullptr, nullptr, packed, N, w_scale, y, false, true)) return e;
    if (!aligned(q, 16) || !aligned(a, 4)) return fail(BL_ERR_ALIGN, "%s: misaligned q or a", fn);
    bl::W1Args w{nullptr, 0, K, nullptr, nullptr, M, K, const_cast<int8_t *>(q), const_cast<float *>(a), packed, N,
                 w_scale, y};
    return check_hip(bl::launch_w1_gemm(&w, 1, (hipStream_t)stream), fn);
}

// Workspace of bl_bitlinear_w1: per problem the codes (M*K bytes) and the
// scales (M floats), each 256-byte aligned.
static size_t w1_ws_layout(const bl_w1_problem *probs, int n, size_t *q_off, size_t *a_off) {
    size_t off = 0;
    for (int i = 0; i < n; ++i) {
        const size_t M = probs[i].M > 0 ? (size_t)probs[i].M : 0, K = probs[i].K > 0 ? (size_t)probs[i].K : 0;
        if (q_off) q_off[i] = off;
        off += align256(M * K);
        if (a_off) a_off[i] = off;
        off += align256(M * sizeof(float));
    }
    return off;
}

size_t bl_bitlinear_w1_workspace_bytes(const bl_w1_problem *probs, int n) {
    if (!probs || n < 1 || n > bl::kMaxProblems) return 0;
    return w1_ws_layout(probs, n, nullptr, nullptr);
}

int bl_bitlinear_w1(const bl_w1_problem *probs, int n, float eps, void *ws, size_t ws_bytes, bl_stream stream) {
    g_err[0] = 0;
    const char *fn = "bl_bitlinear_w1";
    if (!probs) return fail(BL_ERR_NULL, "%s: NULL problem table", fn);
    if (n < 1 || n > bl::kMaxProblems) return fail(BL_ERR_SHAPE, "%s: n=%d (1..%d)", fn, n, bl::kMaxProblems);
    if (!(eps >= 0.0f) || !isfinite(eps)) return fail(BL_ERR_SHAPE, "%s: eps=%g", fn, (double)eps);
    for (int i = 0; i < n; ++i) {
        const bl_w1_problem &p = probs[i];
        if (int e = w1_check(fn, i, p.x, p.x_dtype, p.M, p.K, p.K, p.gamma, p.beta, p.packed, p.N, p.w_scale, p.y,
                             true, true))
            return e;
    }
    if (int e = check_ws(fn, ws, ws_bytes, bl_bitlinear_w1_workspace_bytes(probs, n))) return e;
    size_t q_off[bl::kMaxProblems], a_off[bl::kMaxProblems];
    w1_ws_layout(probs, n, q_off, a_off);
    bl::W1Args w[bl::kMaxProblems];
    for (int i = 0; i < n; ++i) {
        const bl_w1_problem &p = probs[i];
        w[i] = bl::W1Args{p.x, p.x_dtype, p.K, p.gamma, p.beta, p.M, p.K, (int8_t *)((char *)ws + q_off[i]),
                          (float *)((char *)ws + a_off[i]), p.packed, p.N, p.w_scale, p.y};
    }
    hipStream_t s = (hipStream_t)stream;
    if (bl::w1_decode_fits(w, n)) return check_hip(bl::launch_w1_decode(w, n, eps, s), fn);
    if (int e = check_hip(bl::launch_w1_norm(w, n, eps, s), fn)) return e;
    return check_hip(bl::launch_w1_gemm(w, n, s), fn);
}

} // extern "C"
