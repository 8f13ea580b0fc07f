// bl_api.hip -- the C ABI of libbitlinear (declared in include/bitlinear.h):
// argument checks, workspace layout and kernel dispatch.  Every check runs on
// the host before anything is enqueued; nothing here synchronizes.
//
// Workspace layout of the contraction calls (gemv, gemm, ffn_chain):
//   [0, 64 KiB)              tickets of the split decode kernel (u32), zero
//   [64 KiB, 64 KiB + 8 MiB) int32 accumulators of the split decode kernel, zero
//   [kZeroBytes, ...)        per-call scratch: activation codes and scales,
//                            intermediate chain tensors (overwritten each call)
// The zero prefix sits at the same place for every call, so one workspace
// can serve calls of any shape in sequence; the decode kernel returns every
// word it touches there to zero before the call completes.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "bl_common.h"

namespace {

constexpr size_t kTicketBytes = 64 * 1024;
constexpr int kTicketCap = (int)(kTicketBytes / sizeof(unsigned));
constexpr size_t kAccBytes = 8u * 1024 * 1024;
constexpr size_t kZeroBytes = kTicketBytes + kAccBytes;
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

// Scratch of a contraction call beyond the zero prefix.
struct ContractScratch {
    size_t q_off, a_off, end;
};

ContractScratch contract_scratch(int M, int K) {
    ContractScratch s;
    s.q_off = kZeroBytes;
    s.a_off = s.q_off + align256((size_t)M * K);
    s.end = s.a_off + align256((size_t)M * sizeof(float));
    return s;
}

struct ChainScratch {
    size_t q1, a1, p, q2, a2, end;
};

ChainScratch chain_scratch(int M, int H, int I) {
    ChainScratch s;
    s.q1 = kZeroBytes;
    s.a1 = s.q1 + align256((size_t)M * H);
    s.p = s.a1 + align256((size_t)M * sizeof(float));
    s.q2 = s.p + align256((size_t)M * I * sizeof(float));
    s.a2 = s.q2 + align256((size_t)M * I);
    s.end = s.a2 + align256((size_t)M * sizeof(float));
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

int check_act_dtype(int dt, bool allow_i8, const char *name) {
    if (dt == BL_F32 || dt == BL_BF16 || (allow_i8 && dt == BL_I8)) return BL_OK;
    return fail(BL_ERR_DTYPE, "%s dtype %d not allowed", name, dt);
}

// Shared validation and dispatch of bl_gemv_w2a8 / bl_gemm_w2a8.
int contract_call(bool decode, const void *x, int x_dt, int ldx, const float *a, int M, int K,
                  const uint8_t *packed, int N, int n_seg, const int *seg_n, const float *w_mean,
                  void *y, int y_dt, void *ws, size_t ws_bytes, hipStream_t s) {
    const char *fn = decode ? "bl_gemv_w2a8" : "bl_gemm_w2a8";
    if (!x || !packed || !w_mean || !y || !ws) return fail(BL_ERR_NULL, "%s: NULL pointer argument", fn);
    if (int st = check_act_dtype(x_dt, true, "x")) return st;
    if (x_dt == BL_I8 && !a) return fail(BL_ERR_NULL, "%s: x is int8 codes but a is NULL", fn);
    if (y_dt != BL_F32 && y_dt != BL_BF16 && y_dt != BL_I32)
        return fail(BL_ERR_DTYPE, "%s: y dtype %d not allowed", fn, y_dt);
    if (M < 1 || K < 1 || N < 4) return fail(BL_ERR_SHAPE, "%s: M=%d K=%d N=%d out of range", fn, M, K, N);
    if (decode && M > kMaxGemvM) return fail(BL_ERR_SHAPE, "%s: M=%d exceeds %d", fn, M, kMaxGemvM);
    if (K >= kMaxK) return fail(BL_ERR_SHAPE, "%s: K=%d must be below %d", fn, K, kMaxK);
    if (N % 4 != 0) return fail(BL_ERR_SHAPE, "%s: N=%d is not a multiple of 4", fn, N);
    if (ldx == 0) ldx = K;
    if (ldx < K) return fail(BL_ERR_SHAPE, "%s: ldx=%d < K=%d", fn, ldx, K);
    if (!aligned(x, 16) || !aligned(packed, 16) || !aligned(y, 16) || !aligned(ws, 16) ||
        !aligned(w_mean, 4) || (a && !aligned(a, 4)))
        return fail(BL_ERR_ALIGN, "%s: misaligned pointer", fn);
    bl::SegTab seg;
    if (int st = make_segtab(N, n_seg, seg_n, seg)) return st;
    const ContractScratch sc = contract_scratch(M, K);
    if (ws_bytes < sc.end)
        return fail(BL_ERR_WORKSPACE, "%s: workspace %zu bytes < required %zu", fn, ws_bytes, sc.end);

    char *wsb = (char *)ws;
    bl::Contract c;
    if (x_dt == BL_I8) {
        c.q = (const int8_t *)x;
        c.ldq = ldx;
        c.a = a;
    } else {
        int8_t *q = (int8_t *)(wsb + sc.q_off);
        float *aw = (float *)(wsb + sc.a_off);
        if (int st = check_hip(bl::launch_quant_act(x, x_dt, M, K, ldx, q, aw, s), "quant_act launch"))
            return st;
        c.q = q;
        c.ldq = K;
        c.a = aw;
    }
    c.M = M;
    c.K = K;
    c.P = packed;
    c.seg = seg;
    c.R = N / 4;
    c.w_mean = w_mean;
    c.y = y;
    c.y_dt = y_dt;
    c.ldy = N;
    c.pair = false;
    hipError_t e;
    const bool fast = (K % 16 == 0) && (c.ldq % 16 == 0);
    if (!fast)
        e = bl::launch_generic(c, s);
    else if (decode)
        e = bl::launch_gemv(c, (int32_t *)(wsb + kTicketBytes), kAccBytes, (unsigned *)wsb, kTicketCap, s);
    else
        e = bl::launch_gemm(c, s);
    return check_hip(e, fn);
}

} // namespace

extern "C" {

int bl_abi_version(void) { return BL_ABI_VERSION; }

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

int bl_ternarize_pack(const float *W, int N, int K, uint8_t *packed, float *w_mean, void *ws,
                      size_t ws_bytes, bl_stream stream) {
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
    if (int st = check_act_dtype(x_dtype, false, "x")) return st;
    if (M < 1 || K < 1) return fail(BL_ERR_SHAPE, "bl_quant_act: M=%d K=%d out of range", M, K);
    if (ldx == 0) ldx = K;
    if (ldx < K) return fail(BL_ERR_SHAPE, "bl_quant_act: ldx=%d < K=%d", ldx, K);
    if (!aligned(x, 16) || !aligned(q, 16) || !aligned(a, 4))
        return fail(BL_ERR_ALIGN, "bl_quant_act: misaligned pointer");
    return check_hip(bl::launch_quant_act(x, x_dtype, M, K, ldx, q, a, (hipStream_t)stream), "bl_quant_act");
}

size_t bl_gemv_workspace_bytes(int M, int N, int K) {
    (void)N;
    if (M < 1 || K < 1) return kZeroBytes;
    return contract_scratch(M, K).end;
}

size_t bl_gemm_workspace_bytes(int M, int N, int K) { return bl_gemv_workspace_bytes(M, N, K); }

int bl_gemv_w2a8(const void *x, int x_dtype, int ldx, const float *a, int M, int K, const uint8_t *packed,
                 int N, int n_seg, const int *seg_n, const float *w_mean, void *y, int y_dtype, void *ws,
                 size_t ws_bytes, bl_stream stream) {
    g_err[0] = 0;
    return contract_call(true, x, x_dtype, ldx, a, M, K, packed, N, n_seg, seg_n, w_mean, y, y_dtype, ws,
                         ws_bytes, (hipStream_t)stream);
}

int bl_gemm_w2a8(const void *x, int x_dtype, int ldx, const float *a, int M, int K, const uint8_t *packed,
                 int N, int n_seg, const int *seg_n, const float *w_mean, void *y, int y_dtype, void *ws,
                 size_t ws_bytes, bl_stream stream) {
    g_err[0] = 0;
    return contract_call(false, x, x_dtype, ldx, a, M, K, packed, N, n_seg, seg_n, w_mean, y, y_dtype, ws,
                         ws_bytes, (hipStream_t)stream);
}

size_t bl_ffn_chain_workspace_bytes(int M, int H, int I) {
    if (M < 1 || H < 1 || I < 1) return kZeroBytes;
    return chain_scratch(M, H, I).end;
}

int bl_ffn_chain(const void *h, int h_dtype, int M, int H, int I, const float *g_subln, const float *g_ffn,
                 float eps, const uint8_t *packed_gu, const float *w_mean_gu, const uint8_t *packed_down,
                 const float *w_mean_down, void *y, int y_dtype, void *ws, size_t ws_bytes,
                 const bl_ffn_debug *dbg, bl_stream stream) {
    g_err[0] = 0;
    const char *fn = "bl_ffn_chain";
    if (!h || !packed_gu || !w_mean_gu || !packed_down || !w_mean_down || !y || !ws)
        return fail(BL_ERR_NULL, "%s: NULL pointer argument", fn);
    if (int st = check_act_dtype(h_dtype, false, "h")) return st;
    if (y_dtype != BL_F32 && y_dtype != BL_BF16) return fail(BL_ERR_DTYPE, "%s: y dtype %d not allowed", fn, y_dtype);
    if (M < 1 || H < 4 || I < 4 || H % 4 != 0 || I % 4 != 0)
        return fail(BL_ERR_SHAPE, "%s: M=%d H=%d I=%d (H, I must be positive multiples of 4)", fn, M, H, I);
    if (H >= kMaxK || I >= kMaxK) return fail(BL_ERR_SHAPE, "%s: H or I too large", fn);
    if (!(eps >= 0.0f)) return fail(BL_ERR_SHAPE, "%s: eps must be >= 0", fn);
    if (!aligned(h, 16) || !aligned(packed_gu, 16) || !aligned(packed_down, 16) || !aligned(y, 16) ||
        !aligned(ws, 16) || !aligned(w_mean_gu, 4) || !aligned(w_mean_down, 4) ||
        (g_subln && !aligned(g_subln, 4)) || (g_ffn && !aligned(g_ffn, 4)))
        return fail(BL_ERR_ALIGN, "%s: misaligned pointer", fn);
    if (dbg && ((dbg->q1 && !aligned(dbg->q1, 16)) || (dbg->q2 && !aligned(dbg->q2, 16)) ||
                (dbg->p && !aligned(dbg->p, 16)) || (dbg->a1 && !aligned(dbg->a1, 4)) ||
                (dbg->a2 && !aligned(dbg->a2, 4))))
        return fail(BL_ERR_ALIGN, "%s: misaligned debug pointer", fn);
    const ChainScratch sc = chain_scratch(M, H, I);
    if (ws_bytes < sc.end)
        return fail(BL_ERR_WORKSPACE, "%s: workspace %zu bytes < required %zu", fn, ws_bytes, sc.end);

    hipStream_t s = (hipStream_t)stream;
    char *wsb = (char *)ws;
    int8_t *q1 = dbg && dbg->q1 ? dbg->q1 : (int8_t *)(wsb + sc.q1);
    float *a1 = dbg && dbg->a1 ? dbg->a1 : (float *)(wsb + sc.a1);
    float *p = dbg && dbg->p ? dbg->p : (float *)(wsb + sc.p);
    int8_t *q2 = dbg && dbg->q2 ? dbg->q2 : (int8_t *)(wsb + sc.q2);
    float *a2 = dbg && dbg->a2 ? dbg->a2 : (float *)(wsb + sc.a2);
    int32_t *acc = (int32_t *)(wsb + kTicketBytes);
    unsigned *tickets = (unsigned *)wsb;
    const bool decode = M <= kMaxGemvM;

    // 1. subln RMSNorm + quantize
    if (int st = check_hip(bl::launch_rmsnorm_quant(h, h_dtype, M, H, g_subln, eps, q1, a1, s), "subln launch"))
        return st;
    // 2. gate|up with ReLU^2(gate)*up
    bl::Contract c;
    c.q = q1;
    c.ldq = H;
    c.a = a1;
    c.M = M;
    c.K = H;
    c.P = packed_gu;
    make_segtab(I, 1, nullptr, c.seg);
    c.R = I / 4;
    c.w_mean = w_mean_gu;
    c.y = p;
    c.y_dt = BL_F32;
    c.ldy = I;
    c.pair = true;
    hipError_t e;
    if (H % 16 != 0) e = bl::launch_generic(c, s);
    else if (decode) e = bl::launch_gemv(c, acc, kAccBytes, tickets, kTicketCap, s);
    else e = bl::launch_gemm(c, s);
    if (int st = check_hip(e, "gate|up launch")) return st;
    // 3. ffn_sub_norm RMSNorm + quantize
    if (int st = check_hip(bl::launch_rmsnorm_quant(p, BL_F32, M, I, g_ffn, eps, q2, a2, s), "ffn_sub_norm launch"))
        return st;
    // 4. down
    c.q = q2;
    c.ldq = I;
    c.a = a2;
    c.K = I;
    c.P = packed_down;
    make_segtab(H, 1, nullptr, c.seg);
    c.R = H / 4;
    c.w_mean = w_mean_down;
    c.y = y;
    c.y_dt = y_dtype;
    c.ldy = H;
    c.pair = false;
    if (I % 16 != 0) e = bl::launch_generic(c, s);
    else if (decode) e = bl::launch_gemv(c, acc, kAccBytes, tickets, kTicketCap, s);
    else e = bl::launch_gemm(c, s);
    return check_hip(e, "down launch");
}

} // extern "C"
