/*
 * bitlinear.h -- C ABI of libbitlinear: the BitNet b1.58 BitLinear forward
 * (1.58-bit ternary weights, 8-bit activations) on AMD Instinct MI355X
 * (gfx950), hand-written HIP kernels.
 *
 * Sources (page title, then the section on it):
 *  [Q] "BitNet", Transformers quantization guide (Portuguese edition):
 *      numbered list of the three quantization steps; "Kernels".
 *  [T] "Transformers 实战 BitNet 1.58 位量化：BitLinear 原理、量化流程与推理加载全指南":
 *      "BitLinear 的三步量化" (steps 1-3); "推理侧 BitLinear：打包权重、解包与缩放"
 *      (pack, unpack and the inference forward) and the subln paragraph after it.
 *  [M] "BitNet" model documentation (Chinese and Portuguese editions):
 *      "模型详情" / "Detalhes do Modelo" (W1.58A8, ReLU squared, subln, no
 *      bias) and "BitNetConfig" (rms_norm_eps 1e-5, layer shapes).
 *  [S] project summary of a PyTorch "BitNet" implementation of 1-bit
 *      Transformers: "How It Works" (the 1-bit BitLinear: layer
 *      normalization, binarization, absolute-maximum quantization).
 *
 * Numerics (what every call computes, bit for bit):
 *  - weight scale  w_mean = max(float(sum|W| / count), 1e-5), sum in fp64;
 *  - weight code   c = clip(round_half_even(W / w_mean), -1, 1), fp32 division;
 *  - packed weight P[r,k] = sum_i (c[i*N/4 + r, k] + 1) << 2i  (plane order);
 *  - act scale     a_m = 127 / max(max_k |x[m,k]|, 1e-5), fp32 division;
 *  - act code      q = clip(round_half_even(x * a_m), -128, 127), fp32 multiply;
 *  - accumulator   A[m,n] = sum_k q[m,k] * c[n,k]  (exact int32);
 *  - output        y = float(A) * (w_mean_s / a_m), fp32; bf16 = RNE(y);
 *  - RMSNorm       r = float(1/sqrt(sum h^2 / K + eps)) (fp64), out = (h*r)*g.
 *
 * Conventions shared by every call
 *  - Pointers are DEVICE pointers unless marked (host).  The caller owns
 *    every buffer; the library keeps no device memory between calls.
 *  - Row-major, contiguous.  Device buffers must be 16-byte aligned.
 *  - Every call only enqueues work on `stream` (a hipStream_t; NULL is the
 *    null stream) and returns without synchronizing.
 *  - Argument checks run on the host before anything is enqueued.  A failed
 *    check returns a non-zero bl_status, stores a message retrievable with
 *    bl_last_error() (per host thread) and enqueues nothing.  After
 *    launching, a launch error returns BL_ERR_HIP.  Faults inside kernels
 *    surface at the caller's next synchronization.  No C++ exception ever
 *    crosses this interface.
 *  - Inputs must be finite (NaN/Inf are outside the contract).
 *  - Segments: a weight may be several tensors, each ternarized with its own
 *    scale and packed on its own, concatenated along the packed rows (fused
 *    q|k|v, gate|up).  seg_n (host) lists their output widths, each a
 *    multiple of 4, summing to N; w_mean (device) holds one scale per
 *    segment.  n_seg = 1 with seg_n = NULL means one tensor.  At most
 *    BL_MAX_SEGMENTS segments.
 *  - Workspace (ws): device scratch of at least the queried size (the query
 *    is an upper bound; a call that needs none accepts NULL).  Contents are
 *    per call and never read across calls; calls that share a workspace must
 *    not run concurrently.
 */
#ifndef BITLINEAR_H
#define BITLINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BL_ABI_VERSION 2
#define BL_MAX_SEGMENTS 8
#define BL_MAX_PROBLEMS 8

typedef enum {
    BL_OK = 0,
    BL_ERR_NULL = 1,      /* a required pointer is NULL                          */
    BL_ERR_SHAPE = 2,     /* a size is out of range or not a multiple it must be */
    BL_ERR_ALIGN = 3,     /* a device pointer is not 16-byte aligned             */
    BL_ERR_DTYPE = 4,     /* a dtype code is not allowed for that argument       */
    BL_ERR_SEGMENTS = 5,  /* bad segment count or widths                         */
    BL_ERR_WORKSPACE = 6, /* workspace missing or smaller than required          */
    BL_ERR_HIP = 7        /* the HIP runtime reported an error at launch         */
} bl_status;

typedef enum { BL_F32 = 0, BL_BF16 = 1, BL_I8 = 2, BL_I32 = 3 } bl_dtype;

typedef void *bl_stream; /* hipStream_t */

/* Version of this interface (BL_ABI_VERSION). */
int bl_abi_version(void);
/* Static name of a status code; never NULL. */
const char *bl_status_string(int status);
/* Message of the last failed call on this host thread ("" if none). */
const char *bl_last_error(void);

/* ---------------------------------------------------------------------------
 * bl_device_errors -- faults the kernels detect themselves.  The decode
 * kernels' waves wait on each other through flags with a bounded number of
 * polls; a wait that runs out (only a wave held off its compute unit for
 * about 0.2 s could cause it) lets the kernel finish normally and counts
 * itself on the device, and the outputs of that call are then unreliable.
 * This call synchronizes the current device, stores in *expired_waits (host)
 * the number of expired waits since the last reset, and clears the count when
 * reset is non-zero.  Returns BL_OK, BL_ERR_NULL or BL_ERR_HIP.
 * ------------------------------------------------------------------------ */
int bl_device_errors(unsigned int *expired_waits, int reset);

/* ---------------------------------------------------------------------------
 * bl_ternarize_pack -- absmean ternarization and 2-bit packing of one weight
 * tensor.  [Q] steps 1-2; [T] "BitLinear 的三步量化" steps 1-2 (scale = mean
 * |W| over the whole tensor, floored at 1e-5; codes = W / scale rounded and
 * clipped to [-1,1]) and "推理侧 BitLinear" (codes + 1 stored 2 bits each,
 * four per byte, a quarter of the rows; field i under mask 3 << 2i).
 *   W       [N,K] fp32 master weight.
 *   packed  out [N/4,K] uint8; packed row r, bits 2i..2i+1 hold code+1 of
 *           weight row i*N/4 + r (plane order).
 *   w_mean  out, one fp32.
 *   ws      scratch of bl_ternarize_workspace_bytes(N,K) bytes (no zero
 *           requirement).
 * N >= 4, N % 4 == 0, K >= 1, N*K < 2^40.  Deterministic: the fp64 sum runs
 * in a fixed order for a given (N, K).
 * ------------------------------------------------------------------------ */
size_t bl_ternarize_workspace_bytes(int64_t N, int64_t K);
int bl_ternarize_pack(const float *W, int N, int K, uint8_t *packed, float *w_mean,
                      void *ws, size_t ws_bytes, bl_stream stream);

/* ---------------------------------------------------------------------------
 * bl_quant_act -- per-token absmax int8 activation quantization.  [Q] step 3;
 * [T] "BitLinear 的三步量化" step 3; [M] "模型详情" (per token).
 *   x       [M,K] (row stride ldx elements; ldx = 0 means K), dtype BL_F32 or
 *           BL_BF16.
 *   q       out [M,K] int8, contiguous.
 *   a       out [M] fp32 scales a_m = 127 / max(absmax, 1e-5).
 * M >= 1, K >= 1.
 * ------------------------------------------------------------------------ */
int bl_quant_act(const void *x, int x_dtype, int M, int K, int ldx,
                 int8_t *q, float *a, bl_stream stream);

/* ---------------------------------------------------------------------------
 * bl_rmsnorm_quant -- RMSNorm of each row, then bl_quant_act's per-token
 * int8 quantization: the sub-norm in front of a projection (attn_sub_norm
 * before o_proj, ffn_sub_norm before down_proj).  [M] "模型详情" (subln
 * normalization) and "BitNetConfig" (rms_norm_eps); [T] the subln
 * paragraph; the quantization as in bl_quant_act.
 *   h       [M,K] contiguous, dtype BL_F32 or BL_BF16.
 *   gain    [K] fp32 RMSNorm weight, or NULL for all ones.
 *   eps     >= 0 (the model uses 1e-5).
 *   q, a    out: codes [M,K] int8 and scales [M] fp32 of
 *           r = fp32(h * (1/sqrt(sum(h^2)/K + eps))) * gain, the sum in fp64.
 * M >= 1, K >= 1.
 * ------------------------------------------------------------------------ */
int bl_rmsnorm_quant(const void *h, int h_dtype, int M, int K, const float *gain, float eps,
                     int8_t *q, float *a, bl_stream stream);

/* ---------------------------------------------------------------------------
 * bl_gemv_w2a8 / bl_gemm_w2a8 -- the BitLinear contraction with rescale.
 * [T] "推理侧 BitLinear" forward bullet: quantize the activations, multiply
 * with the unpacked ternary weight, rescale by the activation and weight
 * scales.  bl_gemv_w2a8 is the decode path (1 <= M <= 64, weights streamed
 * from HBM once); bl_gemm_w2a8 is the prefill path (any M >= 1, int8 MFMA
 * tiles).  Both compute the same bits.
 *   x       [M,K], row stride ldx elements (0 = K).  x_dtype BL_F32/BL_BF16:
 *           quantized inside the call (bl_quant_act's arithmetic).  BL_I8:
 *           already quantized codes, with their scales in `a`.
 *   a       [M] fp32 activation scales, read when x_dtype == BL_I8, else
 *           ignored (may be NULL).
 *   packed  [N/4,K] uint8 packed weight (segments stacked).
 *   N       total output width; n_seg, seg_n (host), w_mean [n_seg] as above.
 *   y       out [M,N]; y_dtype BL_F32, BL_BF16, or BL_I32 (the exact int32
 *           accumulators A, no rescale).
 *   ws      scratch of bl_gemv_workspace_bytes / bl_gemm_workspace_bytes
 *           bytes (activation codes, scales and row code sums when the call
 *           quantizes x).
 * K >= 1, K < 2^19 (bounds the int32 partial sums); N % 4 == 0.
 * ------------------------------------------------------------------------ */
size_t bl_gemv_workspace_bytes(int M, int N, int K);
int bl_gemv_w2a8(const void *x, int x_dtype, int ldx, const float *a, int M, int K,
                 const uint8_t *packed, int N, int n_seg, const int *seg_n,
                 const float *w_mean, void *y, int y_dtype,
                 void *ws, size_t ws_bytes, bl_stream stream);

/* ---------------------------------------------------------------------------
 * bl_gemv_w2a8_batched -- up to BL_MAX_PROBLEMS independent decode
 * contractions in one launch (for example the seven projections of a layer,
 * each with its own activations).  Each problem has the arguments of
 * bl_gemv_w2a8 and the same rules; the results are identical to n separate
 * bl_gemv_w2a8 calls.  problems is a host array.
 * ------------------------------------------------------------------------ */
typedef struct {
    const void *x;
    int x_dtype;
    int ldx;
    const float *a;
    int M;
    int K;
    const uint8_t *packed;
    int N;
    int n_seg;
    const int *seg_n; /* host */
    const float *w_mean;
    void *y;
    int y_dtype;
} bl_gemv_problem;

size_t bl_gemv_batched_workspace_bytes(int n, const bl_gemv_problem *problems);
int bl_gemv_w2a8_batched(int n, const bl_gemv_problem *problems, void *ws, size_t ws_bytes,
                         bl_stream stream);

size_t bl_gemm_workspace_bytes(int M, int N, int K);
int bl_gemm_w2a8(const void *x, int x_dtype, int ldx, const float *a, int M, int K,
                 const uint8_t *packed, int N, int n_seg, const int *seg_n,
                 const float *w_mean, void *y, int y_dtype,
                 void *ws, size_t ws_bytes, bl_stream stream);

/* ---------------------------------------------------------------------------
 * bl_subln_gemv_w2a8 -- a sub-norm and the projection behind it:
 *   y = BitLinear(RMSNorm(h)), i.e. bl_rmsnorm_quant then bl_gemv_w2a8 /
 *   bl_gemm_w2a8 on the codes (attn_sub_norm before o_proj).  [M] "模型详情"
 *   (subln); [T] the subln paragraph and "推理侧 BitLinear".
 *   h       [M,K] contiguous fp32 / bf16; gain [K] fp32 or NULL; eps >= 0.
 *   packed  [N/4,K] one segment with scale w_mean[0].
 *   y       out [M,N], y_dtype BL_F32 / BL_BF16 / BL_I32.
 *   q_out, a_out  optional (NULL): the codes [M,K] and scales [M] computed.
 *   ws      scratch of bl_subln_gemv_workspace_bytes(M, K) bytes.
 * Any M >= 1.  Decode sizes (M <= 64, K a multiple of 16, M*K small enough
 * for the fused prologue) run as one launch whose decode kernel normalizes
 * and quantizes its own rows; others run the norm kernel, then the
 * contraction.  Same bits either way.
 * ------------------------------------------------------------------------ */
size_t bl_subln_gemv_workspace_bytes(int M, int K);
int bl_subln_gemv_w2a8(const void *h, int h_dtype, int M, int K, const float *gain, float eps,
                       const uint8_t *packed, int N, const float *w_mean, void *y, int y_dtype,
                       int8_t *q_out, float *a_out, void *ws, size_t ws_bytes, bl_stream stream);

/* ---------------------------------------------------------------------------
 * bl_ffn_chain -- the feed-forward half of a BitNet layer, fused:
 *   subln RMSNorm(h) -> quantize -> gate|up -> ReLU^2(gate)*up ->
 *   ffn_sub_norm RMSNorm -> quantize -> down.
 * [T] subln paragraph after "推理侧 BitLinear" (normalize before the next
 * projection); [M] "模型详情" (ReLU squared in the FFN, subln, no bias) and
 * "BitNetConfig" (rms_norm_eps).
 *   h          [M,H] BL_F32 or BL_BF16.
 *   g_subln    [H] fp32 gain or NULL (unit gain); g_ffn [I] or NULL.
 *   eps        RMSNorm epsilon (the model uses 1e-5).
 *   packed_gu  [2I/4,H] uint8: gate tensor packed, then up tensor packed.
 *   w_mean_gu  [2] device: gate scale, up scale.
 *   packed_down [H/4,I] uint8; w_mean_down [1] device.
 *   y          out [M,H], BL_F32 or BL_BF16.
 *   dbg        (host struct, may be NULL) optional device buffers receiving
 *              the stage outputs for stage-wise checks; any member may be NULL.
 *   ws         scratch of bl_ffn_chain_workspace_bytes(M,H,I).
 * H % 4 == 0, I % 4 == 0, M >= 1.  M <= 64 runs the decode kernels, larger
 * M the prefill kernels.
 * ------------------------------------------------------------------------ */
typedef struct {
    int8_t *q1; /* [M,H] codes after subln            */
    float *a1;  /* [M]   their scales                 */
    float *p;   /* [M,I] ReLU^2(gate) * up            */
    int8_t *q2; /* [M,I] codes after ffn_sub_norm     */
    float *a2;  /* [M]   their scales                 */
} bl_ffn_debug;

size_t bl_ffn_chain_workspace_bytes(int M, int H, int I);
int bl_ffn_chain(const void *h, int h_dtype, int M, int H, int I,
                 const float *g_subln, const float *g_ffn, float eps,
                 const uint8_t *packed_gu, const float *w_mean_gu,
                 const uint8_t *packed_down, const float *w_mean_down,
                 void *y, int y_dtype, void *ws, size_t ws_bytes,
                 const bl_ffn_debug *dbg, bl_stream stream);

/* ---------------------------------------------------------------------------
 * bl_stack_decode -- the linear path of a stack of decoder layers for one
 * token (M = 1) in one persistent launch.  Per layer, with attention left
 * out (the stand-in wiring of the 30-layer stack: q's output feeds o, no
 * residual additions):
 *   x -> BitLinear q|k|v (segments H, KV, KV) -> BitLinear o on q's output
 *     -> subln RMSNorm -> BitLinear gate|up -> ReLU^2(gate)*up
 *     -> ffn_sub_norm RMSNorm -> BitLinear down -> the next layer's x.
 * [T] "推理侧 BitLinear" (each BitLinear: per-token quantization, the packed
 * ternary product, the rescale) and the subln paragraph; [M] "模型详情" and
 * "BitNetConfig" (subln, ReLU squared, rms_norm_eps).  Every stage computes
 * the same bits as bl_gemv_w2a8 / bl_ffn_chain (the RMSNorm's fp64 sum aside,
 * whose order may differ in the last bit, as between those calls).
 *   x        [H] fp32 or bf16 (x_dtype), the first layer's input;
 *   layers   host array of n_layers weight sets (device pointers): packed
 *            q|k|v [(H+2KV)/4, H] (q, k, v packed separately and stacked)
 *            with w_qkv [3]; o [H/4, H], w_o [1]; gate|up [2I/4, H] (gate,
 *            then up), w_gu [2]; down [H/4, I], w_down [1]; g_subln [H] and
 *            g_ffn [I] RMSNorm gains or NULL (unit gain);
 *   y        out [H] fp32, the last layer's output;
 *   stages   optional out [n_layers][(H+2KV) + H + I + H] fp32: per layer the
 *            q|k|v output, o's output, ReLU^2(gate)*up and down's output;
 *   ws       bl_stack_decode_workspace_bytes(n_layers, H, KV, I) bytes: the
 *            same stage outputs in the order the workgroups exchange them.
 * 1 <= n_layers <= 32; H and I multiples of 256 up to 8192, KV a multiple of
 * 16, within the kernel's per-workgroup capacity (the BitNet-2B4T shape
 * fits); the kernel needs one resident workgroup per compute unit.  Other
 * shapes return BL_ERR_SHAPE (run the layers with the other calls).  The
 * workgroups exchange stage outputs through device memory with bounded
 * waits: a wait that expires is counted (bl_device_errors) and the launch
 * still ends.  Calls sharing `stages` or ws must be ordered.
 * ------------------------------------------------------------------------ */
typedef struct {
    const uint8_t *packed_qkv;
    const float *w_qkv;
    const uint8_t *packed_o;
    const float *w_o;
    const uint8_t *packed_gu;
    const float *w_gu;
    const uint8_t *packed_down;
    const float *w_down;
    const float *g_subln;
    const float *g_ffn;
} bl_layer;

size_t bl_stack_decode_workspace_bytes(int n_layers, int H, int KV, int I);
int bl_stack_decode(const void *x, int x_dtype, int n_layers, const bl_layer *layers, int H, int KV, int I,
                    float eps, float *y, float *stages, void *ws, size_t ws_bytes, bl_stream stream);

/* ---------------------------------------------------------------------------
 * bl_unpack_bf16 / bl_gemm_unpacked -- the offline-unpacked path: the packed
 * ternary weight expanded once, at load time, to dense bf16 codes, and the
 * BitLinear forward as a dense bf16 product against them.  [T]
 * "BitNetQuantConfig" (AutoBitLinear with quantization_mode "offline": the
 * packed weight is unpacked to the module's compute dtype when loaded, and
 * the weight scale multiplies the output at inference) and "推理侧 BitLinear"
 * (the unpack); [M] the efficiency note (the stock path is not faster than
 * full precision), which this path lets one measure against the packed one.
 * bl_unpack_bf16:
 *   packed  [N/4,K] uint8 (plane order), n_seg segments stacked as for the
 *           contractions (seg_n host widths; n_seg = 1, seg_n = NULL: one);
 *   w_codes out [N,K] bf16, the codes -1, 0, +1 in output-column order (row
 *           n of segment s: packed row n' mod R_s of the segment, field
 *           n' div R_s, n' = n - the segment's first column, R_s = its
 *           width / 4).
 * bl_gemm_unpacked: the arguments of bl_gemm_w2a8 with w_codes [N,K] bf16 (as
 *   bl_unpack_bf16 writes them) in place of the packed weight; int8 codes in
 *   x must be contiguous rows.  The activation codes enter the product as
 *   bf16 (exact); every partial sum is an integer below 2^24 and is exact in
 *   the fp32 accumulators, so y is bit-identical to bl_gemm_w2a8's.  It
 *   streams 2 bytes per weight instead of a quarter byte.
 *   Shapes: N % 4 == 0; M <= 4 with K % 8 == 0, K <= 8192 runs the decode
 *   kernel; larger M needs K % 64 == 0 and N % 128 == 0 (the bf16 MFMA GEMM),
 *   else the decode kernel 4 rows at a time (K % 8 == 0, K <= 8192); other
 *   shapes return BL_ERR_SHAPE.  w_codes, y 16-byte aligned.
 *   ws: bl_gemm_unpacked_workspace_bytes(M, N, K) bytes.
 * ------------------------------------------------------------------------ */
int bl_unpack_bf16(const uint8_t *packed, int N, int K, int n_seg, const int *seg_n, void *w_codes,
                   bl_stream stream);
size_t bl_gemm_unpacked_workspace_bytes(int M, int N, int K);
int bl_gemm_unpacked(const void *x, int x_dtype, int ldx, const float *a, int M, int K,
                     const void *w_codes, int N, int n_seg, const int *seg_n,
                     const float *w_mean, void *y, int y_dtype,
                     void *ws, size_t ws_bytes, bl_stream stream);

/* ---------------------------------------------------------------------------
 * bl_ffn_chain_noalloc -- bl_ffn_chain for callers that cannot allocate
 * device memory or pass a workspace: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  Same arguments and results
 * as bl_ffn_chain without ws / ws_bytes: its scratch is a fixed device array
 * inside the library of bl_ffn_chain_noalloc_max_bytes() bytes (32 MiB), one
 * per device, held until the process ends.  The call allocates nothing.
 * Sizes whose scratch (bl_ffn_chain_workspace_bytes(M, H, I)) exceeds it are
 * rejected with BL_ERR_WORKSPACE before anything is enqueued (at the
 * BitNet-2B4T shape, H 2560 / I 6912, up to 903 rows).  All calls on one
 * device share that array: calls that overlap in time on one device (other
 * streams, other host threads) race and must be ordered by the caller.
 * ------------------------------------------------------------------------ */
size_t bl_ffn_chain_noalloc_max_bytes(void);
int bl_ffn_chain_noalloc(const void *h, int h_dtype, int M, int H, int I,
                         const float *g_subln, const float *g_ffn, float eps,
                         const uint8_t *packed_gu, const float *w_mean_gu,
                         const uint8_t *packed_down, const float *w_mean_down,
                         void *y, int y_dtype, const bl_ffn_debug *dbg, bl_stream stream);

/* ---------------------------------------------------------------------------
 * bl_rope_table / bl_attn_decode -- the attention side of a decoder layer
 * for one new token (decode).  "BitNet" model documentation, "模型详情"
 * (rotary position embeddings) and "BitNetConfig" (20 attention heads, 5
 * key/value heads: grouped-query attention, each key/value head serving
 * n_heads / n_kv_heads consecutive query heads; 128 dimensions per head;
 * rope_theta a parameter).
 *
 * bl_rope_table (host only): cos / sin of pos * base^(-2i/head_dim) for
 *   pos < max_pos, i < head_dim/2, computed in fp64 and rounded to fp32, into
 *   host arrays cos_out / sin_out [max_pos][head_dim/2].  Copy them to the
 *   device for bl_attn_decode.  Returns BL_OK or BL_ERR_NULL / BL_ERR_SHAPE.
 *
 * bl_attn_decode: for the token at position pos,
 *   q [n_heads*128], k_new, v_new [n_kv_heads*128] fp32 device (before RoPE);
 *   k_cache, v_cache [n_kv_heads][max_seq][128] fp32 device: positions
 *     0 .. pos-1 hold the earlier tokens' rotated keys and their values; the
 *     call writes the token's rotated key and its value at position pos;
 *   rope_cos, rope_sin [max_seq][64] device (bl_rope_table);
 *   out [n_heads*128] fp32 device: per query head h,
 *     softmax_j(q'_h . k'_j / sqrt(128)) summed with v_j over j = 0 .. pos,
 *     with the key/value head h / (n_heads / n_kv_heads) and q', k' rotated
 *     by RoPE (dimension i paired with i + 64);
 *   ws device scratch of bl_attn_decode_workspace_bytes(n_heads, max_seq)
 *     bytes (per-chunk partial results); calls that share it must be
 *     ordered on one stream.
 * head_dim must be 128; n_heads a multiple of n_kv_heads with at most 4
 * query heads per key/value head; 0 <= pos < max_seq <= 32768; all device
 * pointers 16-byte aligned.  Arithmetic in fp32 (scores, exponentials, sums).
 * ------------------------------------------------------------------------ */
int bl_rope_table(int max_pos, int head_dim, double base, float *cos_out, float *sin_out);
size_t bl_attn_decode_workspace_bytes(int n_heads, int max_seq);
int bl_attn_decode(const float *q, const float *k_new, const float *v_new, int pos,
                   int n_heads, int n_kv_heads, int head_dim,
                   float *k_cache, float *v_cache, int max_seq,
                   const float *rope_cos, const float *rope_sin,
                   float *out, void *ws, size_t ws_bytes, bl_stream stream);

/* ---------------------------------------------------------------------------
 * bl_attn_prefill -- the attention side of a decoder layer for a prompt of M
 * tokens at positions 0 .. M-1.  Same pages and readings as bl_attn_decode;
 * token p attends to positions 0 .. p (causal).
 *   q [M rows][n_heads*128], k, v [M rows][n_kv_heads*128] fp32 device,
 *     row stride ldx elements (views into one q|k|v row are fine), before RoPE;
 *   k_cache, v_cache [n_kv_heads][max_seq][128] fp32 device: positions
 *     0 .. M-1 receive the rotated keys and the values (for later
 *     bl_attn_decode calls);
 *   rope_cos, rope_sin [>= M][64] device (bl_rope_table);
 *   out [M rows][ldo] fp32 device, head h at columns h*128 .. h*128+127;
 *   ws device scratch of bl_attn_prefill_workspace_bytes(M, n_heads,
 *     n_kv_heads) bytes.
 * Precision: the rotated queries and keys, the values and the probabilities
 * enter the two products as bf16 (round to nearest even), with fp32
 * products' sums, fp32 softmax and an fp32 result; the caches get fp32.
 * head_dim must be 128; n_heads a multiple of n_kv_heads; 1 <= M <= max_seq;
 * ldx, ldo >= n_heads*128, ldo a multiple of 4; out 16-byte aligned.
 * ------------------------------------------------------------------------ */
size_t bl_attn_prefill_workspace_bytes(int M, int n_heads, int n_kv_heads);
int bl_attn_prefill(const float *q, const float *k, const float *v, int ldx, int M,
                    int n_heads, int n_kv_heads, int head_dim,
                    float *k_cache, float *v_cache, int max_seq,
                    const float *rope_cos, const float *rope_sin,
                    float *out, int ldo, void *ws, size_t ws_bytes, bl_stream stream);

/* ---------------------------------------------------------------------------
 * bl_ste_grad_input / bl_ste_grad_weight -- the backward pass of BitLinear in
 * quantization-aware training.  [T] "BitLinear 的三步量化": the weight and
 * activation quantizers of training pass the incoming gradient through
 * unchanged (straight-through estimator), so with the fake-quantized
 * W~ = codes * w_mean and x~ = q / a of the forward:
 *   dX = dY . W~     (bl_ste_grad_input)
 *   dW = dY^T . x~   (bl_ste_grad_weight; the gradient of the fp32 master W)
 *   dy      [M][N] device, contiguous: the output gradient, dy_dtype BL_BF16
 *           or BL_F32 (an fp32 gradient is rounded to bf16 on the device);
 *   packed  [N/4][K] uint8 device, one weight segment; w_mean [1] fp32 device;
 *   q, a    [M][K] int8 and [M] fp32 device: the forward's activation codes
 *           and scales (bl_quant_act);
 *   dx      out [M][K] device = (sum_n bf16(dy[m][n]) code[n][k]) * w_mean, in
 *           dx_dtype BL_F32, or BL_BF16 (that fp32 value rounded to nearest
 *           even: the input dtype of a bf16 layer, so no cast follows);
 *   dw      out [N][K] fp32 device = sum_m bf16(fp32(dy[m][n] / a[m])) q[m][k];
 *   ws      scratch of bl_ste_grad_input_workspace_bytes(M, N, K, dy_dtype) /
 *           bl_ste_grad_weight_workspace_bytes(M, N, K) bytes (the operands
 *           in bf16, padded to whole tiles).
 * Precision: bf16 products (the codes and q exactly) summed in fp32; the
 * plain fp64 definitions differ by at most the bf16 rounding of the gradient
 * (relative 2^-8 per term) plus the fp32 sums.  Any M, N, K >= 1 (N a
 * multiple of 4 for dx), each product of two of them, rounded up to 128,
 * below 2^31; dw and an fp32 dx 16-byte aligned, a bf16 dx 8-byte aligned;
 * dy 16-byte aligned for dx.  An unknown dx_dtype is BL_ERR_DTYPE.
 * ------------------------------------------------------------------------ */
size_t bl_ste_grad_input_workspace_bytes(int M, int N, int K, int dy_dtype);
size_t bl_ste_grad_weight_workspace_bytes(int M, int N, int K);
int bl_ste_grad_input(const void *dy, int dy_dtype, int M, int N, int K, const uint8_t *packed,
                      const float *w_mean, void *dx, int dx_dtype, void *ws, size_t ws_bytes, bl_stream stream);
int bl_ste_grad_weight(const void *dy, int dy_dtype, const int8_t *q, const float *a, int M, int N, int K,
                       float *dw, void *ws, size_t ws_bytes, bl_stream stream);

/* ---------------------------------------------------------------------------
 * The 1-bit BitLinear.  [S] "How It Works": weights binarized to one bit,
 * activations layer-normalized and absmax-quantized.  The page prints no
 * formula; these calls compute (the readings stated with the oracle):
 *  - weight sign   s = -1 where W < 0, else +1 (zeros +1);
 *  - weight scale  w_scale = max(float(sum|W| / count), 1e-5), sum in fp64
 *                  (the ternary path's absmean);
 *  - packed        P[r,k] bit i = (s[i*N/8 + r, k] == +1)  (plane order,
 *                  N/8 packed rows, one bit per weight);
 *  - layer norm    mu = sum x / K and var = sum (x - mu)^2 / K in fp64,
 *                  r = float(1/sqrt(var + eps)),
 *                  x' = (float(x - mu) * r) * gamma + beta (fp32; gamma and
 *                  beta optional);
 *  - act codes     bl_quant_act's per-token absmax int8 of x';
 *  - output        A = sum_k q * s (exact int32), y = float(A) * (w_scale / a).
 *
 * bl_binarize_pack: W [N,K] fp32 -> packed [N/8,K] uint8 and w_scale [1];
 *   ws of bl_binarize_workspace_bytes(N, K) bytes.  N >= 8, N % 8 == 0,
 *   K % 4 == 0, N*K < 2^40.
 * bl_layernorm_quant: x [M,K] (row stride ldx elements, 0 = K; BL_F32 or
 *   BL_BF16) -> q [M,K] int8, a [M] fp32; gamma, beta [K] or NULL.
 *   K % 4 == 0, 4 <= K <= 16384, ldx % 4 == 0.
 * bl_gemm_w1a8: q [M,K] int8 and a [M] -> y [M,N] fp32 with packed [N/8,K]
 *   and w_scale [1].  K % 16 == 0, 16 <= K <= 16384, N % 8 == 0.
 * bl_bitlinear_w1: up to 8 independent forwards (x -> y) in two launches
 *   (all the norms, then all the contractions); each problem as in
 *   bl_layernorm_quant + bl_gemm_w1a8; ws of
 *   bl_bitlinear_w1_workspace_bytes(probs, n) bytes holds the codes and
 *   scales.
 * Every pointer 16-byte aligned (y: 4).  Errors: BL_ERR_NULL, BL_ERR_SHAPE,
 * BL_ERR_DTYPE, BL_ERR_ALIGN, BL_ERR_WORKSPACE before any launch.
 * ------------------------------------------------------------------------ */
typedef struct {
    const void *x;          /* [M, K] fp32 or bf16 activations       */
    int x_dtype;
    int M, K;
    const float *gamma;     /* [K] layer-norm gain or NULL             */
    const float *beta;      /* [K] layer-norm bias or NULL             */
    const uint8_t *packed;  /* [N/8, K] bl_binarize_pack output        */
    int N;
    const float *w_scale;   /* [1]                                      */
    float *y;               /* out [M, N] fp32                          */
} bl_w1_problem;

size_t bl_binarize_workspace_bytes(int64_t N, int64_t K);
int bl_binarize_pack(const float *W, int N, int K, uint8_t *packed, float *w_scale, void *ws, size_t ws_bytes,
                     bl_stream stream);
int bl_layernorm_quant(const void *x, int x_dtype, int M, int K, int ldx, const float *gamma, const float *beta,
                       float eps, int8_t *q, float *a, bl_stream stream);
int bl_gemm_w1a8(const int8_t *q, const float *a, int M, int K, const uint8_t *packed, int N,
                 const float *w_scale, float *y, bl_stream stream);
size_t bl_bitlinear_w1_workspace_bytes(const bl_w1_problem *probs, int n);
int bl_bitlinear_w1(const bl_w1_problem *probs, int n, float eps, void *ws, size_t ws_bytes, bl_stream stream);

#ifdef __cplusplus
}
#endif
#endif /* BITLINEAR_H */
