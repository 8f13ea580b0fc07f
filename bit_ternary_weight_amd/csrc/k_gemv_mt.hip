// k_gemv_mt.hip -- batched decode BitLinear (5 <= M <= 64 tokens) with the
// int8 codes precomputed by the row quantizer: stream the packed ternary
// weights from HBM once and contract them with the codes of all the tokens
// on the matrix cores.
//
// "Transformers 实战 BitNet 1.58 位量化", section "推理侧 BitLinear：打包权重、解包与缩放":
// the inference forward multiplies the per-token int8 activations with the
// unpacked ternary weight and rescales by both scales; the 2-bit fields are
// expanded in registers, never written back.
#include "bl_buffer.h"
#include "bl_common.h"

namespace bl {

// ===========================================================================
// Batched decode with precomputed codes (5 <= M <= 64, the quantizer has
// written the int8 codes tiled by 64-byte pieces of K -- code_offset -- with
// their scales and row code sums): a streaming kernel in the manner of
// k_gemv_v1, with the tokens in the MFMA's 16 columns.  One 8-wave workgroup
// per tile of 16 * G packed rows of one problem over all of K (G = 1, 2, 4,
// 8, sized to the CU's share of the batch's weight bytes); the 8 / G waves of
// a 16-row group split its K into interleaved 256-byte blocks.
//   * A block (16 rows x 256 bytes) arrives as four whole-line loads of 4
//     rows x 256 bytes (lane L: row L >> 4, bytes 16 (L & 15) .. +15;
//     non-temporal) and goes through a 4 KB LDS buffer of the wave (16-byte
//     chunk c of row r at position c ^ r: conflict-free both ways), from
//     which lane (g, l) reads row l, bytes 16 g .. +15 of each 64-byte piece:
//     the MFMA operand layout.  (Loading that layout directly from HBM, 16
//     rows x 16 bytes per quarter wave, was 30 % slower.)
//   * The codes of tokens l, 16 + l, ... (T token tiles of 16) for the same
//     piece are 1 KB contiguous in the tiled layout, loaded straight into
//     registers.
//   * Each field of a piece, masked in place, goes through one
//     v_mfma_i32_16x16x64_i8 per token tile with the weights as the first
//     operand, so lane (g, c) accumulates packed rows 4 g .. 4 g + 3 for
//     token c: four consecutive output columns.
// Blocks go two in flight (with 64 tokens the codes one block ahead), every
// wave issuing the same number of loads on every path (the compiler's waits
// stay exact; past its blocks a wave's loads fall outside their buffer
// range and move no data).  The waves of a row group add their partial sums
// through LDS at the end.
// ===========================================================================
constexpr int kMtWaves = 8;
constexpr int kMtMaxBlocks = 8;   // 256-byte blocks per wave (4 with 64 tokens: registers)
__host__ __device__ constexpr int mt_max_blocks(int T) { return T >= 4 ? 4 : kMtMaxBlocks; }
constexpr int kMtBufBytes = 4096; // a wave's transpose buffer

// Rescale and store four consecutive packed rows vr0 .. vr0 + 3 (vr0 a
// multiple of 4) of field f for token m from their exact sums s (codes + 1,
// times the field scale); qs, am: the token's code sum and scale, wm: the
// weight scale of row vr0's segment (all loaded before the weight stream).
__device__ __forceinline__ void mt_emit4(const GemvProblem &p, int vr0, int m, int f, v4i s, int qs, float am,
                                         float wm) {
    if (m >= p.M || vr0 >= p.R) return;
    const int sh = f == 0 ? 0 : (f == 1 ? 2 : 4);
    int A[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) A[j] = (s[j] >> sh) - qs;
    const size_t rowo = (size_t)m * p.ldy;
    if (p.vout) {
        const ColOf co = col_of(p.seg, vr0, f);
        const float sc = wm / am;   // IEEE fp32 division, as the oracle
        float v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = p.y_dt == BL_I32 ? __int_as_float(A[j]) : (float)A[j] * sc;
        store4(p.y, p.y_dt, rowo + co.col, v);
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (vr0 + j >= p.R) break;
            const ColOf co = col_of(p.seg, vr0 + j, f);
            store_out(p.y, p.y_dt, rowo + co.col, A[j], p.w_mean[co.seg] / am);
        }
    }
}

template <int T, int NB>
__global__ __launch_bounds__(kMtWaves * 64) void k_gemv_mt(GemvBatch b) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    __shared__ int qs_tab[64];
    __shared__ float am_tab[64];
    __shared__ float wm_tab[BL_MAX_SEGMENTS];

    int pi = 0;
#pragma unroll
    for (int i = 1; i < kMaxProblems; ++i)
        if (i < b.n && (int)blockIdx.x >= b.p[i].tile0) pi = i;
    const GemvProblem &p = b.p[pi];
    // the problem's fields read here together (the compiler would issue each
    // kernel-argument load next to its first use, one round trip after
    // another ahead of the first weight load)
    asm volatile("" ::"s"(p.K), "s"(p.cs), "s"(p.tile0), "s"(p.R), "s"(p.M), "s"(p.qtile), "s"(p.P), "s"(p.x),
                 "s"(p.qsum), "s"(p.a), "s"(p.w_mean), "s"(p.seg.n));

    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4;
    const int lr = lane & 15;
    const int K = p.K;
    const int lw = 3 - __builtin_ctz(p.cs);       // log2 waves per 16-row group
    const int grp = wave >> lw;
    const int kr0 = wave & ((1 << lw) - 1);
    const int kstep = 1 << lw;
    const int nkb = K >> 8;                       // 256-byte blocks per row
    const int ks = kr0 < nkb ? (nkb - kr0 + kstep - 1) >> lw : 0;   // <= NB
    // Block t covers the wave's block (t + rot) mod ks: waves and workgroups
    // start at different offsets of their rows (the sum is order-free).
    const int rot = ks > 0 ? (int)(((unsigned)blockIdx.x * 7u + (unsigned)wave * 3u) % (unsigned)ks) : 0;
    auto kb_of = [&](int t) {
        const int j = t + rot;
        return kr0 + kstep * (j >= ks ? j - ks : j);
    };
    const int r0 = ((int)blockIdx.x - p.tile0) * 16 * p.cs;
    // Weights and codes go through buffer resources (gemv_mt_ok bounds both
    // ranges below 2^31 bytes).  The padding loads -- blocks past the wave's
    // own, and rows past R -- fall outside the range: they return zeros and
    // move no data.  (Token tiles past the problem's codes re-read its last
    // tile.)  A load's offset is this lane's in-range offset plus a uniform
    // block offset, kBufOob for a padding block.
    const int rb = r0 + 16 * grp;   // the wave's row group
    const int vrows = p.R - rb <= 0 ? 0 : (p.R - rb < 16 ? p.R - rb : 16);
    const __amdgpu_buffer_rsrc_t wrs = buf_rsrc(p.P + (size_t)(vrows > 0 ? rb : 0) * K, vrows * K);
    unsigned wo[4];   // this lane's offsets of the four loads of block 0
#pragma unroll
    for (int j = 0; j < 4; ++j) wo[j] = (unsigned)((4 * j + (lane >> 4)) * K + 16 * lr);
    const int qt = p.qtile;
    const __amdgpu_buffer_rsrc_t crs = buf_rsrc(p.x, qt * K);
    unsigned co[T];   // this lane's offsets of token tile u in piece 0
#pragma unroll
    for (int u = 0; u < T; ++u) co[u] = (unsigned)((16 * (16 * u < qt ? u : qt / 16 - 1) + lr) * 64 + 16 * g);
    // The epilogue's inputs (token code sums and scales, segment weight
    // scales) are loaded right after the first block, so that their latency
    // is hidden; every lane loads the same number (clamped indices), so the
    // compiler's waits for the stream stay exact.  (With 64 tokens the
    // launcher never makes a wave own whole rows, and the registers are
    // needed elsewhere: only the shared tables are loaded, at the end.)
    constexpr bool kOwn = T < 4;
    const int M = p.M;
    int qs_l[kOwn ? T : 1];
    float am_l[kOwn ? T : 1];
    float wm_l = 0.0f;
    const int mt_ = (int)threadIdx.x < M ? (int)threadIdx.x : M - 1;
    const int sg_ = (int)threadIdx.x < p.seg.n ? (int)threadIdx.x : p.seg.n - 1;
    int qs_t = 0;
    float am_t = 0.0f, wm_t = 0.0f;
    unsigned char *buf = smem + wave * kMtBufBytes;
    // LDS offsets: the block's load j lands at row 4 j + (lane >> 4), chunk
    // lane & 15; piece k of the block is read at row lr, chunk 4 k + g
    int woff[4], roff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = 4 * j + (lane >> 4);
        woff[j] = r * 256 + 16 * ((lane & 15) ^ r);
        roff[j] = lr * 256 + 16 * ((4 * j + g) ^ lr);
    }

    // Two blocks of weights in flight; the codes of two blocks as well below
    // 64 tokens, of one block (issued a block ahead) with 64, whose code
    // registers would not fit twice.
    constexpr int CB = kOwn ? 2 : 1;
    v4i wv[2][4];
    v4i cv[CB][4][T];
    auto issue_w = [&](int t, int sl) {
        const unsigned bo = __builtin_amdgcn_readfirstlane(t < ks ? 256u * (unsigned)kb_of(t) : kBufOob);
#pragma unroll
        for (int j = 0; j < 4; ++j) wv[sl][j] = buf_ld16<kBufNt>(wrs, wo[j] + bo);
    };
    auto issue_c = [&](int t, int sl) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const unsigned po = __builtin_amdgcn_readfirstlane(
                t < ks ? (4u * (unsigned)kb_of(t) + k) * (unsigned)qt * 64u : kBufOob);
#pragma unroll
            for (int u = 0; u < T; ++u) cv[sl][k][u] = buf_ld16<0>(crs, co[u] + po);
        }
    };
    v4i acc[T][4];
#pragma unroll
    for (int u = 0; u < T; ++u)
#pragma unroll
        for (int f = 0; f < 4; ++f) acc[u][f] = v4i{0, 0, 0, 0};
    issue_w(0, 0);
    issue_c(0, 0);
    if constexpr (kOwn) {
#pragma unroll
        for (int u = 0; u < T; ++u) {
            const int m = 16 * u + lr < M ? 16 * u + lr : M - 1;
            qs_l[u] = p.qsum[m];
            am_l[u] = p.a[m];
        }
        const int vr0l = r0 + 16 * grp + 4 * g;
        wm_l = p.w_mean[col_of(p.seg, vr0l < p.R ? vr0l : p.R - 1, 0).seg];
        qs_t = p.qsum[mt_];
        am_t = p.a[mt_];
        wm_t = p.w_mean[sg_];
    }
    if (NB > 1) {
        issue_w(1, 1);
        if (CB == 2) issue_c(1, 1);
    }
#pragma unroll
    for (int t = 0; t < NB; ++t) {
        const int sl = t & 1;
        const int cs = CB == 2 ? sl : 0;
        if (t < ks) {
            // raised priority over the block's products: the other wave of
            // the SIMD issues its loads meanwhile (64 tokens: 22.95 -> 22.45 us)
            __builtin_amdgcn_s_setprio(1);
            // this wave's LDS operations run in order: the reads below see
            // these writes, and the next block's writes come after them
#pragma unroll
            for (int j = 0; j < 4; ++j) *reinterpret_cast<v4i *>(buf + woff[j]) = wv[sl][j];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const v4i w = *reinterpret_cast<const v4i *>(buf + roff[k]);
                v4i f0, f1, f2, f3;
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const uint32_t x = (uint32_t)w[d];
                    f0[d] = (int)(x & 0x03030303u);
                    f1[d] = (int)(x & 0x0C0C0C0Cu);
                    f2[d] = (int)(x & 0x30303030u);
                    f3[d] = (int)((x >> 2) & 0x30303030u);
                }
#pragma unroll
                for (int u = 0; u < T; ++u) {
                    acc[u][0] = mfma16(f0, cv[cs][k][u], acc[u][0]);
                    acc[u][1] = mfma16(f1, cv[cs][k][u], acc[u][1]);
                    acc[u][2] = mfma16(f2, cv[cs][k][u], acc[u][2]);
                    acc[u][3] = mfma16(f3, cv[cs][k][u], acc[u][3]);
                }
            }
            __builtin_amdgcn_s_setprio(0);
        }
        if (CB == 2) {
            if (t + 2 < NB) {
                issue_w(t + 2, sl);
                issue_c(t + 2, sl);
            }
        } else {
            if (t + 1 < NB) issue_c(t + 1, 0);
            if (t + 2 < NB) issue_w(t + 2, sl);
        }
        if (kOwn && t == 0) {
            // the shared tables of the epilogue (their loads, the oldest of
            // the wave, have landed by now); read after the final barrier
            if (threadIdx.x < 64) {
                qs_tab[threadIdx.x] = qs_t;
                am_tab[threadIdx.x] = am_t;
            }
            if (threadIdx.x < BL_MAX_SEGMENTS) wm_tab[threadIdx.x] = wm_t;
        }
    }

    // lane (g, c): packed rows 16 grp + 4 g + j, token 16 u + c
    const int vr0 = r0 + 16 * grp + 4 * g;
    if constexpr (kOwn) {
        if (lw == 0) {
            // one wave per row group: its sums are complete
#pragma unroll
            for (int u = 0; u < T; ++u)
#pragma unroll
                for (int f = 0; f < 4; ++f) mt_emit4(p, vr0, 16 * u + lr, f, acc[u][f], qs_l[u], am_l[u], wm_l);
            return;
        }
    }
    if constexpr (!kOwn) {
        if (threadIdx.x < 64) {
            qs_tab[threadIdx.x] = p.qsum[mt_];
            am_tab[threadIdx.x] = p.a[mt_];
        }
        if (threadIdx.x < BL_MAX_SEGMENTS) wm_tab[threadIdx.x] = p.w_mean[sg_];
    }
    // the partial sums reuse the transpose buffers: every wave must be done
    __syncthreads();
    v4i *part = reinterpret_cast<v4i *>(smem);   // [wave][token tile][field][lane]
#pragma unroll
    for (int u = 0; u < T; ++u)
#pragma unroll
        for (int f = 0; f < 4; ++f) part[((wave * T + u) * 4 + f) * 64 + lane] = acc[u][f];
    __syncthreads();
    const int items = p.cs * T * 4 * 64;
    for (int e = threadIdx.x; e < items; e += kMtWaves * 64) {
        const int ln = e & 63;
        const int f = (e >> 6) & 3;
        const int u = (e >> 8) % T;
        const int ge = (e >> 8) / T;
        v4i sum = v4i{0, 0, 0, 0};
        for (int kr = 0; kr < kstep; ++kr) sum += part[((((ge << lw) + kr) * T + u) * 4 + f) * 64 + ln];
        const int m = 16 * u + (ln & 15);
        const int ve = r0 + 16 * ge + 4 * (ln >> 4);
        const int mc = m < M ? m : M - 1;
        mt_emit4(p, ve, m, f, sum, qs_tab[mc], am_tab[mc], wm_tab[col_of(p.seg, ve < p.R ? ve : p.R - 1, 0).seg]);
    }
}

template <int T, int NB>
hipError_t go_gemv_mt(GemvBatch &o, int tiles, hipStream_t s) {
    const size_t part = (size_t)kMtWaves * T * 4 * 64 * sizeof(v4i);
    const size_t lds = part > (size_t)kMtWaves * kMtBufBytes ? part : (size_t)kMtWaves * kMtBufBytes;
    if (lds > 65536)
        if (hipError_t e = allow_dynamic_lds(reinterpret_cast<const void *>(&k_gemv_mt<T, NB>), lds); e != hipSuccess)
            return e;
    hipLaunchKernelGGL((k_gemv_mt<T, NB>), dim3(tiles), dim3(kMtWaves * 64), lds, s, o);
    return hipGetLastError();
}

template <int T>
hipError_t go_gemv_mt_nb(int nb, GemvBatch &o, int tiles, hipStream_t s) {
    switch (nb) {
    case 1: return go_gemv_mt<T, 1>(o, tiles, s);
    case 2: return go_gemv_mt<T, 2>(o, tiles, s);
    case 3: return go_gemv_mt<T, 3>(o, tiles, s);
    case 4: return go_gemv_mt<T, 4>(o, tiles, s);
    default:
        if constexpr (mt_max_blocks(T) > 4) return nb <= 6 ? go_gemv_mt<T, 6>(o, tiles, s) : go_gemv_mt<T, 8>(o, tiles, s);
        else return hipErrorNotSupported;
    }
}

// Every problem fits k_gemv_mt: tiled codes with their row sums, no
// gate|up pairing, K a multiple of 64, aligned weights.
bool gemv_mt_ok(const GemvBatch &b) {
    for (int i = 0; i < b.n; ++i) {
        const GemvProblem &p = b.p[i];
        if (p.mode != 0 || p.pair != 0 || p.qsum == nullptr || p.a == nullptr || p.M < 1 || p.M > 64 ||
            p.qtile < 16 || p.qtile % 16 != 0 || p.qtile < p.M || p.K < 256 || p.K % 256 != 0 ||
            (size_t)p.qtile * p.K >= ((size_t)1 << 31) || (size_t)16 * p.K >= ((size_t)1 << 31) ||
            ((uintptr_t)p.x % 16) != 0 || ((uintptr_t)p.P % 16) != 0)
            return false;
    }
    return true;
}

bool gemv_mt_plan_ok(int n, const int *Ms, const int *Ks) {
    int maxm = 1;
    for (int i = 0; i < n; ++i) {
        if (Ms[i] < 1 || Ms[i] > 64 || Ks[i] < 256 || Ks[i] % 256 != 0) return false;
        maxm = Ms[i] > maxm ? Ms[i] : maxm;
    }
    const int cap = mt_max_blocks((maxm + 15) / 16);
    for (int i = 0; i < n; ++i)
        if ((Ks[i] / 256 + kMtWaves - 1) / kMtWaves > cap) return false;
    return true;
}

// Tiles as for k_gemv_v1: the largest 16 * G rows (G = 8, 4, 2, 1) within
// 1.25x the CU's even share of the weight bytes whose waves need at most
// mt_max_blocks blocks; largest tiles on the lowest workgroup numbers.
// Returns hipErrorNotSupported when some problem's K needs more units.
hipError_t launch_gemv_mt(GemvBatch &b, hipStream_t s) {
    const int cus = device_cu_count();
    int maxm = 1;
    for (int i = 0; i < b.n; ++i) maxm = b.p[i].M > maxm ? b.p[i].M : maxm;
    const int T = (maxm + 15) / 16;
    const size_t share = even_share(b, 1, cus) * 5 / 4;
    int gv[kMaxProblems];
    size_t tb[kMaxProblems];
    int maxu = 1;
    for (int i = 0; i < b.n; ++i) {
        const GemvProblem &q = b.p[i];
        const int nkb = q.K / 256;
        auto units = [&](int G) {
            const int kstep = kMtWaves / G;
            return (nkb + kstep - 1) / kstep;
        };
        int G = T < 4 ? kMtWaves : kMtWaves / 2;   // 64 tokens: at least two waves per row group
        while (G > 1 && ((size_t)16 * G * q.K > share || units(G) > mt_max_blocks(T))) G >>= 1;
        if (units(G) > mt_max_blocks(T)) return hipErrorNotSupported;
        gv[i] = G;
        tb[i] = (size_t)16 * G * q.K;
        maxu = units(G) > maxu ? units(G) : maxu;
    }
    int order[kMaxProblems];
    for (int i = 0; i < b.n; ++i) order[i] = i;
    for (int i = 1; i < b.n; ++i)
        for (int j = i; j > 0 && tb[order[j]] > tb[order[j - 1]]; --j) {
            const int t = order[j];
            order[j] = order[j - 1];
            order[j - 1] = t;
        }
    GemvBatch o = b;
    int tiles = 0;
    for (int i = 0; i < b.n; ++i) {
        GemvProblem &q = o.p[i];
        q = b.p[order[i]];
        q.cs = gv[order[i]];
        q.tile0 = tiles;
        tiles += (q.R + 16 * q.cs - 1) / (16 * q.cs);
        const size_t esz = q.y_dt == BL_BF16 ? 2 : 4;
        bool v = q.R % 4 == 0 && q.ldy % 4 == 0 && ((uintptr_t)q.y % (4 * esz)) == 0;
        for (int j = 0; j <= q.seg.n; ++j)
            if (q.seg.roff[j] % 4 != 0) v = false;
        q.vout = v ? 1 : 0;
    }
    o.ring_off = 0;
    switch (T) {
    case 1: return go_gemv_mt_nb<1>(maxu, o, tiles, s);
    case 2: return go_gemv_mt_nb<2>(maxu, o, tiles, s);
    case 3: return go_gemv_mt_nb<3>(maxu, o, tiles, s);
    default: return go_gemv_mt_nb<4>(maxu, o, tiles, s);
    }
}

} // namespace bl
