// Scaled FP8 grouped GEMM on gfx950 matrix cores, with the dequantization fused into the
// epilogue (latestnews.news "AMD Boosts PyTorch FP8 Training on Instinct GPUs", third
// paragraph: grouped GEMM for MoE on ROCm; ai-radar.it "FP8 su GPU AMD ...", introduction:
// rowwise activation scales, colwise expert-weight scales and the token offsets that route rows
// to experts; fosswire.org "AMD Primus adds FP8/MXFP8 kernels ...", section "What Primus adds
// for MoE training on MI355X": FP8 and MXFP8 grouped GEMM for the expert FFNs).
//
// Both operands are contraction-contiguous byte matrices ("row" = one output row or column):
//   forward, M-grouped:  out[m,n]   = sum_k A[m,k] * B_g[n,k] / (sa[m] * sb[g,n]),  m in group g
//   wgrad, K-grouped:    out[g,k,n] = sum_{m in g} A[k,m] * B[n,m] / (sa[g,k] * sb[g,n])
//   MX forward:          out[m,n]   = sum_kb 2^(ea+eb) sum_{k in kb} A[m,k] * B_g[n,k]
//
// Kernel: 256 threads (4 waves in 2x2), a 128x128 output tile per block, contraction steps of
// 128 bytes.  Each step, every lane fetches 4 16-byte chunks of each operand tile into
// registers (the next step's fetch is in flight while the current step computes), stores them
// into a double-buffered LDS tile (row r, chunk c at position c ^ (r & 7): the eight 16-byte
// reads of a fragment load hit distinct banks), and each wave runs 4x4
// v_mfma_f32_16x16x128_f8f6f4 (OCP e4m3 operands; the block-scaled form for MX) over its 64x64
// sub-tile.  Operand lane layout of that instruction on gfx950 (established with one-hot
// inputs): lane l holds row l%16; its bytes 0-15 are K offsets 16*(l/16)+[0,16) and bytes 16-31
// are K offsets 64+16*(l/16)+[0,16); lane r+16b supplies the E8M0 scale of row r, K block b;
// result register i of lane l is row 4*(l/16)+i, column l%16.
//
// e4m3fnuz operands: gfx950's matrix cores read OCP e4m3 only (byte 0x7F, the fnuz 240 code, is
// NaN there), so fnuz bytes are re-encoded to the e4m3fn byte of the same value while staging
// into LDS: exponent field - 1 for fnuz exponents >= 2 (exact), and the nearest e4m3fn
// subnormal (ties to even) for fnuz values below 2^-6, which moves a product by at most 2^-10
// quantization units.
//
// Group scheduling stays on the device (no host read of the offsets): the forward grid has
// ceil(M/128) + G row-tile slots, each block finds its (group, row tile) with a block-wide scan
// of per-group tile counts, and surplus slots exit.  Offsets are clamped into [0, M] before use.
#include "common.hpp"

namespace fp8q {

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v4f_t __attribute__((ext_vector_type(4)));

constexpr int GB_M = 128, GB_N = 128, GB_K = 128;
constexpr int MODE_FWD = 0, MODE_WGRAD = 1;

// Bytes of `w` at positions base..base+3 kept where lo <= pos < hi.
__device__ __forceinline__ uint32_t keep_mask4(int lo, int hi, int base) {
    int a = lo - base, b = hi - base;
    a = a < 0 ? 0 : (a > 4 ? 4 : a);
    b = b < 0 ? 0 : (b > 4 ? 4 : b);
    const uint32_t below_b = b >= 4 ? 0xFFFFFFFFu : ((1u << (8 * b)) - 1u);
    const uint32_t from_a = a >= 4 ? 0u : (0xFFFFFFFFu << (8 * a));
    return below_b & from_a;
}
__device__ __forceinline__ void mask_chunk(uint4& v, int lo, int hi) {
    v.x &= keep_mask4(lo, hi, 0);
    v.y &= keep_mask4(lo, hi, 4);
    v.z &= keep_mask4(lo, hi, 8);
    v.w &= keep_mask4(lo, hi, 12);
}

// e4m3fnuz byte -> e4m3fn byte of the same value (four bytes at a time).
__device__ __forceinline__ uint32_t fnuz_to_fn4(uint32_t w) {
    const uint32_t sign = w & 0x80808080u;
    const uint32_t ge2 = ((w & 0x70707070u) + 0x70707070u) & 0x80808080u;  // exponent >= 2
    const uint32_t m8 = (ge2 >> 7) * 0xFFu;
    const uint32_t normal = w - (0x08080808u & m8);
    const uint32_t v = w & 0x0F0F0F0Fu;                  // 8*e + m for e <= 1
    const uint32_t half = (v >> 1) & 0x07070707u;
    const uint32_t rnd = v & (v >> 1) & 0x01010101u;     // odd v with odd v>>1: round up to even
    const uint32_t small = (half + rnd) | sign;
    return (normal & m8) | (small & ~m8);
}
__device__ __forceinline__ void fnuz_to_fn(uint4& v) {
    v.x = fnuz_to_fn4(v.x);
    v.y = fnuz_to_fn4(v.y);
    v.z = fnuz_to_fn4(v.z);
    v.w = fnuz_to_fn4(v.w);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ int lds_off(int r, int ch) { return r * GB_K + ((ch ^ (r & 7)) << 4); }

template <int FMT, int MODE, bool MX>
__global__ __launch_bounds__(256, 2) void grouped_gemm_kernel(
    const uint8_t* __restrict__ a, int64_t lda, const float* __restrict__ a_scales,
    const uint8_t* __restrict__ a_e8, int64_t ld_sa, const uint8_t* __restrict__ b, int64_t ldb,
    int64_t bgs, const float* __restrict__ b_scales, const uint8_t* __restrict__ b_e8,
    int64_t ld_sb, int64_t sbgs, const int32_t* __restrict__ offsets, int G, int64_t M,
    int64_t N, int64_t K, uint16_t* __restrict__ c, int64_t ldc) {
    __shared__ __align__(16) uint8_t smem[2][2][GB_M * GB_K];
    __shared__ int s_scan[256];
    __shared__ int s_info[2];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6, wm = wave >> 1, wn = wave & 1;

    int g;
    int64_t row_lo, row_hi, kb_lo, kb_hi, kstart;
    const int64_t n0 = (int64_t)blockIdx.y * GB_N;
    if (MODE == MODE_FWD) {
        const int slot = blockIdx.x;
        if (t == 0) s_info[0] = -1;
        int base = 0;
        for (int g0 = 0; g0 < G; g0 += 256) {
            const int gg = g0 + t;
            int cnt = 0;
            if (gg < G) {
                int64_t lo = gg == 0 ? 0 : (int64_t)offsets[gg - 1];
                lo = lo < 0 ? 0 : (lo > M ? M : lo);
                int64_t hi = offsets[gg];
                hi = hi < lo ? lo : (hi > M ? M : hi);
                cnt = (int)((hi - lo + GB_M - 1) / GB_M);
            }
            __syncthreads();
            s_scan[t] = cnt;
            __syncthreads();
            for (int off = 1; off < 256; off <<= 1) {
                const int add = t >= off ? s_scan[t - off] : 0;
                __syncthreads();
                s_scan[t] += add;
                __syncthreads();
            }
            const int incl = s_scan[t];
            if (cnt > 0 && slot >= base + incl - cnt && slot < base + incl) {
                s_info[0] = gg;
                s_info[1] = slot - (base + incl - cnt);
            }
            base += s_scan[255];
        }
        __syncthreads();
        g = s_info[0];
        if (g < 0) return;  // surplus slot (block-uniform)
        int64_t glo = g == 0 ? 0 : (int64_t)offsets[g - 1];
        glo = glo < 0 ? 0 : (glo > M ? M : glo);
        int64_t ghi = offsets[g];
        ghi = ghi < glo ? glo : (ghi > M ? M : ghi);
        row_lo = glo + (int64_t)s_info[1] * GB_M;
        row_hi = row_lo + GB_M < ghi ? row_lo + GB_M : ghi;
        kb_lo = 0;
        kb_hi = K;
        kstart = 0;
    } else {
        g = blockIdx.z;
        row_lo = (int64_t)blockIdx.x * GB_M;
        row_hi = row_lo + GB_M < K ? row_lo + GB_M : K;
        int64_t glo = g == 0 ? 0 : (int64_t)offsets[g - 1];
        glo = glo < 0 ? 0 : (glo > M ? M : glo);
        int64_t ghi = offsets[g];
        ghi = ghi < glo ? glo : (ghi > M ? M : ghi);
        kb_lo = glo;
        kb_hi = ghi;
        kstart = glo & ~(int64_t)15;
    }
    const int64_t nk = kb_hi > kstart ? (kb_hi - kstart + GB_K - 1) / GB_K : 0;
    const uint8_t* bbase = MODE == MODE_FWD ? b + (int64_t)g * bgs : b;

    v4f_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) acc[i][j] = v4f_t{0.0f, 0.0f, 0.0f, 0.0f};

    uint4 ra[4], rb[4];
    int sa_cur[4], sb_cur[4], sa_nxt[4], sb_nxt[4];
#pragma unroll
    for (int i = 0; i < 4; i++) sa_cur[i] = sb_cur[i] = sa_nxt[i] = sb_nxt[i] = 127;

    auto gload = [&](int64_t kpos) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int id = t + 256 * i, r = id >> 3, ch = id & 7;
            const int64_t p = kpos + 16 * ch;
            const bool kin = p < kb_hi && p + 16 > kb_lo;
            const bool edge = p < kb_lo || p + 16 > kb_hi;
            const int64_t ar = row_lo + r;
            uint4 va = make_uint4(0, 0, 0, 0);
            if (kin && ar < row_hi) {
                va = *reinterpret_cast<const uint4*>(a + ar * lda + p);
                if (edge) mask_chunk(va, (int)(kb_lo - p), (int)(kb_hi - p));
                if (FMT == FP8Q_E4M3FNUZ) fnuz_to_fn(va);
            }
            ra[i] = va;
            const int64_t bn = n0 + r;
            uint4 vb = make_uint4(0, 0, 0, 0);
            if (kin && bn < N) {
                vb = *reinterpret_cast<const uint4*>(bbase + bn * ldb + p);
                if (edge) mask_chunk(vb, (int)(kb_lo - p), (int)(kb_hi - p));
                if (FMT == FP8Q_E4M3FNUZ) fnuz_to_fn(vb);
            }
            rb[i] = vb;
        }
        if (MX) {
            const int64_t kb = kpos / 32 + (lane >> 4);
            const bool kbin = kpos + 32 * (lane >> 4) < K;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int64_t ar = row_lo + wm * 64 + i * 16 + (lane & 15);
                sa_nxt[i] = (kbin && ar < row_hi) ? (int)a_e8[ar * ld_sa + kb] : 127;
                const int64_t bn = n0 + wn * 64 + i * 16 + (lane & 15);
                sb_nxt[i] = (kbin && bn < N) ? (int)b_e8[(int64_t)g * sbgs + bn * ld_sb + kb] : 127;
            }
        }
    };
    auto sstore = [&](int stage) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int id = t + 256 * i, r = id >> 3, ch = id & 7;
            *reinterpret_cast<uint4*>(&smem[stage][0][lds_off(r, ch)]) = ra[i];
            *reinterpret_cast<uint4*>(&smem[stage][1][lds_off(r, ch)]) = rb[i];
        }
    };

    if (nk > 0) {
        gload(kstart);
        sstore(0);
    }
    for (int64_t kk = 0; kk < nk; kk++) {
        const int cur = (int)(kk & 1);
        if (MX) {
#pragma unroll
            for (int i = 0; i < 4; i++) { sa_cur[i] = sa_nxt[i]; sb_cur[i] = sb_nxt[i]; }
        }
        if (kk + 1 < nk) gload(kstart + (kk + 1) * GB_K);
        __syncthreads();
        const uint8_t* As = smem[cur][0];
        const uint8_t* Bs = smem[cur][1];
        const int kg = lane >> 4;
        v8i_t af[4], bfr[4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int ra_ = wm * 64 + i * 16 + (lane & 15);
            const uint4 lo = *reinterpret_cast<const uint4*>(&As[lds_off(ra_, kg)]);
            const uint4 hi = *reinterpret_cast<const uint4*>(&As[lds_off(ra_, 4 + kg)]);
            af[i] = v8i_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                          (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            const int rb_ = wn * 64 + i * 16 + (lane & 15);
            const uint4 blo = *reinterpret_cast<const uint4*>(&Bs[lds_off(rb_, kg)]);
            const uint4 bhi = *reinterpret_cast<const uint4*>(&Bs[lds_off(rb_, 4 + kg)]);
            bfr[i] = v8i_t{(int)blo.x, (int)blo.y, (int)blo.z, (int)blo.w,
                           (int)bhi.x, (int)bhi.y, (int)bhi.z, (int)bhi.w};
        }
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
            for (int j = 0; j < 4; j++) {
                if (MX)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        af[i], bfr[j], acc[i][j], 0, 0, 0, sa_cur[i], 0, sb_cur[j]);
                else
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        af[i], bfr[j], acc[i][j], 0, 0, 0, 0, 0, 0);
            }
        if (kk + 1 < nk) sstore(cur ^ 1);
    }

    // Epilogue: dequantize (multiply by the reciprocal scales) and round to bf16.
    float csc[4];
    int64_t gn[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
        gn[j] = n0 + wn * 64 + j * 16 + (lane & 15);
        csc[j] = 1.0f;
        if (!MX && gn[j] < N) csc[j] = 1.0f / b_scales[(int64_t)g * N + gn[j]];
    }
#pragma unroll
    for (int i = 0; i < 4; i++) {
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const int64_t gm = row_lo + wm * 64 + i * 16 + 4 * (lane >> 4) + e;
            if (gm >= row_hi) continue;
            float rsc = 1.0f;
            uint16_t* crow;
            if (MODE == MODE_FWD) {
                if (!MX) rsc = 1.0f / a_scales[gm];
                crow = c + gm * ldc;
            } else {
                rsc = 1.0f / a_scales[(int64_t)g * K + gm];
                crow = c + ((int64_t)g * K + gm) * ldc;
            }
#pragma unroll
            for (int j = 0; j < 4; j++)
                if (gn[j] < N) crow[gn[j]] = f32_to_bf16_rne(acc[i][j][e] * rsc * csc[j]);
        }
    }
}

template <int FMT, int MODE, bool MX>
static fp8q_status_t launch_gemm(const uint8_t* a, int64_t lda, const float* sa,
                                 const uint8_t* a_e8, int64_t ld_sa, const uint8_t* b,
                                 int64_t ldb, int64_t bgs, const float* sb, const uint8_t* b_e8,
                                 int64_t ld_sb, int64_t sbgs, const int32_t* offsets, int G,
                                 int64_t M, int64_t N, int64_t K, uint16_t* c, int64_t ldc,
                                 hipStream_t stream) {
    dim3 grid;
    if (MODE == MODE_FWD) {
        const int64_t slots = (M + GB_M - 1) / GB_M + G;
        const int64_t nt = (N + GB_N - 1) / GB_N;
        if (slots > 0x7FFFFFFFLL || nt > 65535) return FP8Q_ERR_UNSUPPORTED;
        grid = dim3((unsigned)slots, (unsigned)nt, 1);
    } else {
        const int64_t kt = (K + GB_M - 1) / GB_M;
        const int64_t nt = (N + GB_N - 1) / GB_N;
        if (kt > 0x7FFFFFFFLL || nt > 65535 || G > 65535) return FP8Q_ERR_UNSUPPORTED;
        grid = dim3((unsigned)kt, (unsigned)nt, (unsigned)G);
    }
    grouped_gemm_kernel<FMT, MODE, MX><<<grid, dim3(256), 0, stream>>>(
        a, lda, sa, a_e8, ld_sa, b, ldb, bgs, sb, b_e8, ld_sb, sbgs, offsets, G, M, N, K, c, ldc);
    FP8Q_CHECK_LAUNCH();
    return FP8Q_OK;
}

}  // namespace fp8q

extern "C" fp8q_status_t fp8_grouped_gemm(fp8q_gemm_mode_t mode, fp8q_format_t fmt,
                                          const uint8_t* a, int64_t lda, const float* a_scales,
                                          const uint8_t* b, int64_t ldb, int64_t b_group_stride,
                                          const float* b_scales, const int32_t* offsets,
                                          int32_t groups, int64_t M, int64_t N, int64_t K,
                                          uint16_t* c, int64_t ldc, hipStream_t stream) {
    using namespace fp8q;
    if (!fp8q_fmt_ok(fmt) || groups < 1 || M < 0 || N < 0 || K < 0 || ldc < N || !offsets)
        return FP8Q_ERR_INVALID_ARG;
    if (mode == FP8Q_GEMM_FWD_MGROUPED) {
        if (lda < K || ldb < K || b_group_stride < 0) return FP8Q_ERR_INVALID_ARG;
        if (M == 0 || N == 0) return FP8Q_OK;
        if (!a || !b || !a_scales || !b_scales || !c) return FP8Q_ERR_INVALID_ARG;
        if (K % 16 || lda % 16 || ldb % 16 || b_group_stride % 16 || !fp8q_aligned(a, 16) ||
            !fp8q_aligned(b, 16))
            return FP8Q_ERR_UNSUPPORTED;
        if (fmt == FP8Q_E4M3FN)
            return launch_gemm<FP8Q_E4M3FN, MODE_FWD, false>(a, lda, a_scales, nullptr, 0, b, ldb,
                                                           b_group_stride, b_scales, nullptr, 0,
                                                           0, offsets, groups, M, N, K, c, ldc,
                                                           stream);
        return launch_gemm<FP8Q_E4M3FNUZ, MODE_FWD, false>(a, lda, a_scales, nullptr, 0, b, ldb,
                                                         b_group_stride, b_scales, nullptr, 0, 0,
                                                         offsets, groups, M, N, K, c, ldc, stream);
    }
    if (mode == FP8Q_GEMM_WGRAD_KGROUPED) {
        if (lda < M || ldb < M || b_group_stride != 0) return FP8Q_ERR_INVALID_ARG;
        if (K == 0 || N == 0) return FP8Q_OK;
        if (!a_scales || !b_scales || !c || (M > 0 && (!a || !b))) return FP8Q_ERR_INVALID_ARG;
        if (lda % 16 || ldb % 16 || !fp8q_aligned(a, 16) || !fp8q_aligned(b, 16))
            return FP8Q_ERR_UNSUPPORTED;
        if (fmt == FP8Q_E4M3FN)
            return launch_gemm<FP8Q_E4M3FN, MODE_WGRAD, false>(a, lda, a_scales, nullptr, 0, b,
                                                             ldb, 0, b_scales, nullptr, 0, 0,
                                                             offsets, groups, M, N, K, c, ldc,
                                                             stream);
        return launch_gemm<FP8Q_E4M3FNUZ, MODE_WGRAD, false>(a, lda, a_scales, nullptr, 0, b, ldb,
                                                           0, b_scales, nullptr, 0, 0, offsets,
                                                           groups, M, N, K, c, ldc, stream);
    }
    return FP8Q_ERR_INVALID_ARG;
}

extern "C" fp8q_status_t fp8_mx_grouped_gemm(const uint8_t* a, int64_t lda, const uint8_t* a_e8m0,
                                             int64_t ld_sa, const uint8_t* b, int64_t ldb,
                                             int64_t b_group_stride, const uint8_t* b_e8m0,
                                             int64_t ld_sb, int64_t sb_group_stride,
                                             const int32_t* offsets, int32_t groups, int64_t M,
                                             int64_t N, int64_t K, uint16_t* c, int64_t ldc,
                                             hipStream_t stream) {
    using namespace fp8q;
    if (groups < 1 || M < 0 || N < 0 || K < 0 || ldc < N || !offsets || lda < K || ldb < K ||
        b_group_stride < 0 || sb_group_stride < 0 || ld_sa < K / 32 || ld_sb < K / 32)
        return FP8Q_ERR_INVALID_ARG;
    if (K % 32) return FP8Q_ERR_INVALID_ARG;
    if (M == 0 || N == 0) return FP8Q_OK;
    if (!a || !b || !a_e8m0 || !b_e8m0 || !c) return FP8Q_ERR_INVALID_ARG;
    if (lda % 16 || ldb % 16 || b_group_stride % 16 || !fp8q_aligned(a, 16) ||
        !fp8q_aligned(b, 16))
        return FP8Q_ERR_UNSUPPORTED;
    return launch_gemm<FP8Q_E4M3FN, MODE_FWD, true>(a, lda, nullptr, a_e8m0, ld_sa, b, ldb,
                                                   b_group_stride, nullptr, b_e8m0, ld_sb,
                                                   sb_group_stride, offsets, groups, M, N, K, c,
                                                   ldc, stream);
}
