// MXFP8 quantization (fosswire.org "AMD Primus adds FP8/MXFP8 kernels ...", section "What
// Primus adds for MoE training on MI355X" names MXFP8 grouped GEMM and quantization kernels; the
// format is the OCP Microscaling Formats v1.0 one): 32 consecutive elements share an E8M0
// scale 2^e with e = floor(log2 amax) - 8 (8 = exponent of e4m3fn's largest value 448),
// clamped to [-127, 127] (-127 for an all-zero block); elements are x * 2^-e clamped to +-448
// and rounded to nearest-even OCP e4m3fn.
//
// floor(log2 amax) of a bf16 amax is read off its exponent field E (bf16 subnormals and zero
// give E = 0 and fall under the -127 clamp), so the E8M0 byte is max(E - 8, 0) and the element
// multiplier 2^-e is built from bits: no log, no division.  x * 2^-e is exact.
#include "common.hpp"

namespace fp8q {

__device__ __forceinline__ float mx_inv_scale(uint32_t e8) {  // 2^-(e8 - 127), e8 in [0, 246]
    return __uint_as_float((uint32_t)(254 - (int)e8) << 23);
}

// Rowwise: 256 threads cover 2048 consecutive elements of one row per pass; each lane holds a
// 16-byte chunk (8 bf16), four neighbouring lanes form one 32-element block (two shuffles for
// its absmax), and each lane stores its 8 output bytes (consecutive lanes -> consecutive bytes).
__global__ __launch_bounds__(256) void mx_rowwise_kernel(const uint16_t* __restrict__ x,
                                                         int64_t cols, int64_t ld_x,
                                                         uint8_t* __restrict__ q, int64_t ld_q,
                                                         uint8_t* __restrict__ e8,
                                                         int64_t ld_s) {
    const int64_t row = blockIdx.y;
    const int64_t nch = cols >> 3;
    const uint16_t* xr = x + row * ld_x;
    constexpr int NV = 4;
    uint4 v[NV];
#pragma unroll
    for (int j = 0; j < NV; j++) {
        const int64_t ch = (int64_t)blockIdx.x * 256 * NV + threadIdx.x + 256 * j;
        v[j] = ch < nch ? ld_nt16(reinterpret_cast<const uint4*>(xr) + ch)
                        : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < NV; j++) {
        const int64_t ch = (int64_t)blockIdx.x * 256 * NV + threadIdx.x + 256 * j;
        uint32_t m = pk_max_u16(pk_max_u16(mag2(v[j].x), mag2(v[j].y)),
                                pk_max_u16(mag2(v[j].z), mag2(v[j].w)));
        m = pk_max_u16(m, (uint32_t)__shfl_xor((int)m, 1, 64));
        m = pk_max_u16(m, (uint32_t)__shfl_xor((int)m, 2, 64));
        const uint32_t amax = hmax16(m);
        const int E = (int)(amax >> 7);
        const uint32_t eb = E > 8 ? (uint32_t)(E - 8) : 0u;
        const float inv = mx_inv_scale(eb);
        if (ch < nch) {
            const uint32_t w0 = enc4<FP8Q_E4M3FN>(bf16_lo(v[j].x) * inv, bf16_hi(v[j].x) * inv,
                                                  bf16_lo(v[j].y) * inv, bf16_hi(v[j].y) * inv);
            const uint32_t w1 = enc4<FP8Q_E4M3FN>(bf16_lo(v[j].z) * inv, bf16_hi(v[j].z) * inv,
                                                  bf16_lo(v[j].w) * inv, bf16_hi(v[j].w) * inv);
            st_nt8(q + row * ld_q + ch * 8, w0, w1);  // streaming: measured faster
            if ((threadIdx.x & 3) == 0) e8[row * ld_s + (ch >> 2)] = (uint8_t)eb;
        }
    }
}

// Columnwise with transposed output: 256x64 tiles; a lane holds 8 rows x 8 columns, four lanes
// with consecutive row octets (lane bits 3-4) form a 32-row block; bytes are encoded along rows,
// transposed through LDS and written as 16-byte chunks of the column-major output.
constexpr int MXC_TR = 256, MXC_TC = 64, MXC_STR = MXC_TR + 16;
// (transposed tile layout with the column-octet XOR swizzle of quant_colwise.hip's tiles)

__global__ __launch_bounds__(256) void mx_colwise_kernel(const uint16_t* __restrict__ x,
                                                         int64_t R, int64_t C, int64_t ld_x,
                                                         uint8_t* __restrict__ qt, int64_t ld_qt,
                                                         uint8_t* __restrict__ e8, int64_t ld_s,
                                                         bool vec_out, bool nt_out, bool vec_e8) {
    const int t = threadIdx.x, o = t & 7, qd = t >> 3;
    const int64_t r0 = (int64_t)blockIdx.x * MXC_TR, c0 = (int64_t)blockIdx.y * MXC_TC;
    __shared__ __align__(16) uint8_t tile[MXC_TC * MXC_STR];
    __shared__ __align__(8) uint8_t se8[MXC_TC * 8];  // [column][32-row block] of this tile
    const int64_t c = c0 + 8 * o;
    uint4 v[8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const int64_t r = r0 + 8 * qd + i;
        v[i] = (r < R && c < C) ? ld_nt16(reinterpret_cast<const uint4*>(x + r * ld_x + c))
                                : make_uint4(0, 0, 0, 0);  // read once: streaming loads
    }
    uint32_t m[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; i++) {
        m[0] = pk_max_u16(m[0], mag2(v[i].x));
        m[1] = pk_max_u16(m[1], mag2(v[i].y));
        m[2] = pk_max_u16(m[2], mag2(v[i].z));
        m[3] = pk_max_u16(m[3], mag2(v[i].w));
    }
#pragma unroll
    for (int d = 0; d < 4; d++) {
        m[d] = pk_max_u16(m[d], (uint32_t)__shfl_xor((int)m[d], 8, 64));
        m[d] = pk_max_u16(m[d], (uint32_t)__shfl_xor((int)m[d], 16, 64));
    }
    uint32_t eb[8];
    float inv[8];
#pragma unroll
    for (int d = 0; d < 4; d++) {
        const int Elo = (int)((m[d] & 0xFFFFu) >> 7), Ehi = (int)((m[d] >> 16) >> 7);
        eb[2 * d] = Elo > 8 ? (uint32_t)(Elo - 8) : 0u;
        eb[2 * d + 1] = Ehi > 8 ? (uint32_t)(Ehi - 8) : 0u;
        inv[2 * d] = mx_inv_scale(eb[2 * d]);
        inv[2 * d + 1] = mx_inv_scale(eb[2 * d + 1]);
    }
    // the block's E8M0 bytes go to LDS and leave as one 8-byte piece per column (a column's 8
    // blocks of this tile are consecutive in its scale row) instead of 8 scattered byte stores
    // per lane
    if ((qd & 3) == 0) {
#pragma unroll
        for (int j = 0; j < 8; j++) se8[(8 * o + j) * 8 + (qd >> 2)] = (uint8_t)eb[j];
    }
#pragma unroll
    for (int j = 0; j < 8; j++) {
        float y[8];
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const uint32_t w = j < 2 ? v[i].x : j < 4 ? v[i].y : j < 6 ? v[i].z : v[i].w;
            y[i] = ((j & 1) ? bf16_hi(w) : bf16_lo(w)) * inv[j];
        }
        const uint32_t w0 = enc4<FP8Q_E4M3FN>(y[0], y[1], y[2], y[3]);
        const uint32_t w1 = enc4<FP8Q_E4M3FN>(y[4], y[5], y[6], y[7]);
        *reinterpret_cast<uint2*>(&tile[(8 * o + j) * MXC_STR + 8 * (qd ^ (2 * o))]) = make_uint2(w0, w1);
    }
    __syncthreads();
    if (t < MXC_TC && c0 + t < C) {
        const int nb = R - r0 < MXC_TR ? (int)((R - r0) / 32) : MXC_TR / 32;  // R % 32 == 0
        uint8_t* dst = e8 + (c0 + t) * ld_s + r0 / 32;
        if (vec_e8 && nb == MXC_TR / 32) {
            *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(&se8[t * 8]);
        } else {
            for (int b = 0; b < nb; b++) dst[b] = se8[t * 8 + b];
        }
    }
#pragma unroll
    for (int k = 0; k < 4; k++) {
        const int ch = t + 256 * k;
        const int col = ch >> 4, seg = ch & 15;
        const int64_t cc = c0 + col, r = r0 + 16 * seg;
        if (cc >= C || r >= R) continue;
        const uint8_t* src = &tile[col * MXC_STR + 16 * (seg ^ ((col >> 3) & 7))];
        uint8_t* dst = qt + cc * ld_qt + r;
        if (vec_out && r + 16 <= R) {
            if (nt_out) st_nt16(dst, *reinterpret_cast<const uint4*>(src));  // block-uniform
            else *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
        } else {
            for (int bb = 0; bb < 16; bb++)
                if (r + bb < R) dst[bb] = src[bb];
        }
    }
}

}  // namespace fp8q

extern "C" fp8q_status_t fp8_mx_quant_rowwise(const uint16_t* x, int64_t rows, int64_t cols,
                                              int64_t ld_x, uint8_t* q, int64_t ld_q,
                                              uint8_t* e8m0, int64_t ld_s, hipStream_t stream) {
    if (rows < 0 || cols < 0 || cols % 32 || ld_x < cols || ld_q < cols || ld_s < cols / 32)
        return FP8Q_ERR_INVALID_ARG;
    if (rows == 0 || cols == 0) return FP8Q_OK;
    if (!x || !q || !e8m0) return FP8Q_ERR_INVALID_ARG;
    if (ld_x % 8 || ld_q % 8 || !fp8q_aligned(x, 16) || !fp8q_aligned(q, 8))
        return FP8Q_ERR_UNSUPPORTED;
    const int64_t spans = (cols / 8 + 1023) / 1024;
    if (rows > 65535 * 1024LL || spans > 0x7FFFFFFFLL) return FP8Q_ERR_UNSUPPORTED;
    // grid.y is limited to 65535: fold extra rows into repeated launches over row slices
    for (int64_t r0 = 0; r0 < rows; r0 += 65535) {
        const int64_t nr = rows - r0 < 65535 ? rows - r0 : 65535;
        fp8q::mx_rowwise_kernel<<<dim3((unsigned)spans, (unsigned)nr), dim3(256), 0, stream>>>(
            x + r0 * ld_x, cols, ld_x, q + r0 * ld_q, ld_q, e8m0 + r0 * ld_s, ld_s);
    }
    FP8Q_CHECK_LAUNCH();
    return FP8Q_OK;
}

extern "C" fp8q_status_t fp8_mx_quant_colwise(const uint16_t* x, int64_t rows, int64_t cols,
                                              int64_t ld_x, uint8_t* q_t, int64_t ld_qt,
                                              uint8_t* e8m0, int64_t ld_s, hipStream_t stream) {
    if (rows < 0 || cols < 0 || rows % 32 || ld_x < cols || ld_qt < rows || ld_s < rows / 32)
        return FP8Q_ERR_INVALID_ARG;
    if (rows == 0 || cols == 0) return FP8Q_OK;
    if (!x || !q_t || !e8m0) return FP8Q_ERR_INVALID_ARG;
    if (cols % 8 || ld_x % 8 || !fp8q_aligned(x, 16)) return FP8Q_ERR_UNSUPPORTED;
    const int64_t rt = (rows + fp8q::MXC_TR - 1) / fp8q::MXC_TR;
    const int64_t ct = (cols + fp8q::MXC_TC - 1) / fp8q::MXC_TC;
    if (rt > 0x7FFFFFFFLL || ct > 65535) return FP8Q_ERR_UNSUPPORTED;
    const bool vec_out = (ld_qt % 16 == 0) && fp8q_aligned(q_t, 16);
    const bool vec_e8 = (ld_s % 8 == 0) && fp8q_aligned(e8m0, 8);  // tiles start at 8-block steps
    fp8q::mx_colwise_kernel<<<dim3((unsigned)rt, (unsigned)ct), dim3(256), 0, stream>>>(
        x, rows, cols, ld_x, q_t, ld_qt, e8m0, ld_s, vec_out,
        (double)cols * (double)ld_qt > fp8q::kStreamBytes, vec_e8);
    FP8Q_CHECK_LAUNCH();
    return FP8Q_OK;
}
