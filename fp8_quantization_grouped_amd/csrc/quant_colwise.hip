// Columnwise FP8 quantization per row group, written transposed (column-major).
//
// What it computes (ai-radar.it "FP8 su GPU AMD ...", introduction: columnwise scales on the
// per-expert weights and an offset tensor routing token rows to experts; section "Il guadagno
// vero e' nel movimento dei dati": the backward's transposed operand is written directly, not
// through a .t().contiguous() copy; the output tile is transposed through LDS before the store
// so that consecutive lanes write consecutive addresses; cross-block maxima use relaxed-order
// atomics because a max is a commutative reduction):
//   for group g (rows [o[g-1], o[g])) and column c:
//     s[g,c] = FMAX / max(amax_g(c), 1e-12f);   q_t[c, r] = ENC(clamp(RN32(x[r,c] * s[g,c])))
//
// gfx950 design.  A column's absmax needs every row of its group before any element can be
// cast, and a group can span thousands of rows, so the work is two passes over 256x64 tiles:
//   1. colwise_amax_kernel: each block loads a 256-row x 64-column tile (8 rows x 8 columns per
//      lane, 16-byte loads, 128 contiguous bytes per row), reduces each group segment of the
//      tile to 64 column maxima (packed 16-bit max on bf16 magnitude bits, lane shuffles, then
//      LDS across the 4 waves) and publishes them with relaxed device-scope atomicMax on the
//      bf16 magnitude bits (exact: for finite values their integer order is the value order).
//   2. colwise_cast_kernel: reloads the tile, turns the finished maxima into scales (per group
//      in LDS), scales/clamps/converts along rows so each lane holds 8 consecutive output
//      bytes of each of its 8 columns, transposes through LDS and writes 16-byte chunks of
//      the column-major output (16 lanes cover one column's 256 contiguous bytes).
// The block whose tile contains a group's first row writes that group's scales; the last row
// tile also writes groups that start at the end (trailing empty groups).
#include "common.hpp"

namespace fp8q {

constexpr int CW_TR = 256;              // tile rows
constexpr int CW_TC = 64;               // tile columns
constexpr int CW_STR = CW_TR + 16;      // LDS bytes per transposed column (16-byte aligned)
constexpr int CW_GB = 8;                // groups per scale batch in LDS

// The lane's 8x8 block: rows r0 + 8*qd + i (i < 8), columns c0 + 8*o .. +7, as bf16 bits
// packed two per dword (column 2d in the low half of dword d).  Out-of-range elements are 0.
template <bool VEC>
__device__ __forceinline__ void cw_load(const uint16_t* __restrict__ x, int64_t R, int64_t C,
                                        int64_t ld_x, int64_t r0, int64_t c0, int o, int qd,
                                        uint4 v[8]) {
    const int64_t c = c0 + 8 * o;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const int64_t r = r0 + 8 * qd + i;
        if (VEC) {
            v[i] = (r < R && c < C) ? *reinterpret_cast<const uint4*>(x + r * ld_x + c)
                                    : make_uint4(0, 0, 0, 0);
        } else {
            uint32_t e[8];
#pragma unroll
            for (int j = 0; j < 8; j++) e[j] = (r < R && c + j < C) ? x[r * ld_x + c + j] : 0u;
            v[i] = make_uint4(e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16),
                              e[6] | (e[7] << 16));
        }
    }
}

__global__ void cw_zero_kernel(uint32_t* __restrict__ p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        p[i] = 0u;
}

template <bool VEC>
__global__ __launch_bounds__(256) void colwise_amax_kernel(const uint16_t* __restrict__ x,
                                                           int64_t R, int64_t C, int64_t ld_x,
                                                           const int32_t* __restrict__ offsets,
                                                           int G, uint32_t* __restrict__ amax) {
    const int t = threadIdx.x, o = t & 7, qd = t >> 3, lane = t & 63, wave = t >> 6;
    const int64_t r0 = (int64_t)blockIdx.x * CW_TR, c0 = (int64_t)blockIdx.y * CW_TC;
    uint4 v[8];
    cw_load<VEC>(x, R, C, ld_x, r0, c0, o, qd, v);
    const int64_t r_end = r0 + CW_TR < R ? r0 + CW_TR : R;
    const int g_first = group_of_row(offsets, G, r0);
    const int g_last = group_of_row(offsets, G, r_end - 1);
    __shared__ uint32_t red[4][8][4];
    for (int g = g_first; g <= g_last; g++) {
        int64_t gs = group_start(offsets, g);
        int64_t ge = g == G - 1 ? r_end : (int64_t)offsets[g];
        gs = gs > r0 ? gs : r0;
        ge = ge < r_end ? ge : r_end;
        if (gs >= ge) continue;  // block-uniform
        uint32_t m0 = 0, m1 = 0, m2 = 0, m3 = 0;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const int64_t r = r0 + 8 * qd + i;
            if (r >= gs && r < ge) {
                m0 = pk_max_u16(m0, mag2(v[i].x));
                m1 = pk_max_u16(m1, mag2(v[i].y));
                m2 = pk_max_u16(m2, mag2(v[i].z));
                m3 = pk_max_u16(m3, mag2(v[i].w));
            }
        }
#pragma unroll
        for (int off = 8; off < 64; off <<= 1) {
            m0 = pk_max_u16(m0, (uint32_t)__shfl_xor((int)m0, off, 64));
            m1 = pk_max_u16(m1, (uint32_t)__shfl_xor((int)m1, off, 64));
            m2 = pk_max_u16(m2, (uint32_t)__shfl_xor((int)m2, off, 64));
            m3 = pk_max_u16(m3, (uint32_t)__shfl_xor((int)m3, off, 64));
        }
        if (lane < 8) {
            red[wave][lane][0] = m0;
            red[wave][lane][1] = m1;
            red[wave][lane][2] = m2;
            red[wave][lane][3] = m3;
        }
        __syncthreads();
        if (t < 32) {
            const int oo = t >> 2, d = t & 3;
            uint32_t mm = pk_max_u16(pk_max_u16(red[0][oo][d], red[1][oo][d]),
                                     pk_max_u16(red[2][oo][d], red[3][oo][d]));
            const int64_t c = c0 + 8 * oo + 2 * d;
            uint32_t lo = mm & 0xFFFFu, hi = mm >> 16;
            uint32_t* dst = amax + (int64_t)g * C + c;
            if (lo && c < C) __hip_atomic_fetch_max(dst, lo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (hi && c + 1 < C) __hip_atomic_fetch_max(dst + 1, hi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
    }
}

// First group whose start row is >= r (G if none); starts are taken as stored.
__device__ __forceinline__ int first_group_starting_at(const int32_t* __restrict__ offsets, int G,
                                                       int64_t r) {
    int lo = 0, hi = G;
    while (lo < hi) {
        int mid = (lo + hi) >> 1;
        if (group_start(offsets, mid) >= r) hi = mid; else lo = mid + 1;
    }
    return lo;
}

template <int FMT, bool VEC, bool VEC_OUT>
__global__ __launch_bounds__(256) void colwise_cast_kernel(
    const uint16_t* __restrict__ x, int64_t R, int64_t C, int64_t ld_x,
    const int32_t* __restrict__ offsets, int G, const uint32_t* __restrict__ amax,
    uint8_t* __restrict__ qt, int64_t ld_qt, float* __restrict__ scales) {
    const int t = threadIdx.x, o = t & 7, qd = t >> 3;
    const int64_t r0 = (int64_t)blockIdx.x * CW_TR, c0 = (int64_t)blockIdx.y * CW_TC;
    __shared__ __align__(16) float sc[CW_GB][CW_TC];
    __shared__ __align__(16) uint8_t tile[CW_TC * CW_STR];

    // Scales of the groups this tile owns (first row inside the tile; the last tile also owns
    // groups starting at or after its end, i.e. trailing empty groups).
    {
        const bool last_tile = r0 + CW_TR >= R;
        int g = first_group_starting_at(offsets, G, r0);
        for (; g < G; g++) {
            if (!last_tile && group_start(offsets, g) >= r0 + CW_TR) break;
            if (t < CW_TC && c0 + t < C) {
                const int64_t idx = (int64_t)g * C + c0 + t;
                scales[idx] = scale_from_amax<FMT>(__uint_as_float(amax[idx] << 16));
            }
        }
    }
    if (r0 >= R) return;  // only the R == 0 launch has such a block (block-uniform)

    uint4 v[8];
    cw_load<VEC>(x, R, C, ld_x, r0, c0, o, qd, v);
    const int64_t r_end = r0 + CW_TR < R ? r0 + CW_TR : R;
    const int g_first = group_of_row(offsets, G, r0);
    const int g_last = group_of_row(offsets, G, r_end - 1);
    // group of each of the lane's rows (-1 past the end)
    int gid[8];
    {
        int g = group_of_row(offsets, G, r0 + 8 * qd);
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const int64_t r = r0 + 8 * qd + i;
            while (g < G - 1 && (int64_t)offsets[g] <= r) g++;
            gid[i] = r < r_end ? g : -1;
        }
    }
    float y[8][8];
#pragma unroll
    for (int i = 0; i < 8; i++)
#pragma unroll
        for (int j = 0; j < 8; j++) y[i][j] = 0.0f;

    for (int gb = g_first; gb <= g_last; gb += CW_GB) {
        __syncthreads();  // previous batch finished reading sc
        for (int idx = t; idx < CW_GB * CW_TC; idx += 256) {
            const int k = idx / CW_TC, cc = idx % CW_TC;
            const int g = gb + k;
            float s = 0.0f;
            if (g <= g_last && c0 + cc < C)
                s = scale_from_amax<FMT>(__uint_as_float(amax[(int64_t)g * C + c0 + cc] << 16)) *
                    Fmt<FMT>::mult;
            sc[k][cc] = s;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const int k = gid[i] - gb;
            if (k >= 0 && k < CW_GB) {
                const float4 sa = *reinterpret_cast<const float4*>(&sc[k][8 * o]);
                const float4 sb = *reinterpret_cast<const float4*>(&sc[k][8 * o + 4]);
                y[i][0] = bf16_lo(v[i].x) * sa.x;
                y[i][1] = bf16_hi(v[i].x) * sa.y;
                y[i][2] = bf16_lo(v[i].y) * sa.z;
                y[i][3] = bf16_hi(v[i].y) * sa.w;
                y[i][4] = bf16_lo(v[i].z) * sb.x;
                y[i][5] = bf16_hi(v[i].z) * sb.y;
                y[i][6] = bf16_lo(v[i].w) * sb.z;
                y[i][7] = bf16_hi(v[i].w) * sb.w;
            }
        }
    }
    // Encode along rows: column j of the lane gets the bytes of rows 8*qd .. 8*qd+7.
#pragma unroll
    for (int j = 0; j < 8; j++) {
        const uint32_t w0 = enc4<FMT>(y[0][j], y[1][j], y[2][j], y[3][j]);
        const uint32_t w1 = enc4<FMT>(y[4][j], y[5][j], y[6][j], y[7][j]);
        *reinterpret_cast<uint2*>(&tile[(8 * o + j) * CW_STR + 8 * qd]) = make_uint2(w0, w1);
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 4; k++) {
        const int ch = t + 256 * k;
        const int col = ch >> 4, seg = ch & 15;
        const int64_t c = c0 + col, r = r0 + 16 * seg;
        if (c >= C || r >= R) continue;
        const uint8_t* src = &tile[col * CW_STR + 16 * seg];
        uint8_t* dst = qt + c * ld_qt + r;
        if (VEC_OUT && r + 16 <= R) {
            *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
        } else {
            for (int b = 0; b < 16; b++)
                if (r + b < R) dst[b] = src[b];
        }
    }
}

template <int FMT, bool VEC, bool VEC_OUT>
static void launch_cast(const uint16_t* x, int64_t R, int64_t C, int64_t ld_x,
                        const int32_t* offsets, int G, const uint32_t* ws, uint8_t* qt,
                        int64_t ld_qt, float* s, hipStream_t stream) {
    const int64_t rt = R > 0 ? (R + CW_TR - 1) / CW_TR : 1;
    const int64_t ct = (C + CW_TC - 1) / CW_TC;
    colwise_cast_kernel<FMT, VEC, VEC_OUT><<<dim3((unsigned)rt, (unsigned)ct), dim3(256), 0, stream>>>(
        x, R, C, ld_x, offsets, G, ws, qt, ld_qt, s);
}

template <int FMT>
static fp8q_status_t colwise_run(const uint16_t* x, int64_t R, int64_t C, int64_t ld_x,
                                 const int32_t* offsets, int G, uint8_t* qt, int64_t ld_qt,
                                 float* s, uint32_t* ws, hipStream_t stream) {
    const bool vec = (C % 8 == 0) && (ld_x % 8 == 0) && fp8q_aligned(x, 16);
    const bool vec_out = (ld_qt % 16 == 0) && fp8q_aligned(qt, 16);
    const int64_t n = (int64_t)G * C;
    int64_t zb = (n + 255) / 256;
    if (zb > 4096) zb = 4096;
    cw_zero_kernel<<<dim3((unsigned)zb), dim3(256), 0, stream>>>(ws, n);
    if (R > 0) {
        const dim3 grid((unsigned)((R + CW_TR - 1) / CW_TR), (unsigned)((C + CW_TC - 1) / CW_TC));
        if (vec) colwise_amax_kernel<true><<<grid, dim3(256), 0, stream>>>(x, R, C, ld_x, offsets, G, ws);
        else colwise_amax_kernel<false><<<grid, dim3(256), 0, stream>>>(x, R, C, ld_x, offsets, G, ws);
    }
    if (vec && vec_out) launch_cast<FMT, true, true>(x, R, C, ld_x, offsets, G, ws, qt, ld_qt, s, stream);
    else if (vec) launch_cast<FMT, true, false>(x, R, C, ld_x, offsets, G, ws, qt, ld_qt, s, stream);
    else if (vec_out) launch_cast<FMT, false, true>(x, R, C, ld_x, offsets, G, ws, qt, ld_qt, s, stream);
    else launch_cast<FMT, false, false>(x, R, C, ld_x, offsets, G, ws, qt, ld_qt, s, stream);
    FP8Q_CHECK_LAUNCH();
    return FP8Q_OK;
}

}  // namespace fp8q

extern "C" size_t fp8_quant_colwise_grouped_workspace_size(int64_t rows, int64_t cols,
                                                           int32_t groups) {
    (void)rows;
    if (cols < 0 || groups < 1) return 0;
    const size_t b = (size_t)groups * (size_t)cols * sizeof(uint32_t);
    return (b + 255) & ~(size_t)255;
}

extern "C" fp8q_status_t fp8_quant_colwise_grouped(const uint16_t* x, int64_t rows, int64_t cols,
                                                   int64_t ld_x, const int32_t* offsets,
                                                   int32_t groups, fp8q_format_t fmt,
                                                   uint8_t* q_t, int64_t ld_qt, float* scales,
                                                   void* workspace, size_t workspace_bytes,
                                                   hipStream_t stream) {
    if (rows < 0 || cols < 0 || groups < 1 || ld_x < cols || ld_qt < rows || !fp8q_fmt_ok(fmt))
        return FP8Q_ERR_INVALID_ARG;
    if (!offsets) return FP8Q_ERR_INVALID_ARG;
    if (cols == 0) return FP8Q_OK;
    if (!scales || (rows > 0 && (!x || !q_t))) return FP8Q_ERR_INVALID_ARG;
    const size_t need = fp8_quant_colwise_grouped_workspace_size(rows, cols, groups);
    if (workspace_bytes < need || !workspace) return FP8Q_ERR_WORKSPACE;
    if ((rows + fp8q::CW_TR - 1) / fp8q::CW_TR > 0x7FFFFFFFLL ||
        (cols + fp8q::CW_TC - 1) / fp8q::CW_TC > 65535)
        return FP8Q_ERR_UNSUPPORTED;
    uint32_t* ws = static_cast<uint32_t*>(workspace);
    if (fmt == FP8Q_E4M3FN)
        return fp8q::colwise_run<FP8Q_E4M3FN>(x, rows, cols, ld_x, offsets, groups, q_t, ld_qt,
                                              scales, ws, stream);
    return fp8q::colwise_run<FP8Q_E4M3FNUZ>(x, rows, cols, ld_x, offsets, groups, q_t, ld_qt,
                                            scales, ws, stream);
}
