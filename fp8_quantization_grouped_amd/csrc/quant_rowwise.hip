// Rowwise FP8 quantization of activations: per row absmax -> scale -> clamp -> cast in ONE
// pass over HBM (ai-radar.it "FP8 su GPU AMD ...": introduction, rowwise scales on the
// activations; section "Il guadagno vero e' nel movimento dei dati", the chain absmax, scale,
// clamp, cast, whose separate kernels each round-tripped HBM).
//
// gfx950 design: each row is owned by WPR wavefronts; every lane loads NV 16-byte chunks (8 bf16)
// of the row into registers up front, the row absmax is a packed 16-bit integer max on the
// bf16 magnitude bits (exact, no unpacking) reduced across the wave, and the same registers are
// then scaled, clamped and converted with v_cvt_pk_fp8_f32 and stored 8 bytes per lane
// (consecutive lanes -> consecutive addresses).  HBM traffic is the algorithmic minimum:
// 2 bytes read + 1 byte written per element + 4 bytes per row scale.
//
// Gathered variant (fosswire.org "AMD Primus adds FP8/MXFP8 kernels ...", section "What Primus
// adds for MoE training on MI355X": the MegaMoE item fuses the token exchange with the kernels
// that consume its rows): output row r quantizes source row index[r], so routed token rows are
// put into expert order and quantized in the same pass, with no permuted bf16 copy in HBM.  The
// index is read once per row (wave-uniform, a scalar load) and clamped into the source rows.
#include "common.hpp"

namespace fp8q {

// Source row of output row `row`: the identity, or index[row] clamped into [0, src_rows).
__device__ __forceinline__ int64_t src_row(const int32_t* __restrict__ index, int64_t src_rows,
                                           int64_t row) {
    if (!index) return row;
    const int64_t r = (int64_t)index[row];
    return r < 0 ? 0 : (r >= src_rows ? src_rows - 1 : r);
}

template <int FMT, int WPR, int NV>
__global__ __launch_bounds__(256) void rowwise_vec_kernel(const uint16_t* __restrict__ x,
                                                          int64_t rows, int64_t cols,
                                                          int64_t ld_x, uint8_t* __restrict__ q,
                                                          int64_t ld_q,
                                                          float* __restrict__ scales,
                                                          const int32_t* __restrict__ index,
                                                          int64_t src_rows, bool nt_out) {
    constexpr int RPB = 4 / WPR;   // rows per 256-thread block
    constexpr int TPR = 64 * WPR;  // threads per row
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * RPB + wave / WPR;
    const int t = (wave % WPR) * 64 + lane;
    const bool row_ok = row < rows;
    const int64_t nchunks = cols >> 3;
    const int64_t sr = row_ok ? src_row(index, src_rows, row) : 0;
    const uint4* xr = reinterpret_cast<const uint4*>(x + sr * ld_x);

    uint4 v[NV];
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < NV; j++) {
        const int64_t c = t + (int64_t)j * TPR;
        if (row_ok && c < nchunks) {
            // streaming loads when each row is read once; a gather may read a row repeatedly
            v[j] = index ? xr[c] : ld_nt16(xr + c);
        } else {
            v[j] = make_uint4(0, 0, 0, 0);
        }
        m = pk_max_u16(m, pk_max_u16(pk_max_u16(mag2(v[j].x), mag2(v[j].y)),
                                     pk_max_u16(mag2(v[j].z), mag2(v[j].w))));
    }
    uint32_t amax_bits = wave_max_u32(hmax16(m));
    if (WPR > 1) {
        __shared__ uint32_t red[4];
        if (lane == 0) red[wave] = amax_bits;
        __syncthreads();
        const int w0 = (wave / WPR) * WPR;
#pragma unroll
        for (int w = 0; w < WPR; w++) amax_bits = amax_bits > red[w0 + w] ? amax_bits : red[w0 + w];
    }
    if (!row_ok) return;
    const float s = scale_from_amax<FMT>(__uint_as_float(amax_bits << 16));
    if (t == 0) scales[row] = s;
    const float sm = s * Fmt<FMT>::mult;
    uint2* qr = reinterpret_cast<uint2*>(q + row * ld_q);
#pragma unroll
    for (int j = 0; j < NV; j++) {
        const int64_t c = t + (int64_t)j * TPR;
        if (c < nchunks) {
            uint32_t w0 = enc4<FMT>(bf16_lo(v[j].x) * sm, bf16_hi(v[j].x) * sm,
                                    bf16_lo(v[j].y) * sm, bf16_hi(v[j].y) * sm);
            uint32_t w1 = enc4<FMT>(bf16_lo(v[j].z) * sm, bf16_hi(v[j].z) * sm,
                                    bf16_lo(v[j].w) * sm, bf16_hi(v[j].w) * sm);
            if (nt_out) st_nt8(qr + c, w0, w1);  // block-uniform branch
            else qr[c] = make_uint2(w0, w1);
        }
    }
}

// Any alignment, any length: one 256-thread block per row, element-wise loads; the second
// sweep re-reads the row (from cache).  Used when the vector path's alignment or length
// conditions do not hold.
template <int FMT>
__global__ __launch_bounds__(256) void rowwise_generic_kernel(const uint16_t* __restrict__ x,
                                                              int64_t cols, int64_t ld_x,
                                                              uint8_t* __restrict__ q,
                                                              int64_t ld_q,
                                                              float* __restrict__ scales,
                                                              const int32_t* __restrict__ index,
                                                              int64_t src_rows) {
    const int64_t row = blockIdx.x;
    const uint16_t* xr = x + src_row(index, src_rows, row) * ld_x;
    uint32_t m = 0;
    for (int64_t c = threadIdx.x; c < cols; c += 256) {
        uint32_t a = xr[c] & 0x7FFFu;
        m = a > m ? a : m;
    }
    m = wave_max_u32(m);
    __shared__ uint32_t red[4];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    m = red[0];
#pragma unroll
    for (int w = 1; w < 4; w++) m = m > red[w] ? m : red[w];
    const float s = scale_from_amax<FMT>(__uint_as_float(m << 16));
    if (threadIdx.x == 0) scales[row] = s;
    const float sm = s * Fmt<FMT>::mult;
    for (int64_t c = threadIdx.x; c < cols; c += 256) {
        uint32_t w = enc4<FMT>(bf16_lo(xr[c]) * sm, 0.0f, 0.0f, 0.0f);
        q[row * ld_q + c] = (uint8_t)(w & 0xFFu);
    }
}

template <int FMT, int WPR, int NV>
static void launch_vec(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* q,
                       int64_t ld_q, float* s, const int32_t* index, int64_t src_rows,
                       hipStream_t stream) {
    constexpr int RPB = 4 / WPR;
    const int64_t blocks = (rows + RPB - 1) / RPB;
    const bool nt_out = (double)rows * (double)ld_q > kStreamBytes;
    rowwise_vec_kernel<FMT, WPR, NV><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(
        x, rows, cols, ld_x, q, ld_q, s, index, src_rows, nt_out);
}

template <int FMT>
static fp8q_status_t rowwise_dispatch(const uint16_t* x, int64_t rows, int64_t cols,
                                      int64_t ld_x, uint8_t* q, int64_t ld_q, float* s,
                                      const int32_t* index, int64_t src_rows,
                                      hipStream_t stream) {
    const bool vec = (cols % 8 == 0) && (ld_x % 8 == 0) && (ld_q % 8 == 0) &&
                     fp8q_aligned(x, 16) && fp8q_aligned(q, 8);
#define RW(WPR, NV) launch_vec<FMT, WPR, NV>(x, rows, cols, ld_x, q, ld_q, s, index, src_rows, stream)
    if (vec && cols <= 512) RW(1, 1);
    else if (vec && cols <= 1024) RW(1, 2);
    else if (vec && cols <= 2048) RW(1, 4);
    else if (vec && cols <= 4096) RW(1, 8);
    else if (vec && cols <= 8192) RW(2, 8);
    else if (vec && cols <= 16384) RW(4, 8);
    else if (vec && cols <= 32768) RW(4, 16);
    else
        rowwise_generic_kernel<FMT><<<dim3((unsigned)rows), dim3(256), 0, stream>>>(
            x, cols, ld_x, q, ld_q, s, index, src_rows);
#undef RW
    FP8Q_CHECK_LAUNCH();
    return FP8Q_OK;
}

}  // namespace fp8q

extern "C" fp8q_status_t fp8_quant_rowwise(const uint16_t* x, int64_t rows, int64_t cols,
                                           int64_t ld_x, fp8q_format_t fmt, uint8_t* q,
                                           int64_t ld_q, float* scales, hipStream_t stream) {
    if (rows < 0 || cols < 0 || ld_x < cols || ld_q < cols || !fp8q_fmt_ok(fmt))
        return FP8Q_ERR_INVALID_ARG;
    if (rows == 0) return FP8Q_OK;
    if (!scales || (cols > 0 && (!x || !q))) return FP8Q_ERR_INVALID_ARG;
    if (rows > 0x7FFFFFFFLL) return FP8Q_ERR_UNSUPPORTED;
    if (fmt == FP8Q_E4M3FN)
        return fp8q::rowwise_dispatch<FP8Q_E4M3FN>(x, rows, cols, ld_x, q, ld_q, scales, nullptr,
                                                   rows, stream);
    return fp8q::rowwise_dispatch<FP8Q_E4M3FNUZ>(x, rows, cols, ld_x, q, ld_q, scales, nullptr,
                                                 rows, stream);
}

extern "C" fp8q_status_t fp8_quant_rowwise_gather(const uint16_t* x, int64_t src_rows,
                                                  int64_t cols, int64_t ld_x,
                                                  const int32_t* row_index, int64_t rows,
                                                  fp8q_format_t fmt, uint8_t* q, int64_t ld_q,
                                                  float* scales, hipStream_t stream) {
    if (rows < 0 || src_rows < 0 || cols < 0 || ld_x < cols || ld_q < cols || !fp8q_fmt_ok(fmt))
        return FP8Q_ERR_INVALID_ARG;
    if (rows == 0) return FP8Q_OK;
    if (src_rows == 0 || !row_index || !scales || (cols > 0 && (!x || !q)))
        return FP8Q_ERR_INVALID_ARG;
    if (rows > 0x7FFFFFFFLL) return FP8Q_ERR_UNSUPPORTED;
    if (fmt == FP8Q_E4M3FN)
        return fp8q::rowwise_dispatch<FP8Q_E4M3FN>(x, rows, cols, ld_x, q, ld_q, scales,
                                                   row_index, src_rows, stream);
    return fp8q::rowwise_dispatch<FP8Q_E4M3FNUZ>(x, rows, cols, ld_x, q, ld_q, scales,
                                                 row_index, src_rows, stream);
}
