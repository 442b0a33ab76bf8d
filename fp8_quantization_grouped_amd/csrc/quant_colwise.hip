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
//   1. colwise_amax_kernel: each block walks 1, 2 or 4 consecutive 256-row x 64-column tiles
//      (8 rows x 8 columns per lane, 16-byte loads, 128 contiguous bytes per row, the next tile's loads
//      in flight while the current one is reduced), keeps per-lane column maxima of the group
//      it is in (packed 16-bit max on bf16 magnitude bits), and when the group changes reduces
//      them to 64 column maxima (lane shuffles, then LDS across the 4 waves) and publishes them
//      with relaxed device-scope atomicMax on the bf16 magnitude bits (exact: for finite values
//      their integer order is the value order).  An input too large to stay in the 256 MB
//      last-level cache until the second pass is read with streaming loads.
//   2. colwise_cast_kernel: one 256x64 tile per block (more resident blocks hide the load
//      latency better than a register prefetch of the next tile), streaming loads (last read);
//      turns the finished maxima into scales (per group in LDS), scales/clamps/converts along
//      rows one column at a time so each lane produces 8 consecutive output bytes of each of its
//      8 columns, transposes through LDS and writes 16-byte chunks of the column-major output
//      with streaming stores (16 lanes cover one column's 256 contiguous bytes).
// The group offsets are staged in LDS once per block, so finding a row's group is a short
// search in LDS instead of a chain of dependent global loads.  The block whose tile contains
// a group's first row writes that group's scales; the last row tile also writes groups that
// start at the end (trailing empty groups).
#include <mutex>

#include "common.hpp"

namespace fp8q {

constexpr int CW_TR = 256;              // tile rows
constexpr int CW_TC = 64;               // tile columns
constexpr int CW_STR = CW_TR + 16;      // LDS bytes per transposed column (16-byte aligned)
// Transposed tiles in LDS (here, in the long-group kernel and in the MX colwise kernel): the
// 8-byte piece of column c holding rows 8q..8q+7 sits at byte c*STR + 8*(q ^ 2*((c>>3)&7)), and
// the 16-byte piece of rows 16s..16s+15 at c*STR + 16*(s ^ ((c>>3)&7)).  A wave writes the
// pieces of 8 column octets at once; without the XOR they fall on 16 of the 64 four-byte banks
// for each half-wave (8 cycles per write instead of 2; rocprof counted 64-80% of these kernels'
// LDS cycles as bank conflicts).  The reads stay conflict-free.
constexpr int CW_GB = 8;                // groups per scale batch in LDS
constexpr int CW_TPB_CAST = 1;          // row tiles per block (cast pass)
constexpr int CW_GLDS = 2048;           // groups whose offsets are staged in LDS

// Group offsets as the kernels read them: from an LDS copy staged once per block (LDS, the
// usual case: G <= CW_GLDS) or straight from global memory.  The two are separate template
// instances and the LDS copy is a file-scope __shared__ array referenced by name, so every
// access compiles to a DS or a global instruction.  Never a generic (flat) pointer that may
// point into LDS: a flat access is routed by the aperture of its base address register, and
// the compiler folds "base - 4" + "offset:4" forms (for o[g-1] / o[g] pairs) whose base lies
// just below the LDS aperture when g == 0.
__shared__ int cw_s_off[CW_GLDS];

template <bool LDS>
struct Offs {
    const int32_t* __restrict__ g;
    int G;
    __device__ __forceinline__ int64_t end(int i) const {
        return LDS ? (int64_t)cw_s_off[i] : (int64_t)g[i];
    }
    __device__ __forceinline__ int64_t start(int i) const { return i == 0 ? 0 : end(i - 1); }
    // first g with end(g) > r, clamped to [0, G-1] (any offsets content stays in range)
    __device__ __forceinline__ int group_of(int64_t r) const {
        int lo = 0, hi = G - 1;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (end(mid) > r) hi = mid; else lo = mid + 1;
        }
        return lo;
    }
    // first group whose start row is >= r (G if none)
    __device__ __forceinline__ int first_starting_at(int64_t r) const {
        int lo = 0, hi = G;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (start(mid) >= r) hi = mid; else lo = mid + 1;
        }
        return lo;
    }
};
template <bool LDS>
__device__ __forceinline__ Offs<LDS> stage_offsets(const int32_t* __restrict__ offsets, int G) {
    if (LDS) {
        for (int i = threadIdx.x; i < G; i += 256) cw_s_off[i] = offsets[i];
        __syncthreads();
    }
    return Offs<LDS>{offsets, G};
}

// The lane's 8x8 block: rows r0 + 8*qd + i (i < 8), columns c0 + 8*o .. +7, as bf16 bits
// packed two per dword (column 2d in the low half of dword d).  Out-of-range elements are 0.
template <bool VEC, bool NT = false>
__device__ __forceinline__ void cw_load(const uint16_t* __restrict__ x, int64_t R, int64_t C,
                                        int64_t ld_x, int64_t r0, int64_t c0, int o, int qd,
                                        uint4 v[8]) {
    const int64_t c = c0 + 8 * o;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const int64_t r = r0 + 8 * qd + i;
        if (VEC) {
            v[i] = (r < R && c < C) ? (NT ? ld_nt16(x + r * ld_x + c)
                                          : *reinterpret_cast<const uint4*>(x + r * ld_x + c))
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

// Column j (0..7) of a lane's 8-column row chunk as fp32 (column 2d in the low half of dword d).
__device__ __forceinline__ float cw_elem(const uint4& r, int j) {
    const uint32_t w = j < 2 ? r.x : j < 4 ? r.y : j < 6 ? r.z : r.w;
    return (j & 1) ? bf16_hi(w) : bf16_lo(w);
}

__global__ void cw_zero_kernel(uint32_t* __restrict__ p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        p[i] = 0u;
}

// ROWP: also write each row's maximum over the tile's 64 columns (bf16 magnitude bits) to
// rowp[blockIdx.y * Rp + r] (Rp = R rounded up to 8; each lane of a row group stores its 8
// consecutive rows at once): the dual-layout call reduces them into rowwise scales.
template <bool VEC, bool LDS, bool NT, bool ROWP, int TPB>
__global__ __launch_bounds__(256) void colwise_amax_kernel(const uint16_t* __restrict__ x,
                                                           int64_t R, int64_t C, int64_t ld_x,
                                                           const int32_t* __restrict__ offsets,
                                                           int G, uint32_t* __restrict__ amax,
                                                           uint16_t* __restrict__ rowp) {
    const int t = threadIdx.x, o = t & 7, qd = t >> 3, lane = t & 63, wave = t >> 6;
    const int64_t rb = (int64_t)blockIdx.x * CW_TR * TPB, c0 = (int64_t)blockIdx.y * CW_TC;
    __shared__ uint32_t red[4][8][4];
    const Offs<LDS> off = stage_offsets<LDS>(offsets, G);
    // running per-lane maxima of group cur_g (block-uniform), published when the group ends
    int cur_g = -1;
    uint32_t m0 = 0, m1 = 0, m2 = 0, m3 = 0;
    auto flush = [&]() {
#pragma unroll
        for (int sh = 8; sh < 64; sh <<= 1) {
            m0 = pk_max_u16(m0, (uint32_t)__shfl_xor((int)m0, sh, 64));
            m1 = pk_max_u16(m1, (uint32_t)__shfl_xor((int)m1, sh, 64));
            m2 = pk_max_u16(m2, (uint32_t)__shfl_xor((int)m2, sh, 64));
            m3 = pk_max_u16(m3, (uint32_t)__shfl_xor((int)m3, sh, 64));
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
            const uint32_t mm = pk_max_u16(pk_max_u16(red[0][oo][d], red[1][oo][d]),
                                           pk_max_u16(red[2][oo][d], red[3][oo][d]));
            const int64_t c = c0 + 8 * oo + 2 * d;
            const uint32_t lo = mm & 0xFFFFu, hi = mm >> 16;
            uint32_t* dst = amax + (int64_t)cur_g * C + c;
            if (lo && c < C) __hip_atomic_fetch_max(dst, lo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (hi && c + 1 < C) __hip_atomic_fetch_max(dst + 1, hi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        m0 = m1 = m2 = m3 = 0;
    };
    uint4 v[8], vn[8];
    cw_load<VEC, NT>(x, R, C, ld_x, rb, c0, o, qd, v);
    for (int k = 0; k < TPB; k++) {
        const int64_t r0 = rb + (int64_t)k * CW_TR;
        if (r0 >= R) break;  // block-uniform
        if (k + 1 < TPB) cw_load<VEC, NT>(x, R, C, ld_x, r0 + CW_TR, c0, o, qd, vn);
        const int64_t r_end = r0 + CW_TR < R ? r0 + CW_TR : R;
        if (ROWP) {
            // the 8 lanes of a row group (o = 0..7, consecutive lanes) hold its 64 columns;
            // lane o = 0 stores the maxima of its 8 rows as one 16-byte piece
            uint32_t pk[4] = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int i = 0; i < 8; i++) {
                uint32_t m = pk_max_u16(pk_max_u16(mag2(v[i].x), mag2(v[i].y)),
                                        pk_max_u16(mag2(v[i].z), mag2(v[i].w)));
                m = hmax16(m);
                m = max(m, (uint32_t)__shfl_xor((int)m, 1, 64));
                m = max(m, (uint32_t)__shfl_xor((int)m, 2, 64));
                m = max(m, (uint32_t)__shfl_xor((int)m, 4, 64));
                pk[i >> 1] |= m << (16 * (i & 1));
            }
            const int64_t Rp = (R + 7) & ~(int64_t)7, r = r0 + 8 * qd;
            if (o == 0 && r < Rp)
                *reinterpret_cast<uint4*>(rowp + (int64_t)blockIdx.y * Rp + r) =
                    make_uint4(pk[0], pk[1], pk[2], pk[3]);
        }
        const int g_first = off.group_of(r0);
        const int g_last = off.group_of(r_end - 1);
        for (int g = g_first; g <= g_last; g++) {
            int64_t gs = off.start(g);
            int64_t ge = g == G - 1 ? r_end : off.end(g);
            gs = gs > r0 ? gs : r0;
            ge = ge < r_end ? ge : r_end;
            if (gs >= ge) continue;  // block-uniform
            if (g != cur_g) {
                if (cur_g >= 0) flush();
                cur_g = g;
            }
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
        }
#pragma unroll
        for (int i = 0; i < 8; i++) v[i] = vn[i];
    }
    if (cur_g >= 0) flush();
}

// ROWQ: also cast the tile along rows with the rowwise scales s_rows (already computed) and
// write the row-major bytes q[r * ld_q + c] (the dual-layout call); ROWQ_VEC: 8-byte stores.
template <int FMT, bool VEC, bool VEC_OUT, bool LDS, bool ROWQ = false, bool ROWQ_VEC = false>
__global__ __launch_bounds__(256) void colwise_cast_kernel(
    const uint16_t* __restrict__ x, int64_t R, int64_t C, int64_t ld_x,
    const int32_t* __restrict__ offsets, int G, const uint32_t* __restrict__ amax,
    uint8_t* __restrict__ qt, int64_t ld_qt, float* __restrict__ scales,
    const float* __restrict__ s_rows, uint8_t* __restrict__ q, int64_t ld_q) {
    const int t = threadIdx.x, o = t & 7, qd = t >> 3;
    const int64_t rb = (int64_t)blockIdx.x * CW_TR * CW_TPB_CAST, c0 = (int64_t)blockIdx.y * CW_TC;
    __shared__ __align__(16) float sc[CW_GB][CW_TC];
    __shared__ __align__(16) uint8_t tile[CW_TC * CW_STR];
    const Offs<LDS> off = stage_offsets<LDS>(offsets, G);

    // Scales of the groups this block owns (first row inside one of its tiles; the block with
    // the last tile also owns groups starting at or after the end, i.e. trailing empty groups).
    {
        const int64_t r_stop = rb + (int64_t)CW_TR * CW_TPB_CAST;
        const bool last_block = r_stop >= R;
        for (int g = off.first_starting_at(rb); g < G; g++) {
            if (!last_block && off.start(g) >= r_stop) break;
            if (t < CW_TC && c0 + t < C) {
                const int64_t idx = (int64_t)g * C + c0 + t;
                scales[idx] = scale_from_amax<FMT>(__uint_as_float(amax[idx] << 16));
            }
        }
    }
    if (rb >= R) return;  // only the R == 0 launch has such a block (block-uniform)

    int sc_lo = -1, sc_hi = -2;  // groups held in sc (block-uniform)
    uint4 v[8], vn[8];
    cw_load<VEC, true>(x, R, C, ld_x, rb, c0, o, qd, v);
    // ROWQ: the rowwise scales of the lane's 8 rows, loaded with the tile (one tile per block)
    static_assert(!ROWQ || CW_TPB_CAST == 1, "row scales are loaded for the block's one tile");
    float srow[8];
    if (ROWQ) {
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const int64_t r = rb + 8 * qd + i;
            srow[i] = r < R ? s_rows[r] * Fmt<FMT>::mult : 0.0f;
        }
    }
    for (int k = 0; k < CW_TPB_CAST; k++) {
        const int64_t r0 = rb + (int64_t)k * CW_TR;
        if (r0 >= R) break;  // block-uniform
        if (k + 1 < CW_TPB_CAST) cw_load<VEC, true>(x, R, C, ld_x, r0 + CW_TR, c0, o, qd, vn);
        const int64_t r_end = r0 + CW_TR < R ? r0 + CW_TR : R;
        if (ROWQ) {
            // rowwise bytes of the lane's 8 rows x 8 columns, with each row's own scale
            const int64_t c = c0 + 8 * o;
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const int64_t r = r0 + 8 * qd + i;
                if (r >= R || c >= C) continue;
                const float sr = srow[i];
                const uint32_t lo = enc4<FMT>(cw_elem(v[i], 0) * sr, cw_elem(v[i], 1) * sr,
                                              cw_elem(v[i], 2) * sr, cw_elem(v[i], 3) * sr);
                const uint32_t hi = enc4<FMT>(cw_elem(v[i], 4) * sr, cw_elem(v[i], 5) * sr,
                                              cw_elem(v[i], 6) * sr, cw_elem(v[i], 7) * sr);
                uint8_t* dst = q + r * ld_q + c;
                if (ROWQ_VEC) {
                    *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
                } else {
                    const uint32_t w[2] = {lo, hi};
                    for (int j = 0; j < 8 && c + j < C; j++) dst[j] = (uint8_t)(w[j >> 2] >> (8 * (j & 3)));
                }
            }
        }
        const int g_first = off.group_of(r0);
        const int g_last = off.group_of(r_end - 1);
        // group of each of the lane's rows (-1 past the end)
        int gid[8];
        {
            int g = off.group_of(r0 + 8 * qd);
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const int64_t r = r0 + 8 * qd + i;
                while (g < G - 1 && off.end(g) <= r) g++;
                gid[i] = r < r_end ? g : -1;
            }
        }
        uint32_t ow0[8], ow1[8];
#pragma unroll
        for (int j = 0; j < 8; j++) ow0[j] = ow1[j] = 0u;
        for (int gb = g_first; gb <= g_last; gb += CW_GB) {
            const int gb_hi = gb + CW_GB - 1 < g_last ? gb + CW_GB - 1 : g_last;
            if (!(gb >= sc_lo && gb_hi <= sc_hi)) {
                __syncthreads();  // previous users of sc are done
                for (int idx = t; idx < CW_GB * CW_TC; idx += 256) {
                    const int kk = idx / CW_TC, cc = idx % CW_TC;
                    const int g = gb + kk;
                    float s = 0.0f;
                    if (g < G && c0 + cc < C)
                        s = scale_from_amax<FMT>(__uint_as_float(amax[(int64_t)g * C + c0 + cc] << 16)) *
                            Fmt<FMT>::mult;
                    sc[kk][cc] = s;
                }
                __syncthreads();
                sc_lo = gb;
                sc_hi = gb + CW_GB - 1;
            }
            if (g_first == g_last) {
                const int kk = g_first - sc_lo;
                const float4 sa = *reinterpret_cast<const float4*>(&sc[kk][8 * o]);
                const float4 sb = *reinterpret_cast<const float4*>(&sc[kk][8 * o + 4]);
                const float sj[8] = {sa.x, sa.y, sa.z, sa.w, sb.x, sb.y, sb.z, sb.w};
#pragma unroll
                for (int j = 0; j < 8; j++) {
                    float y[8];
#pragma unroll
                    for (int i = 0; i < 8; i++) y[i] = cw_elem(v[i], j) * sj[j];
                    ow0[j] = enc4<FMT>(y[0], y[1], y[2], y[3]);
                    ow1[j] = enc4<FMT>(y[4], y[5], y[6], y[7]);
                }
            } else {
#pragma unroll
                for (int pr = 0; pr < 4; pr++) {
                    float y[2][8];
#pragma unroll
                    for (int ii = 0; ii < 2; ii++) {
                        const int i = 2 * pr + ii;
                        const bool in = gid[i] >= gb && gid[i] <= gb_hi;
                        const int kk = in ? gid[i] - sc_lo : 0;
                        const float4 sa = *reinterpret_cast<const float4*>(&sc[kk][8 * o]);
                        const float4 sb = *reinterpret_cast<const float4*>(&sc[kk][8 * o + 4]);
                        const float sj[8] = {sa.x, sa.y, sa.z, sa.w, sb.x, sb.y, sb.z, sb.w};
#pragma unroll
                        for (int j = 0; j < 8; j++) y[ii][j] = in ? cw_elem(v[i], j) * sj[j] : 0.0f;
                    }
#pragma unroll
                    for (int j = 0; j < 8; j++) {
                        const uint32_t w = enc4<FMT>(y[0][j], y[1][j], 0.0f, 0.0f) << (16 * (pr & 1));
                        if (pr < 2) ow0[j] |= w; else ow1[j] |= w;
                    }
                }
            }
        }
        __syncthreads();  // previous tile's transposed bytes have been stored
#pragma unroll
        for (int j = 0; j < 8; j++)
            *reinterpret_cast<uint2*>(&tile[(8 * o + j) * CW_STR + 8 * (qd ^ (2 * o))]) = make_uint2(ow0[j], ow1[j]);
        __syncthreads();
#pragma unroll
        for (int kq = 0; kq < 4; kq++) {
            const int ch = t + 256 * kq;
            const int col = ch >> 4, seg = ch & 15;
            const int64_t c = c0 + col, r = r0 + 16 * seg;
            if (c >= C || r >= R) continue;
            const uint8_t* src = &tile[col * CW_STR + 16 * (seg ^ ((col >> 3) & 7))];
            uint8_t* dst = qt + c * ld_qt + r;
            if (VEC_OUT && r + 16 <= R) {
                st_nt16(dst, *reinterpret_cast<const uint4*>(src));  // measured faster at every size
            } else {
                for (int bb = 0; bb < 16; bb++)
                    if (r + bb < R) dst[bb] = src[bb];
            }
        }
#pragma unroll
        for (int i = 0; i < 8; i++)
            if (k + 1 < CW_TPB_CAST) v[i] = vn[i];
    }
}

// ------------------------------------------------------------------ long groups, one block each
// For long groups (the expert weights: K rows per expert) one 1024-thread block owns a whole
// (group, 64-column strip): it streams the strip once for the column maxima (lanes keep packed
// maxima, then lane shuffles and LDS across the 16 waves; no atomics, no workspace), turns them
// into scales, and streams it again to cast, transposing 1024-row tiles through LDS so that each
// column is written in 1 KB runs.  One block runs per CU (the LDS tile is padded past 80 KB), so
// the strips being walked at any moment total ~256 x 0.9 MB and the second read of a strip is
// served by the 256 MB last-level cache.  Measured on the 32 x 7168 x 2048 weights: 410 us with
// one block per CU, 497 us when two fit; streaming loads on the second read 388 us.
// Lane layout as in the two-pass kernels: lane (o = t & 7, qd = t >> 3) holds rows
// r0 + 8*qd + i (i < 8) x columns c0 + 8*o .. +7; a tile is 1024 rows x 64 columns.
// LDS bytes per transposed column: 1024-row tiles are padded past 80 KB in all (one block per
// CU); smaller tiles let several blocks share a CU.
template <int TR>
struct LongTile {
    static constexpr int STR = TR == 1024 ? TR + 272 : TR + 16;
};

template <int FMT, bool VEC_OUT, int TR>
__global__ __launch_bounds__(TR) void colwise_long_kernel(
    const uint16_t* __restrict__ x, int64_t R, int64_t C, int64_t ld_x,
    const int32_t* __restrict__ offsets, int G, uint8_t* __restrict__ qt, int64_t ld_qt,
    float* __restrict__ scales) {
    const int t = threadIdx.x, o = t & 7, qd = t >> 3, lane = t & 63, wave = t >> 6;
    const int64_t ST = (C + CW_TC - 1) / CW_TC;
    const int g = (int)(blockIdx.x / ST);
    const int64_t c0 = (int64_t)(blockIdx.x % ST) * CW_TC;
    const int64_t c = c0 + 8 * o;
    // the group's rows, clamped into [0, R] so that any offsets content keeps accesses in range
    int64_t gs = g == 0 ? 0 : (int64_t)offsets[g - 1];
    int64_t ge = offsets[g];
    gs = gs < 0 ? 0 : (gs > R ? R : gs);
    ge = ge < gs ? gs : (ge > R ? R : ge);
    constexpr int CL_TR = TR, CL_STR = LongTile<TR>::STR, NW = TR / 64;
    __shared__ uint32_t red[NW][8][4];
    __shared__ __align__(16) float scl[CW_TC];
    __shared__ __align__(16) uint8_t tile[CW_TC * CL_STR];
    const int64_t tb = gs & ~(int64_t)(CL_TR - 1);  // tiles start at multiples of 1024 rows

    // rows outside the group load as zero; the second (last) read of a row streams (NT)
    auto load = [&](int64_t r0, uint4 v[8], bool nt) {
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const int64_t r = r0 + 8 * qd + i;
            const uint16_t* px = x + r * ld_x + c;
            v[i] = (r >= gs && r < ge && c < C)
                       ? (nt ? ld_nt16(px) : *reinterpret_cast<const uint4*>(px))
                       : make_uint4(0, 0, 0, 0);
        }
    };
    // pass 1: column maxima of the group
    uint32_t m0 = 0, m1 = 0, m2 = 0, m3 = 0;
    for (int64_t r0 = tb; r0 < ge; r0 += CL_TR) {
        uint4 v[8];
        load(r0, v, false);
#pragma unroll
        for (int i = 0; i < 8; i++) {
            m0 = pk_max_u16(m0, mag2(v[i].x));
            m1 = pk_max_u16(m1, mag2(v[i].y));
            m2 = pk_max_u16(m2, mag2(v[i].z));
            m3 = pk_max_u16(m3, mag2(v[i].w));
        }
    }
#pragma unroll
    for (int sh = 8; sh < 64; sh <<= 1) {
        m0 = pk_max_u16(m0, (uint32_t)__shfl_xor((int)m0, sh, 64));
        m1 = pk_max_u16(m1, (uint32_t)__shfl_xor((int)m1, sh, 64));
        m2 = pk_max_u16(m2, (uint32_t)__shfl_xor((int)m2, sh, 64));
        m3 = pk_max_u16(m3, (uint32_t)__shfl_xor((int)m3, sh, 64));
    }
    if (lane < 8) {
        red[wave][lane][0] = m0;
        red[wave][lane][1] = m1;
        red[wave][lane][2] = m2;
        red[wave][lane][3] = m3;
    }
    __syncthreads();
    if (t < CW_TC) {
        const int oo = t >> 3, d = (t & 7) >> 1, half = t & 1;
        uint32_t mm = 0;
#pragma unroll
        for (int w = 0; w < NW; w++) mm = pk_max_u16(mm, red[w][oo][d]);
        const uint32_t bits = half ? (mm >> 16) : (mm & 0xFFFFu);
        const float sc = scale_from_amax<FMT>(__uint_as_float(bits << 16));
        if (c0 + t < C) scales[(int64_t)g * C + c0 + t] = sc;
        scl[t] = sc * Fmt<FMT>::mult;
    }
    __syncthreads();
    const float4 sa = *reinterpret_cast<const float4*>(&scl[8 * o]);
    const float4 sb = *reinterpret_cast<const float4*>(&scl[8 * o + 4]);
    const float sj[8] = {sa.x, sa.y, sa.z, sa.w, sb.x, sb.y, sb.z, sb.w};
    // pass 2: cast, transpose through LDS, write 16-byte chunks of each column's run; the next
    // tile's loads are issued before this tile's transpose and stores
    uint4 v[8];
    if (tb < ge) load(tb, v, true);
    for (int64_t r0 = tb; r0 < ge; r0 += CL_TR) {
        uint4 vn[8];
        const bool more = r0 + CL_TR < ge;  // block-uniform
        if (more) load(r0 + CL_TR, vn, true);
        __syncthreads();  // the previous tile's bytes have been stored
#pragma unroll
        for (int j = 0; j < 8; j++) {
            float y[8];
#pragma unroll
            for (int i = 0; i < 8; i++) y[i] = cw_elem(v[i], j) * sj[j];
            *reinterpret_cast<uint2*>(&tile[(8 * o + j) * CL_STR + 8 * (qd ^ (2 * o))]) =
                make_uint2(enc4<FMT>(y[0], y[1], y[2], y[3]), enc4<FMT>(y[4], y[5], y[6], y[7]));
        }
        __syncthreads();
#pragma unroll
        for (int kq = 0; kq < 4; kq++) {
            const int ch = t + TR * kq;
            const int col = ch / (TR / 16), seg = ch % (TR / 16);  // TR/16 chunks per column
            const int64_t cc = c0 + col, r = r0 + 16 * seg;
            if (cc >= C || r + 16 <= gs || r >= ge) continue;
            const uint8_t* src = &tile[col * CL_STR + 16 * (seg ^ ((col >> 3) & 7))];
            uint8_t* dst = qt + cc * ld_qt + r;
            if (VEC_OUT && r >= gs && r + 16 <= ge) {
                st_nt16(dst, *reinterpret_cast<const uint4*>(src));
            } else {
                for (int bb = 0; bb < 16; bb++)
                    if (r + bb >= gs && r + bb < ge) dst[bb] = src[bb];
            }
        }
        if (more) {
#pragma unroll
            for (int i = 0; i < 8; i++) v[i] = vn[i];
        }
    }
}

template <int FMT, bool VEC, bool VEC_OUT>
static void launch_cast(const uint16_t* x, int64_t R, int64_t C, int64_t ld_x,
                        const int32_t* offsets, int G, const uint32_t* ws, uint8_t* qt,
                        int64_t ld_qt, float* s, hipStream_t stream) {
    const int64_t rt = R > 0 ? (R + CW_TR * CW_TPB_CAST - 1) / (CW_TR * CW_TPB_CAST) : 1;
    const int64_t ct = (C + CW_TC - 1) / CW_TC;
    const dim3 grid((unsigned)rt, (unsigned)ct);
    if (G <= CW_GLDS)
        colwise_cast_kernel<FMT, VEC, VEC_OUT, true><<<grid, dim3(256), 0, stream>>>(
            x, R, C, ld_x, offsets, G, ws, qt, ld_qt, s, nullptr, nullptr, 0);
    else
        colwise_cast_kernel<FMT, VEC, VEC_OUT, false><<<grid, dim3(256), 0, stream>>>(
            x, R, C, ld_x, offsets, G, ws, qt, ld_qt, s, nullptr, nullptr, 0);
}

// ------------------------------------------------------------------ weights in both layouts
// Pass 1 (wdual_rows_kernel): one 1024-thread block per 128 rows of one expert; wave w quantizes
// rows w, w+16, .. (8 rows, one at a time, the next row's loads in flight) exactly as
// fp8_quant_rowwise does: lane chunk j is columns 8*(lane + 64j) .. +7, the row maximum is a
// wave reduction, then scale, cast and 8-byte stores.  Each lane also keeps the maxima of its
// columns over its rows; the 16 waves combine them in LDS at the end and the block stores its
// 128-row column maxima as bf16 magnitude bits per (block, column): plain stores, no atomics.
// (Measured on the 32 x 7168 x 2048 weights, whole call: 4 waves x 16 rows 592 us, 8 x 8
// 570 us, 16 x 4 563 us, 16 x 8 557 us.)
// wdual_colmax_kernel reduces them per (expert, column) into the maxima layout of the colwise
// cast pass (and writes the offsets K, 2K, ..), which then runs unchanged.
constexpr int WD_RB = 128;  // rows per block of pass 1
constexpr int WD_NW = 16;  // waves per block of pass 1 (WD_RB / WD_NW rows each)
constexpr int WD_NV = 4;   // 16-byte chunks per lane: N <= 64 * 8 * WD_NV = 2048
constexpr int WD_NMAX = 64 * 8 * WD_NV;

template <int FMT>
__global__ __launch_bounds__(64 * WD_NW) void wdual_rows_kernel(
    const uint16_t* __restrict__ w, int64_t K, int64_t N, int64_t ld_w, int64_t nb,
    uint8_t* __restrict__ qr, int64_t ld_qr, float* __restrict__ s_rows,
    uint16_t* __restrict__ part, bool nt_out) {
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int64_t e = blockIdx.x / nb, b = blockIdx.x % nb;
    const int64_t kr0 = b * WD_RB + wave;  // this wave's first row within the expert
    __shared__ __align__(16) uint32_t cred[WD_NW][64 * WD_NV][4];
    auto load = [&](int64_t kr, uint4 v[WD_NV]) {
#pragma unroll
        for (int j = 0; j < WD_NV; j++) {
            const int64_t col = 8 * (int64_t)(lane + 64 * j);
            v[j] = (kr < K && col < N) ? ld_nt16(w + (e * K + kr) * ld_w + col)
                                       : make_uint4(0, 0, 0, 0);
        }
    };
    uint32_t cm[WD_NV][4];
#pragma unroll
    for (int j = 0; j < WD_NV; j++) cm[j][0] = cm[j][1] = cm[j][2] = cm[j][3] = 0u;
    uint4 v[WD_NV], vn[WD_NV];
    load(kr0, v);
    for (int i = 0; i < WD_RB / WD_NW; i++) {
        const int64_t kr = kr0 + WD_NW * i;
        if (i + 1 < WD_RB / WD_NW) load(kr + WD_NW, vn);
        if (kr < K) {  // wave-uniform
            uint32_t m = 0;
#pragma unroll
            for (int j = 0; j < WD_NV; j++) {
                m = pk_max_u16(m, pk_max_u16(pk_max_u16(mag2(v[j].x), mag2(v[j].y)),
                                             pk_max_u16(mag2(v[j].z), mag2(v[j].w))));
                cm[j][0] = pk_max_u16(cm[j][0], mag2(v[j].x));
                cm[j][1] = pk_max_u16(cm[j][1], mag2(v[j].y));
                cm[j][2] = pk_max_u16(cm[j][2], mag2(v[j].z));
                cm[j][3] = pk_max_u16(cm[j][3], mag2(v[j].w));
            }
            const uint32_t amax = wave_max_u32(hmax16(m));
            const float sc = scale_from_amax<FMT>(__uint_as_float(amax << 16));
            if (lane == 0) s_rows[e * K + kr] = sc;
            const float sm = sc * Fmt<FMT>::mult;
#pragma unroll
            for (int j = 0; j < WD_NV; j++) {
                const int64_t col = 8 * (int64_t)(lane + 64 * j);
                if (col >= N) continue;
                const uint32_t w0 = enc4<FMT>(bf16_lo(v[j].x) * sm, bf16_hi(v[j].x) * sm,
                                              bf16_lo(v[j].y) * sm, bf16_hi(v[j].y) * sm);
                const uint32_t w1 = enc4<FMT>(bf16_lo(v[j].z) * sm, bf16_hi(v[j].z) * sm,
                                              bf16_lo(v[j].w) * sm, bf16_hi(v[j].w) * sm);
                uint8_t* dst = qr + (e * K + kr) * ld_qr + col;
                if (nt_out) st_nt8(dst, w0, w1);  // block-uniform
                else *reinterpret_cast<uint2*>(dst) = make_uint2(w0, w1);
            }
        }
#pragma unroll
        for (int j = 0; j < WD_NV; j++) v[j] = vn[j];
    }
#pragma unroll
    for (int j = 0; j < WD_NV; j++)
        *reinterpret_cast<uint4*>(&cred[wave][lane + 64 * j][0]) =
            make_uint4(cm[j][0], cm[j][1], cm[j][2], cm[j][3]);
    __syncthreads();
    // chunk q = t holds columns 8q .. 8q+7 (64 * WD_NV = 256 chunks)
    if (t < 64 * WD_NV && 8 * (int64_t)t < N) {
        uint32_t mm[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int ww = 0; ww < WD_NW; ww++)
#pragma unroll
            for (int d = 0; d < 4; d++) mm[d] = pk_max_u16(mm[d], cred[ww][t][d]);
        *reinterpret_cast<uint4*>(part + (e * nb + b) * N + 8 * (int64_t)t) =
            make_uint4(mm[0], mm[1], mm[2], mm[3]);
    }
}

__global__ void wdual_colmax_kernel(const uint16_t* __restrict__ part, int64_t nb, int64_t E,
                                    int64_t N, int64_t K, uint32_t* __restrict__ amax,
                                    int32_t* __restrict__ offs) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < E) offs[i] = (int32_t)((i + 1) * K);  // host: E * K < 2^31
    if (i >= E * N) return;
    const int64_t e = i / N, n = i % N;
    uint32_t m = 0;
#pragma unroll 8
    for (int64_t b = 0; b < nb; b++) {  // unrolled: eight loads in flight
        const uint32_t u = part[(e * nb + b) * N + n];
        m = u > m ? u : m;
    }
    amax[i] = m;
}

// Workspace: column maxima [E][N] u32 | offsets [E] int32 | block maxima [E*nb][N] u16, each
// part 256-byte aligned.
static inline void wdual_layout(int64_t E, int64_t K, int64_t N, size_t& o_offs, size_t& o_part,
                                size_t& total) {
    auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
    const int64_t nb = (K + WD_RB - 1) / WD_RB;
    o_offs = up((size_t)E * (size_t)N * 4);
    o_part = o_offs + up((size_t)E * 4);
    total = o_part + up((size_t)E * (size_t)nb * (size_t)N * 2);
}

// The maxima pass walks TPB consecutive row tiles per block (the next tile's loads in flight
// while one is reduced; fewer blocks, fewer atomics): 4, unless that leaves fewer than
// CW_AMAX_MIN_BLOCKS blocks to hide the loads' latency (then 2, or 1).  dsv3 X^T (16384 x 7168,
// one tile per block): 134 -> 126 us, dual-layout X 170 -> 161 us against 4 tiles per block.
constexpr int64_t CW_AMAX_MIN_BLOCKS = 4096;
static int amax_tpb(int64_t R, int64_t C) {
    const int64_t strips = (C + CW_TC - 1) / CW_TC;
    for (int tp = 4; tp > 1; tp >>= 1)
        if ((R + CW_TR * tp - 1) / (CW_TR * tp) * strips >= CW_AMAX_MIN_BLOCKS) return tp;
    return 1;
}
template <bool VEC, bool LDS, bool NT, bool ROWP>
static void launch_amax(int tpb, const uint16_t* x, int64_t R, int64_t C, int64_t ld_x,
                        const int32_t* offsets, int G, uint32_t* amax, uint16_t* rowp,
                        hipStream_t stream) {
    const unsigned gy = (unsigned)((C + CW_TC - 1) / CW_TC);
    auto gx = [&](int tp) { return (unsigned)((R + CW_TR * tp - 1) / (CW_TR * tp)); };
    if (tpb == 1)
        colwise_amax_kernel<VEC, LDS, NT, ROWP, 1><<<dim3(gx(1), gy), dim3(256), 0, stream>>>(
            x, R, C, ld_x, offsets, G, amax, rowp);
    else if (tpb == 2)
        colwise_amax_kernel<VEC, LDS, NT, ROWP, 2><<<dim3(gx(2), gy), dim3(256), 0, stream>>>(
            x, R, C, ld_x, offsets, G, amax, rowp);
    else
        colwise_amax_kernel<VEC, LDS, NT, ROWP, 4><<<dim3(gx(4), gy), dim3(256), 0, stream>>>(
            x, R, C, ld_x, offsets, G, amax, rowp);
}

template <int FMT>
static fp8q_status_t colwise_run(const uint16_t* x, int64_t R, int64_t C, int64_t ld_x,
                                 const int32_t* offsets, int G, uint8_t* qt, int64_t ld_qt,
                                 float* s, uint32_t* ws, hipStream_t stream) {
    const bool vec = (C % 8 == 0) && (ld_x % 8 == 0) && fp8q_aligned(x, 16);
    const bool vec_out = (ld_qt % 16 == 0) && fp8q_aligned(qt, 16);
    // Long groups (average at least 4096 rows, e.g. expert weights) with enough (group, strip)
    // pairs to fill the device: one block per pair, no workspace.
    const int64_t strips = (C + CW_TC - 1) / CW_TC;
    if (vec && R >= 4096 * (int64_t)G && (int64_t)G * strips >= 512 &&
        (int64_t)G * strips <= 0x7FFFFFFFLL) {
        const dim3 grid((unsigned)(G * strips));
        if (vec_out)
            colwise_long_kernel<FMT, true, 1024><<<grid, dim3(1024), 0, stream>>>(
                x, R, C, ld_x, offsets, G, qt, ld_qt, s);
        else
            colwise_long_kernel<FMT, false, 1024><<<grid, dim3(1024), 0, stream>>>(
                x, R, C, ld_x, offsets, G, qt, ld_qt, s);
        FP8Q_CHECK_LAUNCH();
        return FP8Q_OK;
    }
    const int64_t n = (int64_t)G * C;
    int64_t zb = (n + 255) / 256;
    if (zb > 4096) zb = 4096;
    cw_zero_kernel<<<dim3((unsigned)zb), dim3(256), 0, stream>>>(ws, n);
    if (R > 0) {
        const bool lds = G <= CW_GLDS;
        // The cast pass reads the input again.  An input of up to 128 MB can stay in the 256 MB
        // last-level cache until then, so this pass reads it with ordinary loads; a larger one
        // cannot, and is read with streaming loads.
        const bool nt = (double)R * (double)ld_x * 2.0 > kStreamBytes;
        const int tpb = amax_tpb(R, C);
        if (vec && lds && nt)
            launch_amax<true, true, true, false>(tpb, x, R, C, ld_x, offsets, G, ws, nullptr, stream);
        else if (vec && lds)
            launch_amax<true, true, false, false>(tpb, x, R, C, ld_x, offsets, G, ws, nullptr, stream);
        else if (vec && nt)
            launch_amax<true, false, true, false>(4, x, R, C, ld_x, offsets, G, ws, nullptr, stream);
        else if (vec)
            launch_amax<true, false, false, false>(4, x, R, C, ld_x, offsets, G, ws, nullptr, stream);
        else if (lds)
            launch_amax<false, true, false, false>(4, x, R, C, ld_x, offsets, G, ws, nullptr, stream);
        else
            launch_amax<false, false, false, false>(4, x, R, C, ld_x, offsets, G, ws, nullptr, stream);
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

namespace fp8q {

// ------------------------------------------------------------------ both layouts of activations
// Rowwise scales from the per-(row, 64-column tile) maxima of the dual maxima pass.
template <int FMT>
__global__ __launch_bounds__(256) void dual_rowscale_kernel(const uint16_t* __restrict__ rowp,
                                                            int64_t R, int nct,
                                                            float* __restrict__ s_rows) {
    // 64 rows per block, each reduced by 4 threads (one per wave) over every 4th column tile:
    // the loads of a wave cover 64 consecutive rows of one column tile
    __shared__ uint32_t red[4][64];
    const int t = threadIdx.x, part = t >> 6;
    const int64_t Rp = (R + 7) & ~(int64_t)7, r = (int64_t)blockIdx.x * 64 + (t & 63);
    uint32_t m = 0;
    if (r < R)
        for (int i = part; i < nct; i += 4) m = max(m, (uint32_t)rowp[(int64_t)i * Rp + r]);
    red[part][t & 63] = m;
    __syncthreads();
    if (t < 64 && r < R) {
        const uint32_t mm = max(max(red[0][t], red[1][t]), max(red[2][t], red[3][t]));
        s_rows[r] = scale_from_amax<FMT>(__uint_as_float(mm << 16));
    }
}

// Workspace of the dual call: the (group, column) maxima, then the (column tile, row) maxima.
static void dual_layout(int64_t R, int64_t C, int64_t G, size_t& o_rowp, size_t& total) {
    const size_t a = ((size_t)G * (size_t)C * 4 + 255) & ~(size_t)255;
    const size_t Rp = ((size_t)R + 7) & ~(size_t)7;  // rows of each column tile, padded to 8
    const size_t b = (Rp * (size_t)((C + CW_TC - 1) / CW_TC) * 2 + 255) & ~(size_t)255;
    o_rowp = a;
    total = a + b;
}

template <int FMT, bool VEC, bool VEC_OUT, bool LDS>
static void launch_cast_dual(const uint16_t* x, int64_t R, int64_t C, int64_t ld_x,
                             const int32_t* offsets, int G, const uint32_t* ws, uint8_t* qt,
                             int64_t ld_qt, float* s, const float* s_rows, uint8_t* q,
                             int64_t ld_q, bool rowq_vec, hipStream_t stream) {
    const int64_t rt = R > 0 ? (R + CW_TR * CW_TPB_CAST - 1) / (CW_TR * CW_TPB_CAST) : 1;
    const dim3 grid((unsigned)rt, (unsigned)((C + CW_TC - 1) / CW_TC));
    if (rowq_vec)
        colwise_cast_kernel<FMT, VEC, VEC_OUT, LDS, true, true><<<grid, dim3(256), 0, stream>>>(
            x, R, C, ld_x, offsets, G, ws, qt, ld_qt, s, s_rows, q, ld_q);
    else
        colwise_cast_kernel<FMT, VEC, VEC_OUT, LDS, true, false><<<grid, dim3(256), 0, stream>>>(
            x, R, C, ld_x, offsets, G, ws, qt, ld_qt, s, s_rows, q, ld_q);
}

template <int FMT>
static fp8q_status_t dual_run(const uint16_t* x, int64_t R, int64_t C, int64_t ld_x,
                              const int32_t* offsets, int G, uint8_t* q, int64_t ld_q,
                              float* s_rows, uint8_t* qt, int64_t ld_qt, float* s_cols,
                              uint8_t* ws, hipStream_t stream) {
    size_t o_rowp, total;
    dual_layout(R, C, G, o_rowp, total);
    uint32_t* amax = reinterpret_cast<uint32_t*>(ws);
    uint16_t* rowp = reinterpret_cast<uint16_t*>(ws + o_rowp);
    const bool vec = (C % 8 == 0) && (ld_x % 8 == 0) && fp8q_aligned(x, 16);
    const bool vec_out = (ld_qt % 16 == 0) && fp8q_aligned(qt, 16);
    const bool rowq_vec = (C % 8 == 0) && (ld_q % 8 == 0) && fp8q_aligned(q, 8);
    const bool lds = G <= CW_GLDS;
    const int64_t n = (int64_t)G * C;
    int64_t zb = (n + 255) / 256;
    if (zb > 4096) zb = 4096;
    cw_zero_kernel<<<dim3((unsigned)zb), dim3(256), 0, stream>>>(amax, n);
    if (R > 0) {
        const unsigned strips = (unsigned)((C + CW_TC - 1) / CW_TC);
        // the cast pass re-reads the input: streaming loads only past the last-level cache size
        const bool nt = (double)R * (double)ld_x * 2.0 > kStreamBytes;
        const int tpb = amax_tpb(R, C);
        if (vec && lds && nt)
            launch_amax<true, true, true, true>(tpb, x, R, C, ld_x, offsets, G, amax, rowp, stream);
        else if (vec && lds)
            launch_amax<true, true, false, true>(tpb, x, R, C, ld_x, offsets, G, amax, rowp, stream);
        else if (vec && nt)
            launch_amax<true, false, true, true>(4, x, R, C, ld_x, offsets, G, amax, rowp, stream);
        else if (vec)
            launch_amax<true, false, false, true>(4, x, R, C, ld_x, offsets, G, amax, rowp, stream);
        else if (lds)
            launch_amax<false, true, false, true>(4, x, R, C, ld_x, offsets, G, amax, rowp, stream);
        else
            launch_amax<false, false, false, true>(4, x, R, C, ld_x, offsets, G, amax, rowp, stream);
        dual_rowscale_kernel<FMT><<<dim3((unsigned)((R + 63) / 64)), dim3(256), 0, stream>>>(
            rowp, R, (int)strips, s_rows);
    }
    if (vec && vec_out && lds)
        launch_cast_dual<FMT, true, true, true>(x, R, C, ld_x, offsets, G, amax, qt, ld_qt, s_cols, s_rows, q, ld_q, rowq_vec, stream);
    else if (vec && vec_out)
        launch_cast_dual<FMT, true, true, false>(x, R, C, ld_x, offsets, G, amax, qt, ld_qt, s_cols, s_rows, q, ld_q, rowq_vec, stream);
    else if (vec && lds)
        launch_cast_dual<FMT, true, false, true>(x, R, C, ld_x, offsets, G, amax, qt, ld_qt, s_cols, s_rows, q, ld_q, rowq_vec, stream);
    else if (vec)
        launch_cast_dual<FMT, true, false, false>(x, R, C, ld_x, offsets, G, amax, qt, ld_qt, s_cols, s_rows, q, ld_q, rowq_vec, stream);
    else if (vec_out && lds)
        launch_cast_dual<FMT, false, true, true>(x, R, C, ld_x, offsets, G, amax, qt, ld_qt, s_cols, s_rows, q, ld_q, rowq_vec, stream);
    else if (vec_out)
        launch_cast_dual<FMT, false, true, false>(x, R, C, ld_x, offsets, G, amax, qt, ld_qt, s_cols, s_rows, q, ld_q, rowq_vec, stream);
    else if (lds)
        launch_cast_dual<FMT, false, false, true>(x, R, C, ld_x, offsets, G, amax, qt, ld_qt, s_cols, s_rows, q, ld_q, rowq_vec, stream);
    else
        launch_cast_dual<FMT, false, false, false>(x, R, C, ld_x, offsets, G, amax, qt, ld_qt, s_cols, s_rows, q, ld_q, rowq_vec, stream);
    FP8Q_CHECK_LAUNCH();
    return FP8Q_OK;
}

}  // namespace fp8q

extern "C" size_t fp8_quant_dual_grouped_workspace_size(int64_t rows, int64_t cols,
                                                        int32_t groups) {
    if (rows < 0 || cols < 0 || groups < 1) return 0;
    size_t o, total;
    fp8q::dual_layout(rows, cols, groups, o, total);
    return total < 256 ? 256 : total;
}

extern "C" fp8q_status_t fp8_quant_dual_grouped(const uint16_t* x, int64_t rows, int64_t cols,
                                                int64_t ld_x, const int32_t* offsets,
                                                int32_t groups, fp8q_format_t fmt, uint8_t* q,
                                                int64_t ld_q, float* s_rows, uint8_t* q_t,
                                                int64_t ld_qt, float* s_cols, void* workspace,
                                                size_t workspace_bytes, hipStream_t stream) {
    if (rows < 0 || cols < 0 || groups < 1 || ld_x < cols || ld_q < cols || ld_qt < rows ||
        !fp8q_fmt_ok(fmt) || !offsets)
        return FP8Q_ERR_INVALID_ARG;
    if (cols == 0) return FP8Q_OK;
    if (!s_cols || (rows > 0 && (!x || !q || !s_rows || !q_t))) return FP8Q_ERR_INVALID_ARG;
    if (workspace_bytes < fp8_quant_dual_grouped_workspace_size(rows, cols, groups) || !workspace)
        return FP8Q_ERR_WORKSPACE;
    if (!fp8q_aligned(workspace, 16)) return FP8Q_ERR_INVALID_ARG;  // 16-byte row-maxima stores
    if ((rows + fp8q::CW_TR - 1) / fp8q::CW_TR > 0x7FFFFFFFLL ||
        (cols + fp8q::CW_TC - 1) / fp8q::CW_TC > 65535)
        return FP8Q_ERR_UNSUPPORTED;
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    if (fmt == FP8Q_E4M3FN)
        return fp8q::dual_run<FP8Q_E4M3FN>(x, rows, cols, ld_x, offsets, groups, q, ld_q, s_rows,
                                           q_t, ld_qt, s_cols, ws, stream);
    return fp8q::dual_run<FP8Q_E4M3FNUZ>(x, rows, cols, ld_x, offsets, groups, q, ld_q, s_rows,
                                         q_t, ld_qt, s_cols, ws, stream);
}

namespace fp8q {

// Argument checks and dispatch shared by both colwise entry points.
static fp8q_status_t colwise_entry(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                                   const int32_t* offsets, int32_t groups, fp8q_format_t fmt,
                                   uint8_t* q_t, int64_t ld_qt, float* scales, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream) {
    if (rows < 0 || cols < 0 || groups < 1 || ld_x < cols || ld_qt < rows || !fp8q_fmt_ok(fmt))
        return FP8Q_ERR_INVALID_ARG;
    if (!offsets) return FP8Q_ERR_INVALID_ARG;
    if (cols == 0) return FP8Q_OK;
    if (!scales || (rows > 0 && (!x || !q_t))) return FP8Q_ERR_INVALID_ARG;
    const size_t need = fp8_quant_colwise_grouped_workspace_size(rows, cols, groups);
    if (workspace_bytes < need || !workspace) return FP8Q_ERR_WORKSPACE;
    if ((rows + CW_TR - 1) / CW_TR > 0x7FFFFFFFLL || (cols + CW_TC - 1) / CW_TC > 65535)
        return FP8Q_ERR_UNSUPPORTED;
    uint32_t* ws = static_cast<uint32_t*>(workspace);
    if (fmt == FP8Q_E4M3FN)
        return colwise_run<FP8Q_E4M3FN>(x, rows, cols, ld_x, offsets, groups, q_t, ld_qt, scales,
                                        ws, stream);
    return colwise_run<FP8Q_E4M3FNUZ>(x, rows, cols, ld_x, offsets, groups, q_t, ld_qt, scales,
                                      ws, stream);
}

// Cross-block maxima of fp8_quant_colwise_grouped_noalloc: one array per GPU, held until the
// process ends.  In host code this name is only a stand-in for the device symbol, never an
// address: the device address of each GPU's copy comes from hipGetSymbolAddress, taken once per
// device with that device current, and is what the kernels receive.
static __device__ __align__(256) uint32_t scratch[FP8Q_NOALLOC_SCRATCH_BYTES / sizeof(uint32_t)];
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[64];

static fp8q_status_t noalloc_scratch(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return FP8Q_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FP8Q_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return FP8Q_OK;
}

}  // namespace fp8q

extern "C" fp8q_status_t fp8_quant_colwise_grouped(const uint16_t* x, int64_t rows, int64_t cols,
                                                   int64_t ld_x, const int32_t* offsets,
                                                   int32_t groups, fp8q_format_t fmt,
                                                   uint8_t* q_t, int64_t ld_qt, float* scales,
                                                   void* workspace, size_t workspace_bytes,
                                                   hipStream_t stream) {
    return fp8q::colwise_entry(x, rows, cols, ld_x, offsets, groups, fmt, q_t, ld_qt, scales,
                               workspace, workspace_bytes, stream);
}

extern "C" fp8q_status_t fp8_quant_colwise_grouped_noalloc(const uint16_t* x, int64_t rows,
                                                           int64_t cols, int64_t ld_x,
                                                           const int32_t* offsets,
                                                           int32_t groups, fp8q_format_t fmt,
                                                           uint8_t* q_t, int64_t ld_qt,
                                                           float* scales, hipStream_t stream) {
    // sizes beyond the static array are rejected before anything else touches the device
    if (cols > 0 && groups >= 1 &&
        fp8_quant_colwise_grouped_workspace_size(rows, cols, groups) > FP8Q_NOALLOC_SCRATCH_BYTES)
        return FP8Q_ERR_WORKSPACE;
    void* ws = nullptr;
    const fp8q_status_t st = fp8q::noalloc_scratch(&ws);
    if (st != FP8Q_OK) return st;
    return fp8q::colwise_entry(x, rows, cols, ld_x, offsets, groups, fmt, q_t, ld_qt, scales, ws,
                               FP8Q_NOALLOC_SCRATCH_BYTES, stream);
}

extern "C" size_t fp8_quant_weights_dual_workspace_size(int64_t experts, int64_t K, int64_t N) {
    if (experts < 0 || K < 0 || N < 0) return 0;
    size_t a, b, total;
    fp8q::wdual_layout(experts, K, N, a, b, total);
    return total < 256 ? 256 : total;
}

extern "C" fp8q_status_t fp8_quant_weights_dual(const uint16_t* w, int64_t experts, int64_t K,
                                                int64_t N, int64_t ld_w, fp8q_format_t fmt,
                                                uint8_t* q_rows, int64_t ld_qr, float* s_rows,
                                                uint8_t* q_t, int64_t ld_qt, float* s_cols,
                                                void* workspace, size_t workspace_bytes,
                                                hipStream_t stream) {
    if (experts < 0 || K < 0 || N < 0 || ld_w < N || ld_qr < N || ld_qt < experts * K ||
        !fp8q_fmt_ok(fmt))
        return FP8Q_ERR_INVALID_ARG;
    if (experts == 0 || K == 0 || N == 0) return FP8Q_OK;
    if (!w || !q_rows || !s_rows || !q_t || !s_cols) return FP8Q_ERR_INVALID_ARG;
    const int64_t nb = (K + fp8q::WD_RB - 1) / fp8q::WD_RB;
    if (N > fp8q::WD_NMAX || N % 8 || ld_w % 8 || ld_qr % 8 || !fp8q_aligned(w, 16) ||
        !fp8q_aligned(q_rows, 8) || experts * nb > 0x7FFFFFFFLL ||
        experts * K > 0x7FFFFFFFLL || experts > 0x7FFFFFFFLL / 256 ||
        (experts * K + fp8q::CW_TR - 1) / fp8q::CW_TR > 0x7FFFFFFFLL ||
        (N + fp8q::CW_TC - 1) / fp8q::CW_TC > 65535)
        return FP8Q_ERR_UNSUPPORTED;
    size_t o_offs, o_part, total;
    fp8q::wdual_layout(experts, K, N, o_offs, o_part, total);
    if (!workspace || workspace_bytes < total) return FP8Q_ERR_WORKSPACE;
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    uint32_t* amax = reinterpret_cast<uint32_t*>(ws);
    int32_t* offs = reinterpret_cast<int32_t*>(ws + o_offs);
    uint16_t* part = reinterpret_cast<uint16_t*>(ws + o_part);
    const bool nt_out = (double)experts * (double)K * (double)ld_qr > fp8q::kStreamBytes;
    const int64_t R = experts * K;
    const bool vec_out = (ld_qt % 16 == 0) && fp8q_aligned(q_t, 16);
    const int64_t nred = (experts * N > experts ? experts * N : experts);
    if (fmt == FP8Q_E4M3FN)
        fp8q::wdual_rows_kernel<FP8Q_E4M3FN><<<dim3((unsigned)(experts * nb)), dim3(64 * fp8q::WD_NW), 0, stream>>>(
            w, K, N, ld_w, nb, q_rows, ld_qr, s_rows, part, nt_out);
    else
        fp8q::wdual_rows_kernel<FP8Q_E4M3FNUZ><<<dim3((unsigned)(experts * nb)), dim3(64 * fp8q::WD_NW), 0, stream>>>(
            w, K, N, ld_w, nb, q_rows, ld_qr, s_rows, part, nt_out);
    fp8q::wdual_colmax_kernel<<<dim3((unsigned)((nred + 255) / 256)), dim3(256), 0, stream>>>(
        part, nb, experts, N, K, amax, offs);
    if (fmt == FP8Q_E4M3FN) {
        if (vec_out)
            fp8q::launch_cast<FP8Q_E4M3FN, true, true>(w, R, N, ld_w, offs, (int)experts, amax, q_t, ld_qt, s_cols, stream);
        else
            fp8q::launch_cast<FP8Q_E4M3FN, true, false>(w, R, N, ld_w, offs, (int)experts, amax, q_t, ld_qt, s_cols, stream);
    } else {
        if (vec_out)
            fp8q::launch_cast<FP8Q_E4M3FNUZ, true, true>(w, R, N, ld_w, offs, (int)experts, amax, q_t, ld_qt, s_cols, stream);
        else
            fp8q::launch_cast<FP8Q_E4M3FNUZ, true, false>(w, R, N, ld_w, offs, (int)experts, amax, q_t, ld_qt, s_cols, stream);
    }
    FP8Q_CHECK_LAUNCH();
    return FP8Q_OK;
}
