// Scaled FP8 grouped GEMM on gfx950 matrix cores, with the dequantization fused into the
// epilogue (latestnews.news "AMD Boosts PyTorch FP8 Training on Instinct GPUs", third
// paragraph: grouped GEMM for MoE on ROCm; ai-radar.it "FP8 su GPU AMD ...", introduction:
// rowwise activation scales, colwise expert-weight scales and the token offsets that route rows
// to experts; fosswire.org "AMD Primus adds FP8/MXFP8 kernels ...", section "What Primus adds
// for MoE training on MI355X": FP8 and MXFP8 grouped GEMM for the expert FFNs).
//
// Both operands are contraction-contiguous byte matrices:
//   forward, M-grouped:  out[m,n]   = sum_k A[m,k] * B_g[n,k] / (sa[m] * sb[g,n]),  m in group g
//   wgrad, K-grouped:    out[g,k,n] = sum_{m in g} A[k,m] * B[n,m] / (sa[g,k] * sb[g,n])
//   MX forward:          out[m,n]   = sum_kb 2^(ea+eb) sum_{k in kb} A[m,k] * B_g[n,k]
//
// Kernel (persistent: one block per CU):
//   * 256x256 output tile, 128-byte contraction steps.  Plain FP8: 16 waves, four per SIMD,
//     each owning a 128x32 sub-tile (16 v_mfma_f32_16x16x128_f8f6f4 per step, 64 accumulators
//     per lane), so the other waves' matrix instructions cover one wave's LDS reads, DMA issue
//     and waits (one wave per SIMD is bound by its own instruction issue, not by the matrix
//     cores).  MX with its scales by DMA: the same 16 waves; MX with byte-loaded scales: 8
//     waves, two per SIMD, each 128x64 (32 MFMAs per step, 128 accumulators).
//   * Operand tiles go HBM/L2 -> LDS directly with buffer_load_dwordx4 ... lds (no staging
//     registers), double-buffered: after the barrier of step k the loads of step k+1 are
//     issued in 32 parts of 8 rows x 128 bytes per operand (16 waves: 2 parts each; 8 waves:
//     4 parts each; all before the wave's first matrix instruction of the step), and
//     waited for only at the top of step k+1, so one barrier per step.
//     Rows and chunks outside the operand are turned into out-of-range buffer offsets and read
//     back as zeros.  Chunks are stored XOR-swizzled
//     per row (swz, swzB) so that every fragment read is free of LDS bank conflicts.
//   * The MFMA's A operand is the N-side tile and its B operand the M-side tile; N-side rows
//     are permuted in LDS (brow) so that each lane ends with 8 consecutive output columns of
//     one row, stored as one 16-byte bf16 octet.
//   * Operand lane layout of the 16x16x128 f8f6f4 instruction on gfx950 (established with
//     one-hot inputs): lane l holds row l%16; its bytes 0-15 are K offsets 16*(l/16)+[0,16) and
//     bytes 16-31 are K offsets 64+16*(l/16)+[0,16); lane r+16b supplies the E8M0 scale of row
//     r, K block b.
//   * Accumulation: the matrix cores add each 32-product block in fixed point whose last bit
//     is 2^-13 of the block's largest product (products truncated toward zero) and combine
//     block sums in fp32 (measured on gfx950; the same for the older fp8 instruction).
//
// e4m3fnuz operands: the matrix cores read OCP e4m3 only (byte 0x7F, the fnuz 240 code, is NaN
// there), so fnuz bytes are re-encoded in LDS, once per step by the lanes that loaded them, to
// the e4m3fn byte of the same value: exponent field - 1 for fnuz exponents >= 2 (exact), and
// the nearest e4m3fn subnormal (ties to even) for fnuz values below 2^-6, which moves a product
// by at most 2^-10 quantization units.  (Re-encoding every fragment after its LDS read instead
// costs each wave ~12 VALU operations per fragment dword: the e4m3fnuz GEMMs ran 4x slower.)
//
// Weight gradient: a group's token range starts and ends anywhere, so the chunk holding the
// first (last) token of the group can carry neighbouring groups' bytes; those bytes of the
// activation operand are zeroed in LDS on the (at most two) edge steps of a tile.
//
// Group scheduling stays on the device (no host read of the offsets): each block scans the
// per-group tile counts (forward) or work units (weight gradient, groups ordered by size,
// largest first) in LDS, takes an even share of the work for its XCD, and walks its tiles.
// Offsets are clamped into [0, M] before use, so any offsets content keeps every access in
// range.
#include <type_traits>

#include "common.hpp"

namespace fp8q {

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v4f_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int GT = 256;         // output tile edge (rows and columns)

constexpr int GK = 128;         // contraction bytes per step
constexpr int STAGE = GT * GK;  // bytes of one operand tile in LDS
constexpr uint32_t OOB = 0x80000000u;
constexpr int MODE_FWD = 0, MODE_WGRAD = 1;

// 16-byte slot of chunk c in row r: c ^ (2*((r >> 2) & 3) + ((r >> 1) & 1)).  A fragment read
// is served as two 32-lane halves, each touching 16 consecutive rows at chunks kg ^ s and
// (kg+1) ^ s; the rows that share a 512-byte LDS window (same r & 3) get distinct
// 2*((r >> 2) & 3), so all 32 16-byte slots of a half are distinct (no bank conflicts).
__device__ __forceinline__ int swz(int r) { return (((r >> 2) & 3) << 1) | ((r >> 1) & 1); }
__device__ __forceinline__ int lds_off(int r, int ch) { return r * GK + ((ch ^ swz(r)) << 4); }
// N-side tile: its fragments take rows 32j' + 8q + 4h + e (q = lane%16 / 4, e = lane%4) so that
// each lane's results are 8 consecutive output columns; slot c ^ (2*((r>>3)&3) + ((r>>1)&1))
// puts those 16 rows in 16 distinct 16-byte bank slots.
__device__ __forceinline__ int swzB(int r) { return (((r >> 3) & 3) << 1) | ((r >> 1) & 1); }
__device__ __forceinline__ int lds_offB(int r, int ch) { return r * GK + ((ch ^ swzB(r)) << 4); }
// Row of the N-side tile that feeds MFMA row lr of column block j (see swzB).
__device__ __forceinline__ int brow(int j, int lr) {
    return 32 * (j >> 1) + 8 * (lr >> 2) + 4 * (j & 1) + (lr & 3);
}

typedef int i32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4_t make_rsrc4(const void* base, uint32_t bytes) {
    const uint64_t a = (uint64_t)base;  // block-uniform: keep the descriptor in SGPRs
    return i32x4_t{__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
                   __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32)),
                   __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000};
}
// 16 bytes per lane from a buffer straight into LDS at lds_base + 16*lane (lds_base is
// wave-uniform).  Written as inline assembly so that the compiler does not order every later
// LDS read after it: the waits are explicit (s_waitcnt vmcnt before the step's barrier).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(i32x4_t rsrc, uint32_t voff, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds_base), "v"(voff), "s"(rsrc)
                 : "memory", "m0");
}
#pragma clang diagnostic pop
__device__ __forceinline__ void dma4(i32x4_t rsrc, uint32_t voff, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                 :
                 : "s"(lds_base), "v"(voff), "s"(rsrc)
                 : "memory", "m0");
}
__device__ __forceinline__ void wait_vm0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_ptr_t)p);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
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

// Bytes at positions base..base+3 of a chunk kept where lo <= pos < hi.
__device__ __forceinline__ uint32_t keep_mask4(int lo, int hi, int base) {
    int a = lo - base, b = hi - base;
    a = a < 0 ? 0 : (a > 4 ? 4 : a);
    b = b < 0 ? 0 : (b > 4 ? 4 : b);
    const uint32_t below_b = b >= 4 ? 0xFFFFFFFFu : ((1u << (8 * b)) - 1u);
    const uint32_t from_a = a >= 4 ? 0u : (0xFFFFFFFFu << (8 * a));
    return below_b & from_a;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    uint32_t a = __float_as_uint(lo), b = __float_as_uint(hi);
    a += 0x7FFFu + ((a >> 16) & 1u);
    b += 0x7FFFu + ((b >> 16) & 1u);
    return (a >> 16) | (b & 0xFFFF0000u);
}

template <bool NSIDE>
__device__ __forceinline__ v8i_t frag(const uint8_t* tile, int r, int kg, bool fnuz) {
    const uint4 lo = *reinterpret_cast<const uint4*>(tile + (NSIDE ? lds_offB(r, kg) : lds_off(r, kg)));
    const uint4 hi =
        *reinterpret_cast<const uint4*>(tile + (NSIDE ? lds_offB(r, 4 + kg) : lds_off(r, 4 + kg)));
    v8i_t f = v8i_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                    (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    if (fnuz) {
#pragma unroll
        for (int i = 0; i < 8; i++) f[i] = (int)fnuz_to_fn4((uint32_t)f[i]);
    }
    return f;
}

struct GemmArgs {
    const uint8_t* a;
    int64_t lda;
    const float* a_scales;
    const uint8_t* a_e8;
    int64_t ld_sa;
    const uint8_t* b;
    int64_t ldb;
    int64_t bgs;
    const float* b_scales;
    const uint8_t* b_e8;
    int64_t ld_sb;
    int64_t sbgs;
    const int32_t* offsets;
    int G;
    int64_t M, N, K;
    uint8_t* c;       // bf16 or fp32 elements (out_f32), row stride ldc elements
    int64_t ldc;
    int32_t* status;  // offsets check result (two words), written by block 0
    int nt_n;         // column tiles
    int nt_k;         // wgrad: row tiles along K
    bool out_f32;     // fp32 output instead of bf16
    bool vec_store;   // N, ldc multiples of 8 and c 16-byte aligned: whole 16-byte stores
};

constexpr int GMAX = 2048;  // groups whose schedule prefix fits in LDS

struct Tile {  // all extents < 2^31 (checked on the host)
    int g, par;  // group; parity of the tile in the block's sequence (scale buffer)
    int mx_slot;  // MX_DMA: slot of the tile's first 4-step scale chunk
    int raw_lo, raw_hi;  // the group's offsets as loaded (before clamping)
    int row_lo, row_hi, n0, kb_lo, kb_hi, kstart, nk, a_rows, b_rows;
};

// One block per CU runs its share of the tile sequence (persistent schedule; see the schedule
// comments in the kernel).  The first contraction step of a block's next tile is fetched while
// the current tile finishes.
// MX scale loading: none (plain FP8); per-step byte loads into registers (any scale strides);
// one 16-byte DMA per row and side every 4 contraction steps (16-byte aligned scale rows, the
// forward); or one dword DMA per row and side per step (MX_DW: 4-byte aligned scale rows, the
// weight gradient, whose tiles then start on 128-token boundaries so that a step's 4 scale
// bytes are one aligned dword).
constexpr int MX_NONE = 0, MX_BYTES = 1, MX_DMA = 2, MX_DW = 3;

template <int FMT, int MODE, int MXV, int NW>
__global__ __launch_bounds__(64 * NW, 1) void gemm256_kernel(const GemmArgs p) {
    constexpr bool MX = MXV != MX_NONE;
    // prefix sums: forward row-tile slots, weight-gradient work units; both < 2^31 (checked
    // on the host)
    typedef int pref_t;
    // group offsets staged in LDS once, except for the MX kernel whose LDS holds the scale
    // chunks instead (its tiles are long, so the per-tile offsets loads do not matter there)
    constexpr bool OFF_LDS = MXV != MX_DMA;
    __shared__ __align__(16) uint8_t smem[2][2][STAGE];
    // MX_BYTES, MX_DW: 4 E8M0 bytes per row and step (by stage); otherwise the fp32 dequant
    // scales of the tile's rows [0] and columns [1] (by tile parity)
    __shared__ __align__(16) uint32_t sscale[2][2][GT];
    // MX_DMA: E8M0 bytes of 4 steps (16 K blocks) per row: [slot][side][row][16]
    __shared__ __align__(16) uint8_t smx[MXV == MX_DMA ? 2 * 2 * GT * 16 : 16];
    __shared__ pref_t s_pref[GMAX + 1];                    // per-group prefix of tiles / work
    __shared__ int s_off[OFF_LDS ? GMAX : 1];               // offsets as given (unclamped)
    pref_t* s_part = reinterpret_cast<pref_t*>(&smem[1][0][0]);  // scan scratch (set-up only)
    // weight gradient: groups in schedule order (most contraction steps first)
    __shared__ unsigned short s_perm[MODE == MODE_WGRAD ? GMAX : 1];
    __shared__ int s_bad;                                   // offsets check (block 0)
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    // NW = 4: each wave owns 128 x 128 of the tile; NW = 8: 128 x 64; NW = 16: 128 x 32
    static_assert(NW == 4 || NW == 8 || NW == 16, "4, 8 or 16 waves");
    constexpr int NT = 64 * NW;          // threads
    constexpr int NP = 32 / NW;          // operand DMA parts per wave and step (8 rows each)
    constexpr int NJ = NW == 16 ? 2 : NW == 8 ? 4 : 8;  // 16-column blocks per wave
    constexpr int WNC = 16 * NJ;         // columns per wave
    const bool row_thread = NW == 4 || wave < 4;  // threads owning one tile row (t < 256; wave-uniform)
    const int wm = wave / (NW / 2), wn = wave % (NW / 2);
    constexpr bool FNUZ = FMT == FP8Q_E4M3FNUZ;
    const int64_t tiles_per_group = (int64_t)p.nt_k * p.nt_n;
    // weight gradient: a tile's contraction starts at its group's first token rounded down to
    // 16 (one LDS chunk), or to 32 for MX so that the steps' 32-token blocks are the scale blocks
    // (128 with dword scale DMA: a step's four scale bytes are then one aligned dword)
    constexpr int64_t KALIGN = MXV == MX_DW ? 127 : MX ? 31 : 15;

    if (OFF_LDS) {
        for (int i = t; i < p.G; i += NT) s_off[i] = p.offsets[i];
        __syncthreads();
    }
    auto off_at = [&](int g) -> int { return OFF_LDS ? s_off[g] : p.offsets[g]; };
    // Offsets check, block 0: the first group whose end lies below its start or past M, or a
    // last end other than M, is reported in status[1] (status[0] = FP8Q_ERR_INVALID_ARG);
    // valid offsets give {FP8Q_OK, -1}.  The kernel itself only ever uses clamped offsets, so
    // invalid ones change results but never the memory accessed.
    if (p.status != nullptr && blockIdx.x == 0) {
        if (t == 0) s_bad = 0x7FFFFFFF;
        __syncthreads();
        for (int i = t; i < p.G; i += NT) {
            const int64_t lo = i == 0 ? 0 : (int64_t)off_at(i - 1);
            const int64_t hi = off_at(i);
            if (hi < lo || hi > p.M || (i == p.G - 1 && hi != p.M)) atomicMin(&s_bad, i);
        }
        __syncthreads();
        if (t == 0) {
            const int bad = s_bad;
            p.status[0] = bad == 0x7FFFFFFF ? (int32_t)FP8Q_OK : (int32_t)FP8Q_ERR_INVALID_ARG;
            p.status[1] = bad == 0x7FFFFFFF ? -1 : bad;
        }
    }
    // group g's token rows, clamped into [0, M] so that any offsets content stays in range
    auto rows_of = [&](int g, int64_t& lo, int64_t& hi) {
        lo = g == 0 ? 0 : (int64_t)off_at(g - 1);
        lo = lo < 0 ? 0 : (lo > p.M ? p.M : lo);
        hi = off_at(g);
        hi = hi < lo ? lo : (hi > p.M ? p.M : hi);
    };
    // --- weight gradient: order the groups by contraction steps, largest first, so that the
    // evenly split ranges end with short tiles (longest-processing-time order); bitonic sort of
    // (steps, group) keys in the not yet used operand buffer
    if (MODE == MODE_WGRAD) {
        long long* key = reinterpret_cast<long long*>(&smem[0][0][0]);  // 16 KB of 32 KB
        int n = 1;
        while (n < p.G) n <<= 1;
        for (int i = t; i < n; i += NT) {
            long long k = -1;  // padding sorts last
            if (i < p.G) {
                int64_t lo, hi;
                rows_of(i, lo, hi);
                const int64_t ks = lo & ~KALIGN;
                const int64_t nk = hi > ks ? (hi - ks + GK - 1) / GK : 0;
                k = ((long long)nk << 11) | (long long)(GMAX - 1 - i);
            }
            key[i] = k;
        }
        __syncthreads();
        for (int kb = 2; kb <= n; kb <<= 1) {
            for (int j = kb >> 1; j > 0; j >>= 1) {
                for (int i = t; i < n; i += NT) {
                    const int l = i ^ j;
                    if (l > i) {
                        const long long a = key[i], b = key[l];
                        if ((i & kb) == 0 ? a < b : a > b) {
                            key[i] = b;
                            key[l] = a;
                        }
                    }
                }
                __syncthreads();
            }
        }
        for (int i = t; i < p.G; i += NT)
            s_perm[i] = (unsigned short)(GMAX - 1 - (int)(key[i] & (GMAX - 1)));
        __syncthreads();
    }
    auto group_at = [&](int pos) -> int { return MODE == MODE_WGRAD ? (int)s_perm[pos] : pos; };

    // --- forward schedule prefix: row-tile slots per group
    if (t == 0) s_pref[0] = 0;
    pref_t base = 0;
    for (int g0 = 0; MODE == MODE_FWD && g0 < p.G; g0 += 256) {
        const int gg = g0 + t;  // threads 0..255 scan one chunk of 256 groups
        pref_t cnt = 0;
        if (row_thread && gg < p.G) {
            int64_t lo, hi;
            rows_of(group_at(gg), lo, hi);
            if (MODE == MODE_FWD) {
                cnt = (hi - lo + GT - 1) / GT;
            } else {
                const int64_t ks = lo & ~(int64_t)15;
                const int64_t nk = hi > ks ? (hi - ks + GK - 1) / GK : 0;
                cnt = tiles_per_group * (nk + 1);
            }
        }
        __syncthreads();
        if (row_thread) s_part[t] = cnt;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {
            const pref_t add = (row_thread && t >= off) ? s_part[t - off] : 0;
            __syncthreads();
            if (row_thread) s_part[t] += add;
            __syncthreads();
        }
        if (row_thread && gg < p.G) s_pref[gg + 1] = base + s_part[t];
        base += s_part[255];
    }
    __syncthreads();
    // Forward: every tile costs the same, so the row-tile slots x column tiles are split evenly
    // over the XCDs (blocks are dealt to the 8 XCDs round-robin) and dealt round-robin to the
    // blocks inside each XCD's contiguous range: tiles running at the same moment are
    // neighbours and share operand tiles in that XCD's L2.
    // Weight gradient: tiles cost (steps + epilogue) and differ by group, so they are taken in
    // the size order above, one round of gridDim tiles at a time, alternating the direction
    // of each round (longest processing time first, snake order).
    const int nb = gridDim.x;
    int ti = 0, t_end = 0, bpx = 1, round = 0, par_next = 0;
    if (MODE == MODE_FWD) {
        const long long total = (long long)s_pref[p.G] * p.nt_n;  // < 2^31 (host check)
        const int nx = nb % 8 == 0 ? 8 : 1;
        const int xcd = nx == 8 ? (int)(blockIdx.x % 8) : 0;
        const int lb = nx == 8 ? (int)(blockIdx.x / 8) : (int)blockIdx.x;
        bpx = nb / nx;  // blocks per XCD
        ti = (int)(total * xcd / nx) + lb;
        t_end = (int)(total * (xcd + 1) / nx);
    }
    const int w_tiles = MODE == MODE_WGRAD ? p.G * (int)tiles_per_group : 0;  // < 2^31 (host)
    int mx_next_slot = 0;
    // The block's next tile, in two halves: tile_start picks the tile and reads its group's
    // offsets; tile_finish (called later, after other work) derives its extents.  Returns
    // false when the block's share is exhausted.
    auto tile_start = [&](Tile& T) -> bool {
        if (MODE == MODE_FWD) {
            if (ti >= t_end) return false;
            // the row tiles sharing a weight tile run side by side in one XCD
            int lo = 0, hi = p.G - 1;  // last group whose tiles start at or before ti
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (s_pref[mid] * p.nt_n <= ti) lo = mid; else hi = mid - 1;
            }
            T.g = lo;
            const int rt = s_pref[lo + 1] - s_pref[lo];  // row tiles of the group (> 0 here)
            const int l = ti - s_pref[lo] * p.nt_n;
            // bands of up to 8 row tiles, each band ordered (column tile, row tile) with the row
            // tile fastest: an XCD's 32 concurrent tiles cover 4 columns x 8 rows of a large
            // group (12 distinct operand tiles instead of up to 33 for one column of row tiles;
            // dense 8192 x 4096 x 14336: 493 -> 448 us)
            constexpr int BAND = 8;
            const int bt = BAND * p.nt_n, b = l / bt, r = l - b * bt;
            const int rows_b = rt - b * BAND < BAND ? rt - b * BAND : BAND;
            T.n0 = (r / rows_b) * GT;
            T.row_lo = (b * BAND + r % rows_b) * GT;  // relative to the group start
            ti += bpx;
        } else {
            // round r takes tiles [r*nb, r*nb + nb) of the size order; XCD x (blocks are dealt
            // to the 8 XCDs round-robin) takes one contiguous chunk of them, so the blocks of an
            // XCD work on neighbouring tiles (shared operand rows in its L2); chunk and position
            // inside the chunk alternate direction from round to round
            int idx;
            if (nb % 8 == 0) {
                const int cpx = nb / 8, x = (int)blockIdx.x % 8, j = (int)blockIdx.x / 8;
                const int chunk = (round & 1) ? 7 - x : x;
                idx = round * nb + chunk * cpx + ((round & 1) ? cpx - 1 - j : j);
            } else {
                idx = round * nb + ((round & 1) ? nb - 1 - (int)blockIdx.x : (int)blockIdx.x);
            }
            if (idx >= w_tiles) return false;
            round++;
            const int tpg = (int)tiles_per_group;
            T.g = group_at(idx / tpg);
            const int l = idx % tpg;
            T.row_lo = (l / p.nt_n) * GT;
            T.n0 = (l % p.nt_n) * GT;
        }
        T.raw_lo = T.g == 0 ? 0 : off_at(T.g - 1);
        T.raw_hi = off_at(T.g);
        T.par = par_next;
        par_next ^= 1;
        return true;
    };
    auto tile_finish = [&](Tile& T) {
        // the group's token rows, clamped into [0, M] so that any offsets content stays in range
        int64_t glo = T.raw_lo, ghi = T.raw_hi;
        glo = glo < 0 ? 0 : (glo > p.M ? p.M : glo);
        ghi = ghi < glo ? glo : (ghi > p.M ? p.M : ghi);
        if (MODE == MODE_FWD) {
            T.row_lo = (int)(glo + T.row_lo);
            T.row_hi = T.row_lo + GT < ghi ? T.row_lo + GT : (int)ghi;
            T.kb_lo = 0;
            T.kb_hi = (int)p.K;
            T.kstart = 0;
            T.a_rows = T.row_hi - T.row_lo;
        } else {
            T.row_hi = T.row_lo + GT < p.K ? T.row_lo + GT : (int)p.K;
            T.kb_lo = (int)glo;
            T.kb_hi = (int)ghi;
            T.kstart = (int)(glo & ~KALIGN);
            T.a_rows = T.row_hi - T.row_lo;
        }
        T.nk = T.kb_hi > T.kstart ? (T.kb_hi - T.kstart + GK - 1) / GK : 0;
        T.b_rows = p.N - T.n0 < GT ? (int)(p.N - T.n0) : GT;
        // scale chunks alternate between the two slots across the block's tiles
        T.mx_slot = mx_next_slot;
        mx_next_slot = (mx_next_slot + (T.nk + 3) / 4) & 1;
    };
    auto next_tile = [&](Tile& T) -> bool {
        if (!tile_start(T)) return false;
        tile_finish(T);
        return true;
    };

    uint32_t sa_pack = 0, sb_pack = 0;
    // A contraction step whose operand loads are still to be issued: buffer resources rebased
    // at the tile's first rows (offsets stay 32-bit) and the stage's LDS addresses.  Forward:
    // A's range ends at the tile's last row of its group (row_hi), so the rows of the next
    // group in a partial tile are not fetched; a DMA part whose 8 rows all lie past it is not
    // issued at all, and those LDS rows keep stale bytes, which only reach accumulator rows the
    // epilogue never stores (measured: forward 334 -> 322 us, data gradient 356 -> 322 us).
    struct Pend {
        i32x4_t ra, rb;
        uint32_t as, bs;
        int kpos, kb_lo, kb_hi, a_rows, b_rows;
    };
    // This lane's row in part i is row0 + 8i (row0 = 8*NP*wave + lane/8); with that row the
    // swizzles reduce to swz = 4*(i&1) + 2*((lane/32)&1) + ((lane/16)&1) and
    // swzB = 2*(i&3) + ((lane/16)&1) (general form where a wave has fewer than 4 parts).
    const int row0 = wave * (8 * NP) + (lane >> 3);
    const int l3 = lane >> 3;
    // Sets up the step starting at kpos of tile T for LDS stage `stage` and issues the scale
    // loads that ride along with it.
    auto prep = [&](const Tile& T, int kpos, int stage) -> Pend {
        Pend P;
        P.ra = make_rsrc4(p.a + (int64_t)T.row_lo * p.lda, (uint32_t)(T.a_rows * p.lda));
        P.rb = make_rsrc4(
            p.b + (MODE == MODE_FWD ? (int64_t)T.g * p.bgs : 0) + (int64_t)T.n0 * p.ldb,
            (uint32_t)(T.b_rows * p.ldb));
        P.as = lds_addr(smem[stage][0]);
        P.bs = lds_addr(smem[stage][1]);
        P.kpos = kpos;
        P.kb_lo = T.kb_lo;
        P.kb_hi = T.kb_hi;
        P.a_rows = T.a_rows;
        P.b_rows = T.b_rows;
        if (!MX && kpos == T.kstart) {
            // the tile's dequant scales (row t of each side) ride along with its first step;
            // waves 0-3 own the 256 rows (the LDS addresses are formed outside the branch)
            const int64_t sm0 = MODE == MODE_FWD ? (int64_t)T.row_lo : (int64_t)T.g * p.K + T.row_lo;
            const i32x4_t rsm = make_rsrc4(p.a_scales + sm0, (uint32_t)(T.row_hi - T.row_lo) * 4u);
            const i32x4_t rsn = make_rsrc4(p.b_scales + (int64_t)T.g * p.N + T.n0,
                                           (uint32_t)T.b_rows * 4u);
            const uint32_t dsm = lds_addr(&sscale[T.par][0][(wave & 3) * 64]);
            const uint32_t dsn = lds_addr(&sscale[T.par][1][(wave & 3) * 64]);
            if (row_thread) {
                dma4(rsm, (uint32_t)t * 4u, dsm);
                dma4(rsn, (uint32_t)t * 4u, dsn);
            }
        }
        if (MXV == MX_DMA && ((kpos - T.kstart) / GK) % 4 == 0 && row_thread) {
            // rows t of both tiles: the 16 E8M0 bytes of this step and the next three (K blocks
            // kpos/32 .. +15; a scale row is 16-byte aligned and at least that long, blocks past
            // K are never used)
            const int slot = (T.mx_slot + (kpos - T.kstart) / (4 * GK)) & 1;
            const i32x4_t rsa =
                make_rsrc4(p.a_e8 + (int64_t)T.row_lo * p.ld_sa, (uint32_t)(T.a_rows * p.ld_sa));
            const i32x4_t rsb =
                make_rsrc4(p.b_e8 + (int64_t)T.g * p.sbgs + (int64_t)T.n0 * p.ld_sb,
                           (uint32_t)(T.b_rows * p.ld_sb));
            const uint32_t kb0 = (uint32_t)(kpos / 32);
            const uint32_t oa = t < T.a_rows ? (uint32_t)t * (uint32_t)p.ld_sa + kb0 : OOB;
            const uint32_t ob = t < T.b_rows ? (uint32_t)t * (uint32_t)p.ld_sb + kb0 : OOB;
            dma16(rsa, oa, lds_addr(&smx[((slot * 2 + 0) * GT + wave * 64) * 16]));
            dma16(rsb, ob, lds_addr(&smx[((slot * 2 + 1) * GT + wave * 64) * 16]));
        }
        if (MXV == MX_DW && row_thread) {
            // rows t of both tiles: the 4 E8M0 bytes of this step (kpos is a multiple of 128, so
            // they are one aligned dword) straight into the stage's scale rows.  Blocks past
            // the group's end are replaced by 2^0 where they are read.
            const i32x4_t rsa =
                make_rsrc4(p.a_e8 + (int64_t)T.row_lo * p.ld_sa, (uint32_t)(T.a_rows * p.ld_sa));
            const i32x4_t rsb = make_rsrc4(p.b_e8 + (int64_t)T.g * p.sbgs + (int64_t)T.n0 * p.ld_sb,
                                           (uint32_t)(T.b_rows * p.ld_sb));
            const uint32_t kb0 = (uint32_t)(kpos / 32);
            const uint32_t oa = t < T.a_rows ? (uint32_t)t * (uint32_t)p.ld_sa + kb0 : OOB;
            const uint32_t ob = t < T.b_rows ? (uint32_t)t * (uint32_t)p.ld_sb + kb0 : OOB;
            dma4(rsa, oa, lds_addr(&sscale[stage][0][(wave & 3) * 64]));
            dma4(rsb, ob, lds_addr(&sscale[stage][1][(wave & 3) * 64]));
        }
        if (MXV == MX_BYTES && row_thread) {
            // rows t of both tiles: the 4 E8M0 bytes of this 128-byte step, packed into one
            // dword per row (blocks past K get 127 = 2^0: their data bytes are zero)
            const __amdgpu_buffer_rsrc_t rsa =
                make_rsrc(p.a_e8 + (int64_t)T.row_lo * p.ld_sa, (uint32_t)(T.a_rows * p.ld_sa));
            const __amdgpu_buffer_rsrc_t rsb =
                make_rsrc(p.b_e8 + (int64_t)T.g * p.sbgs + (int64_t)T.n0 * p.ld_sb,
                          (uint32_t)(T.b_rows * p.ld_sb));
            const int kb0 = kpos / 32;
            sa_pack = sb_pack = 0;
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const bool ok = kpos + 32 * j < (MODE == MODE_FWD ? p.K : p.M);
                const uint32_t oa = (ok && t < T.a_rows) ? (uint32_t)(t * p.ld_sa + kb0 + j) : OOB;
                const uint32_t ob = (ok && t < T.b_rows) ? (uint32_t)(t * p.ld_sb + kb0 + j) : OOB;
                const uint32_t ea =
                    ok ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rsa, oa, 0, 0) : 127u;
                const uint32_t eb =
                    ok ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rsb, ob, 0, 0) : 127u;
                sa_pack |= ea << (8 * j);
                sb_pack |= eb << (8 * j);
            }
        }
        return P;
    };
    // Operand loads of part i of a step: row group (wave*8 + i) of both tiles, 8 rows x 128
    // bytes per instruction; lane chunk goes to LDS slot (wave*8+i)*64 + lane.
    auto part = [&](const Pend& P, int i) {
        // MX: lane-dependent terms from an opaque copy of the lane id, recomputed per step
        // rather than held in registers (or spilled) across the tile loop; plain FP8 has the
        // registers and keeps them (measured 2-3% faster)
        int pl = lane;
        if constexpr (MX) asm volatile("" : "+v"(pl));
        const int q = MX ? pl >> 3 : l3;
        const int row = (MX ? wave * (8 * NP) + q : row0) + 8 * i;
        const int sa = ((i & 1) << 2) | (((q >> 2) & 1) << 1) | ((q >> 1) & 1);  // swz(row)
        const int sb = NW == 16 ? swzB(row) : (((i & 3) << 1) | ((q >> 1) & 1));  // swzB(row)
        const int cha = (pl & 7) ^ sa, chb = (pl & 7) ^ sb;
        const int pa = P.kpos + 16 * cha, pb = P.kpos + 16 * chb;
        const bool ka = pa < P.kb_hi && pa + 16 > P.kb_lo;
        const bool kb = pb < P.kb_hi && pb + 16 > P.kb_lo;
        const uint32_t aoff =
            (ka && row < P.a_rows) ? (uint32_t)row * (uint32_t)p.lda + (uint32_t)pa : OOB;
        const uint32_t boff =
            (kb && row < P.b_rows) ? (uint32_t)row * (uint32_t)p.ldb + (uint32_t)pb : OOB;
        if (MODE == MODE_WGRAD || wave * 8 * NP + 8 * i < P.a_rows)  // wave-uniform
            dma16(P.ra, aoff, P.as + (uint32_t)(wave * NP + i) * 1024u);
        dma16(P.rb, boff, P.bs + (uint32_t)(wave * NP + i) * 1024u);
    };
    auto issue = [&](const Tile& T, int kpos, int stage) {
        const Pend P = prep(T, kpos, stage);
#pragma unroll
        for (int i = 0; i < NP; i++) part(P, i);
    };
    // MX_BYTES: a step's scale bytes are loaded into registers with its operand loads and
    // written to LDS at the top of that step, after its wait for the loads.  Using them any
    // earlier would wait for every operand load issued after them as well (the vector-memory
    // counter completes in issue order), serializing the prefetch.
    bool scales_pending = false;
    auto commit_scales = [&](int stage) {
        if (MXV == MX_BYTES && row_thread) {
            sscale[stage][0][t] = sa_pack;
            sscale[stage][1][t] = sb_pack;
        }
    };

    Tile cur, nxt;
    bool have = next_tile(cur);
    int stage0 = 0;  // LDS stage holding the current tile's first step
    if (have && cur.nk > 0) {
        issue(cur, cur.kstart, 0);
        scales_pending = true;
    }
    const int kg = lane >> 4, lr = lane & 15, lq = lane >> 4;
    while (have) {
        v4f_t acc[8][NJ];
#pragma unroll
        for (int i = 0; i < 8; i++)
#pragma unroll
            for (int j = 0; j < NJ; j++) acc[i][j] = v4f_t{0.0f, 0.0f, 0.0f, 0.0f};
        bool have_next = false, next_issued = false;

        for (int kk = 0; kk < cur.nk; kk++) {
            const int cur_st = (stage0 + (kk & 1)) & 1;
            const int kpos = cur.kstart + kk * GK;
            wait_vm0();  // this wave's loads of step kk have landed
            if (FNUZ) {
                // e4m3fnuz operands: each lane re-encodes the 16-byte chunks it brought into
                // the stage to the e4m3fn bytes of the same values, in place, before the
                // barrier that publishes the stage (once per byte, not once per fragment read)
#pragma unroll
                for (int i = 0; i < NP; i++) {
                    const int slot = (wave * NP + i) * 1024 + lane * 16;
                    if (MODE == MODE_WGRAD || wave * 8 * NP + 8 * i < cur.a_rows) {
                        uint4* q = reinterpret_cast<uint4*>(&smem[cur_st][0][slot]);
                        uint4 w = *q;
                        *q = make_uint4(fnuz_to_fn4(w.x), fnuz_to_fn4(w.y), fnuz_to_fn4(w.z),
                                        fnuz_to_fn4(w.w));
                    }
                    uint4* q = reinterpret_cast<uint4*>(&smem[cur_st][1][slot]);
                    uint4 w = *q;
                    *q = make_uint4(fnuz_to_fn4(w.x), fnuz_to_fn4(w.y), fnuz_to_fn4(w.z),
                                    fnuz_to_fn4(w.w));
                }
            }
            if (MXV == MX_BYTES && scales_pending) {
                commit_scales(cur_st);  // read after this step's barrier
                scales_pending = false;
            }
            if (MODE == MODE_WGRAD && (kpos < cur.kb_lo || kpos + GK > cur.kb_hi)) {
                // zero the bytes of other tokens (neighbouring groups, or the padding past M)
                // in the straddling chunks of BOTH operands: such a byte may hold any code,
                // NaN included, and 0 * NaN would reach the group's sums
                __syncthreads();
                const int lo = cur.kb_lo - kpos, hi = cur.kb_hi - kpos;
                // threads 0-255 take the rows of the activation tile, 256-511 those of the
                // gradient tile (at least 8 waves: wave-uniform sides)
                static_assert(NW >= 8, "two tile sides over 512 threads");
                // an opaque copy of the thread id: the addresses below are recomputed here
                // instead of being held in registers across the whole tile
                int tt = t;
                asm volatile("" : "+v"(tt));
                if (tt < 2 * GT) {
                    const int zr = tt & (GT - 1);
                    uint8_t* side = smem[cur_st][tt >> 8];
#pragma unroll
                    for (int ch = 0; ch < 8; ch++) {
                        const int b0 = 16 * ch;
                        if ((lo > b0 && lo < b0 + 16) || (hi > b0 && hi < b0 + 16)) {
                            uint4* q = reinterpret_cast<uint4*>(
                                side + (tt < GT ? lds_off(zr, ch) : lds_offB(zr, ch)));
                            uint4 w = *q;
                            w.x &= keep_mask4(lo, hi, b0);
                            w.y &= keep_mask4(lo, hi, b0 + 4);
                            w.z &= keep_mask4(lo, hi, b0 + 8);
                            w.w &= keep_mask4(lo, hi, b0 + 12);
                            *q = w;
                        }
                    }
                }
            }
            __syncthreads();
            // the next step's operand loads (this tile's, or the next tile's first) are issued
            // in 8 parts between the first four rows of this step's matrix instructions, so the
            // last of them still has half a step to land (MX: between all eight rows)
            // the next tile is looked up on the first step (its offsets loads then have the
            // whole tile to arrive) and its first step is fetched during the last one
            if (kk == 0) have_next = tile_start(nxt);
            Pend P{};
            bool pend = false;
            if (kk + 1 < cur.nk) {
                P = prep(cur, kpos + GK, cur_st ^ 1);
                pend = true;
            } else {
                if (have_next) tile_finish(nxt);
                if (have_next && nxt.nk > 0) {
                    P = prep(nxt, nxt.kstart, cur_st ^ 1);
                    pend = true;
                    next_issued = true;
                }
            }

            const uint8_t* As = smem[cur_st][0];
            const uint8_t* Bs = smem[cur_st][1];
            const bool kb_in = kpos + 32 * kg < cur.kb_hi;  // MX: this lane's K block exists
            const int mslot = (cur.mx_slot + (kk >> 2)) & 1, msub = 4 * (kk & 3);
            // LDS indices of the scale of this lane's first A row (row wm*128 + lr); the masks
            // change no value (both stay inside their arrays) but let the compiler fold the
            // per-row offsets into the LDS instructions' immediates instead of holding one
            // address register per row (16 waves: the difference between spilling and not)
            const uint32_t ma_dma =
                (uint32_t)(((mslot * 2 + 0) * GT + wm * 128 + lr) * 16 + msub + kg) & 0x3FFFu;
            const uint32_t ma_byt = (uint32_t)(wm * 128 + lr) & 0xFFu;
            v8i_t bf[NJ];
            int sb_[NJ];
#pragma unroll
            for (int j = 0; j < NJ; j++) {
                const int rn = wn * WNC + brow(j, lr);
                bf[j] = frag<true>(Bs, rn, kg, false);
                // scale bytes are read unconditionally (in-range LDS) and then selected: a
                // conditional read becomes a branch per row, and the compiler then gathers all
                // fragment reads ahead of the matrix instructions (registers spill)
                if (MXV == MX_BYTES || MXV == MX_DW) {
                    const int e = (int)((sscale[cur_st][1][rn] >> (8 * kg)) & 0xFFu);
                    sb_[j] = kb_in ? e : 127;
                }
                if (MXV == MX_DMA) {
                    const int e = (int)smx[((mslot * 2 + 1) * GT + rn) * 16 + msub + kg];
                    sb_[j] = kb_in ? e : 127;
                }
            }
            // 16 waves: a wave issuing its matrix instructions goes ahead of the other waves'
            // memory instructions (weight gradient 517 -> 510 us; forward unchanged)
            if (NW == 16) __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const int rm = wm * 128 + i * 16 + lr;
                const v8i_t af = frag<false>(As, rm, kg, false);
                if (pend && !MX && NW == 4 && i < NP / 2) {  // two parts per row in the first rows
                    part(P, 2 * i);
                    part(P, 2 * i + 1);
                }
                if (pend && NW >= 8 && i == 0) {  // 8-16 waves: all parts up front
#pragma unroll                                          // (measured 1-2% faster than spread)
                    for (int q = 0; q < NP; q++) part(P, q);
                }
                if (pend && MX && NW == 4 && i < NP) part(P, i);  // 4-wave MX: one part per row
                int sa_ = 0;
                if (MXV == MX_BYTES || MXV == MX_DW) {
                    const int e = (int)((sscale[cur_st][0][ma_byt + 16 * i] >> (8 * kg)) & 0xFFu);
                    sa_ = kb_in ? e : 127;
                }
                if (MXV == MX_DMA) {
                    const int e = (int)smx[ma_dma + 256 * i];
                    sa_ = kb_in ? e : 127;
                }
#pragma unroll
                for (int j = 0; j < NJ; j++) {
                    if (MX)
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            bf[j], af, acc[i][j], 0, 0, 0, sb_[j], 0, sa_);
                    else
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            bf[j], af, acc[i][j], 0, 0, 0, 0, 0, 0);
                }
            }
            if (NW == 16) __builtin_amdgcn_s_setprio(0);
            if (kk + 1 < cur.nk || next_issued) scales_pending = true;
        }
        if (cur.nk == 0) {
            // nothing was computed; start the next tile's first step in the free stage once
            // every wave is past the previous tile's epilogue (it read the scale buffer the
            // next tile's scales go to)
            __syncthreads();
            have_next = next_tile(nxt);
            if (have_next && nxt.nk > 0) {
                issue(nxt, nxt.kstart, stage0);
                scales_pending = true;
            }
        }

        // The lane's coordinates for the epilogue; MX: from an opaque copy of its id,
        // recomputed for every tile rather than held in registers across the contraction loop
        // (MX weight gradient: 10 spilled registers before, 566 -> 540 us)
        int eln = lane;
        if constexpr (MX) asm volatile("" : "+v"(eln));
        const int elr = eln & 15, elq = eln >> 4;
        // Epilogue: eln holds rows row_lo + wm*128 + 16i + eln%16 and, per column-block pair
        // j', the 8 consecutive columns n0 + wn*WNC + 32j' + 8*(eln/16) + 0..7 (blocks 2j' and
        // 2j'+1 give 4 each).  Dequantize with the reciprocal scales and store 8 outputs at once.
        const float* s_rows = reinterpret_cast<const float*>(sscale[cur.par][0]);
        const float* s_cols = reinterpret_cast<const float*>(sscale[cur.par][1]);
        const bool scaled = !MX && cur.nk > 0;  // an empty contraction stores zeros
        float rs[8];
#pragma unroll
        for (int i = 0; i < 8; i++)
            rs[i] = scaled ? __builtin_amdgcn_rcpf(s_rows[wm * 128 + i * 16 + elr]) : 1.0f;
        const int64_t crow0 = MODE == MODE_FWD ? (int64_t)cur.row_lo : (int64_t)cur.g * p.K + cur.row_lo;
        const int trows = cur.row_hi - cur.row_lo;
        // Stores go through a buffer resource over the tile's output rows; a row past the
        // tile's last one or a column past N gets an out-of-range eln offset and its store is
        // dropped (the range check covers the eln offset only, never the scalar offset, so the
        // whole address is in the eln offset).  Branch-free: every wave issues the same store
        // instructions.
        const uint32_t esz = p.out_f32 ? 4u : 2u;
        const __amdgpu_buffer_rsrc_t rc = make_rsrc(
            p.c + crow0 * p.ldc * (int64_t)esz, (uint32_t)trows * (uint32_t)p.ldc * esz);
        const uint32_t row16 = 16u * (uint32_t)p.ldc * esz;  // bytes of 16 output rows
        auto epilogue = [&](auto f32, auto vec) {
            constexpr bool F32 = decltype(f32)::value, VEC = decltype(vec)::value;
            constexpr uint32_t ES = F32 ? 4u : 2u;
#pragma unroll
            for (int jp = 0; jp < NJ / 2; jp++) {
                const int nl = wn * WNC + 32 * jp + 8 * elq;
                const int n = cur.n0 + nl;
                const uint32_t lane_off =
                    ((uint32_t)(wm * 128 + elr) * (uint32_t)p.ldc + (uint32_t)n) * ES;
                float cs[8];
#pragma unroll
                for (int e = 0; e < 8; e++)
                    cs[e] = scaled ? __builtin_amdgcn_rcpf(s_cols[nl + e]) : 1.0f;
#pragma unroll
                for (int i = 0; i < 8; i++) {
                    const bool row_ok = wm * 128 + i * 16 + elr < trows;
                    const uint32_t roff = lane_off + (uint32_t)i * row16;
                    const v4f_t a0 = acc[i][2 * jp], a1 = acc[i][2 * jp + 1];
                    const float r_ = rs[i];
                    float v[8];
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        v[e] = a0[e] * r_ * cs[e];
                        v[4 + e] = a1[e] * r_ * cs[4 + e];
                    }
                    if (VEC) {
                        // N is a multiple of 8: a eln's 8 columns are all inside or all past N
                        const uint32_t off = row_ok && n < p.N ? roff : OOB;
                        if (F32) {
                            __builtin_amdgcn_raw_buffer_store_b128(
                                i32x4_t{(int)__float_as_uint(v[0]), (int)__float_as_uint(v[1]),
                                        (int)__float_as_uint(v[2]), (int)__float_as_uint(v[3])},
                                rc, off, 0, 0);
                            __builtin_amdgcn_raw_buffer_store_b128(
                                i32x4_t{(int)__float_as_uint(v[4]), (int)__float_as_uint(v[5]),
                                        (int)__float_as_uint(v[6]), (int)__float_as_uint(v[7])},
                                rc, off + 16u, 0, 0);
                        } else {
                            __builtin_amdgcn_raw_buffer_store_b128(
                                i32x4_t{(int)pack_bf16x2(v[0], v[1]), (int)pack_bf16x2(v[2], v[3]),
                                        (int)pack_bf16x2(v[4], v[5]), (int)pack_bf16x2(v[6], v[7])},
                                rc, off, 0, 0);
                        }
                    } else {
                        // any N, ldc and (element-aligned) c: one store per element
#pragma unroll
                        for (int e = 0; e < 8; e++) {
                            const uint32_t off =
                                row_ok && n + e < p.N ? roff + (uint32_t)e * ES : OOB;
                            if (F32)
                                __builtin_amdgcn_raw_buffer_store_b32((int)__float_as_uint(v[e]), rc,
                                                                      off, 0, 0);
                            else
                                __builtin_amdgcn_raw_buffer_store_b16(
                                    (short)(pack_bf16x2(v[e], 0.0f) & 0xFFFFu), rc, off, 0, 0);
                        }
                    }
                }
            }
        };
        if (p.vec_store) {
            if (p.out_f32)
                epilogue(std::true_type{}, std::true_type{});
            else
                epilogue(std::false_type{}, std::true_type{});
        } else {
            if (p.out_f32)
                epilogue(std::true_type{}, std::false_type{});
            else
                epilogue(std::false_type{}, std::false_type{});
        }
        stage0 = (stage0 + (cur.nk & 1)) & 1;
        have = have_next;
        cur = nxt;
    }
}

static int num_cus() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cached[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

template <int FMT, int MODE, int MXV>
static fp8q_status_t launch_gemm(GemmArgs p, hipStream_t stream) {
    p.nt_n = (int)((p.N + GT - 1) / GT);
    p.nt_k = MODE == MODE_FWD ? 1 : (int)((p.K + GT - 1) / GT);
    if (p.G > GMAX || p.M > 0x7FFFFFFFLL || p.N > 0x7FFFFFFFLL || p.K > 0x7FFFFFFFLL)
        return FP8Q_ERR_UNSUPPORTED;
    // tile indices are 32-bit: forward row-tile slots (at most one partial per group) times
    // column tiles, weight-gradient groups times tiles per group
    const int64_t max_tiles = MODE == MODE_FWD ? ((p.M + GT - 1) / GT + p.G) * p.nt_n
                                               : (int64_t)p.G * p.nt_k * p.nt_n;
    if (max_tiles >= 0x7FFFFFFFLL) return FP8Q_ERR_UNSUPPORTED;
    int64_t grid = num_cus();
    if (max_tiles < grid) grid = max_tiles;
    if (grid < 1) grid = 1;
    // whole 16-byte output stores through a 32-bit buffer range over a tile's 256 rows
    const int64_t esz = p.out_f32 ? 4 : 2;
    if ((int64_t)GT * p.ldc * esz >= 0x7FFFFFFFLL) return FP8Q_ERR_UNSUPPORTED;
    if (!fp8q_aligned(p.c, (uintptr_t)esz)) return FP8Q_ERR_INVALID_ARG;
    p.vec_store = p.N % 8 == 0 && p.ldc % 8 == 0 && fp8q_aligned(p.c, 16);
    // Plain FP8: 16 waves (four per SIMD, 128 x 32 each; 124-128 registers).  Measured on the
    // dsv3 step, 4 / 8 / 16 waves: forward 368 / 352 / 328 us, weight gradient 606 / 589 /
    // 498 us, data gradient 396 / 364 / 345 us.  MX with scales by DMA: 16 waves as well
    // (127 registers, no spills): MX forward 455 / 406 / 392 us at 4 / 8 / 16 waves.  MX with
    // byte-loaded scales (the MX weight gradient): 8 waves (256 registers): 801 -> 713 us
    // against 4 waves; at 16 waves its registers spill inside the loop (1267 us).
    constexpr int NW = MXV == MX_BYTES ? 8 : 16;
    gemm256_kernel<FMT, MODE, MXV, NW><<<dim3((unsigned)grid), dim3(64 * NW), 0, stream>>>(p);
    FP8Q_CHECK_LAUNCH();
    return FP8Q_OK;
}

// 32-bit buffer offsets: a 256-row tile of either operand must span less than 2^31 bytes.
static inline bool offsets_fit(int64_t lda, int64_t ldb) {
    return (int64_t)GT * lda < 0x7FFFFFFFLL && (int64_t)GT * ldb < 0x7FFFFFFFLL;
}

// Workspace of every grouped GEMM: the two status words of the offsets check, padded.
constexpr size_t kGemmWorkspace = 256;

// Output type, workspace and the fields they set; FP8Q_OK or the status to return.
static fp8q_status_t gemm_common(GemmArgs& p, fp8q_out_t out_dtype, void* workspace,
                                 size_t workspace_bytes) {
    if (out_dtype != FP8Q_OUT_BF16 && out_dtype != FP8Q_OUT_FP32) return FP8Q_ERR_INVALID_ARG;
    if (!workspace || workspace_bytes < kGemmWorkspace) return FP8Q_ERR_WORKSPACE;
    if (!fp8q_aligned(workspace, 4)) return FP8Q_ERR_INVALID_ARG;
    p.out_f32 = out_dtype == FP8Q_OUT_FP32;
    p.status = reinterpret_cast<int32_t*>(workspace);
    return FP8Q_OK;
}

}  // namespace fp8q

extern "C" size_t fp8_grouped_gemm_workspace_size(fp8q_gemm_mode_t mode, int64_t M, int64_t N,
                                                  int64_t K, int32_t groups) {
    (void)mode; (void)M; (void)N; (void)K; (void)groups;
    return fp8q::kGemmWorkspace;
}

extern "C" fp8q_status_t fp8_grouped_gemm(fp8q_gemm_mode_t mode, fp8q_format_t fmt,
                                          const uint8_t* a, int64_t lda, const float* a_scales,
                                          const uint8_t* b, int64_t ldb, int64_t b_group_stride,
                                          const float* b_scales, const int32_t* offsets,
                                          int32_t groups, int64_t M, int64_t N, int64_t K,
                                          void* c, int64_t ldc, fp8q_out_t out_dtype,
                                          void* workspace, size_t workspace_bytes,
                                          hipStream_t stream) {
    using namespace fp8q;
    if (!fp8q_fmt_ok(fmt) || groups < 1 || M < 0 || N < 0 || K < 0 || ldc < N || !offsets)
        return FP8Q_ERR_INVALID_ARG;
    GemmArgs p{};
    const fp8q_status_t cs = gemm_common(p, out_dtype, workspace, workspace_bytes);
    if (cs != FP8Q_OK) return cs;
    p.a = a; p.lda = lda; p.a_scales = a_scales; p.b = b; p.ldb = ldb; p.bgs = b_group_stride;
    p.b_scales = b_scales; p.offsets = offsets; p.G = groups; p.M = M; p.N = N; p.K = K;
    p.c = reinterpret_cast<uint8_t*>(c); p.ldc = ldc;
    if (mode == FP8Q_GEMM_FWD_MGROUPED) {
        if (lda < K || ldb < K || b_group_stride < 0) return FP8Q_ERR_INVALID_ARG;
        if (M == 0 || N == 0) return FP8Q_OK;
        if (!a || !b || !a_scales || !b_scales || !c) return FP8Q_ERR_INVALID_ARG;
        if (K % 16 || lda % 16 || ldb % 16 || b_group_stride % 16 || !fp8q_aligned(a, 16) ||
            !fp8q_aligned(b, 16) || !offsets_fit(lda, ldb))
            return FP8Q_ERR_UNSUPPORTED;
        if (fmt == FP8Q_E4M3FN) return launch_gemm<FP8Q_E4M3FN, MODE_FWD, MX_NONE>(p, stream);
        return launch_gemm<FP8Q_E4M3FNUZ, MODE_FWD, MX_NONE>(p, stream);
    }
    if (mode == FP8Q_GEMM_WGRAD_KGROUPED) {
        if (lda < M || ldb < M || b_group_stride != 0) return FP8Q_ERR_INVALID_ARG;
        if (K == 0 || N == 0) return FP8Q_OK;
        if (!a_scales || !b_scales || !c || (M > 0 && (!a || !b))) return FP8Q_ERR_INVALID_ARG;
        if (lda % 16 || ldb % 16 || !fp8q_aligned(a, 16) || !fp8q_aligned(b, 16) ||
            !offsets_fit(lda, ldb))
            return FP8Q_ERR_UNSUPPORTED;
        if (fmt == FP8Q_E4M3FN) return launch_gemm<FP8Q_E4M3FN, MODE_WGRAD, MX_NONE>(p, stream);
        return launch_gemm<FP8Q_E4M3FNUZ, MODE_WGRAD, MX_NONE>(p, stream);
    }
    return FP8Q_ERR_INVALID_ARG;
}

extern "C" fp8q_status_t fp8_mx_grouped_gemm_wgrad(const uint8_t* a, int64_t lda,
                                                   const uint8_t* a_e8m0, int64_t ld_sa,
                                                   const uint8_t* b, int64_t ldb,
                                                   const uint8_t* b_e8m0, int64_t ld_sb,
                                                   const int32_t* offsets, int32_t groups,
                                                   int64_t M, int64_t N, int64_t K, void* c,
                                                   int64_t ldc, fp8q_out_t out_dtype,
                                                   void* workspace, size_t workspace_bytes,
                                                   hipStream_t stream) {
    using namespace fp8q;
    if (groups < 1 || M < 0 || N < 0 || K < 0 || ldc < N || !offsets || lda < M || ldb < M ||
        ld_sa < M / 32 || ld_sb < M / 32)
        return FP8Q_ERR_INVALID_ARG;
    if (M % 32) return FP8Q_ERR_INVALID_ARG;
    GemmArgs p{};
    const fp8q_status_t cs = gemm_common(p, out_dtype, workspace, workspace_bytes);
    if (cs != FP8Q_OK) return cs;
    if (K == 0 || N == 0) return FP8Q_OK;
    if (!a_e8m0 || !b_e8m0 || !c || (M > 0 && (!a || !b))) return FP8Q_ERR_INVALID_ARG;
    if (lda % 16 || ldb % 16 || !fp8q_aligned(a, 16) || !fp8q_aligned(b, 16) ||
        !offsets_fit(lda, ldb) || !offsets_fit(ld_sa, ld_sb))
        return FP8Q_ERR_UNSUPPORTED;
    p.a = a; p.lda = lda; p.a_e8 = a_e8m0; p.ld_sa = ld_sa; p.b = b; p.ldb = ldb;
    p.bgs = 0; p.b_e8 = b_e8m0; p.ld_sb = ld_sb; p.sbgs = 0;
    p.offsets = offsets; p.G = groups; p.M = M; p.N = N; p.K = K;
    p.c = reinterpret_cast<uint8_t*>(c); p.ldc = ldc;
    // scale rows 4-byte aligned: one dword of scales per row, side and step by DMA, tiles
    // starting on 128-token boundaries; otherwise per-step byte loads of the scales
    const bool dw = ld_sa % 4 == 0 && ld_sb % 4 == 0 && fp8q_aligned(a_e8m0, 4) &&
                    fp8q_aligned(b_e8m0, 4);
    if (dw) return launch_gemm<FP8Q_E4M3FN, MODE_WGRAD, MX_DW>(p, stream);
    return launch_gemm<FP8Q_E4M3FN, MODE_WGRAD, MX_BYTES>(p, stream);
}

extern "C" fp8q_status_t fp8_mx_grouped_gemm(const uint8_t* a, int64_t lda, const uint8_t* a_e8m0,
                                             int64_t ld_sa, const uint8_t* b, int64_t ldb,
                                             int64_t b_group_stride, const uint8_t* b_e8m0,
                                             int64_t ld_sb, int64_t sb_group_stride,
                                             const int32_t* offsets, int32_t groups, int64_t M,
                                             int64_t N, int64_t K, void* c, int64_t ldc,
                                             fp8q_out_t out_dtype, void* workspace,
                                             size_t workspace_bytes, hipStream_t stream) {
    using namespace fp8q;
    if (groups < 1 || M < 0 || N < 0 || K < 0 || ldc < N || !offsets || lda < K || ldb < K ||
        b_group_stride < 0 || sb_group_stride < 0 || ld_sa < K / 32 || ld_sb < K / 32)
        return FP8Q_ERR_INVALID_ARG;
    if (K % 32) return FP8Q_ERR_INVALID_ARG;
    GemmArgs p{};
    const fp8q_status_t cs = gemm_common(p, out_dtype, workspace, workspace_bytes);
    if (cs != FP8Q_OK) return cs;
    if (M == 0 || N == 0) return FP8Q_OK;
    if (!a || !b || !a_e8m0 || !b_e8m0 || !c) return FP8Q_ERR_INVALID_ARG;
    if (lda % 16 || ldb % 16 || b_group_stride % 16 || !fp8q_aligned(a, 16) ||
        !fp8q_aligned(b, 16) || !offsets_fit(lda, ldb) || !offsets_fit(ld_sa, ld_sb))
        return FP8Q_ERR_UNSUPPORTED;
    p.a = a; p.lda = lda; p.a_e8 = a_e8m0; p.ld_sa = ld_sa; p.b = b; p.ldb = ldb;
    p.bgs = b_group_stride; p.b_e8 = b_e8m0; p.ld_sb = ld_sb; p.sbgs = sb_group_stride;
    p.offsets = offsets; p.G = groups; p.M = M; p.N = N; p.K = K;
    p.c = reinterpret_cast<uint8_t*>(c); p.ldc = ldc;
    const bool dma = ld_sa % 16 == 0 && ld_sb % 16 == 0 && sb_group_stride % 16 == 0 &&
                     fp8q_aligned(a_e8m0, 16) && fp8q_aligned(b_e8m0, 16);
    if (dma) return launch_gemm<FP8Q_E4M3FN, MODE_FWD, MX_DMA>(p, stream);
    return launch_gemm<FP8Q_E4M3FN, MODE_FWD, MX_BYTES>(p, stream);
}
