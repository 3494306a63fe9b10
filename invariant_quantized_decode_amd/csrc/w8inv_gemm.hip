// w8inv_gemm.hip -- the W8A16 (int8 group-32, fp16 scales, bf16 activations)
// decode projection at a fixed width T_pad, with one reduction schedule for
// every t.
//
// Method: the ninfer issue on t-dependent kernel dispatch (GitHub issue 80),
// "Proposal: opt-in fixed decode width": one reduction schedule serves every
// t <= T_pad, padding columns are never read from the caller nor stored, and
// no output column's arithmetic involves another column.  Format: table
// "Where t selects arithmetic", row "ops::linear W8G32".
//
// Design for gfx950 (CDNA4):
//  * The K plan is a function of K alone: 8 contiguous K-slices made of whole
//    pairs of 32-element groups, the first four three times as long as the
//    last four (kslice_begin); each slice is summed in ascending group order in
//    fp64 and the 8 slice sums are combined by a left fold.  Two kernels run
//    this same plan and give the same bits for every row:
//    - gemm_w8g32_split_lds: one workgroup = 32 output rows x all K, its 8
//      waves take the 8 slices; activations (and, for the plain layout, the
//      scales) are staged in LDS by direct loads; each wave parks its slice
//      sum in LDS, one barrier, and the waves fold and store.  Template
//      options: the store epilogue (plain, + residual, SwiGLU of gate/up row
//      pairs) and the weight layout (plain row-major or packed).
//    - gemm_w8g32_tiles (large N, T_pad <= 32): persistent workgroups stream
//      256-row tiles; each wave owns a 32-row strip and walks all of K,
//      keeping the running slice sum and the fold in registers, while the
//      activation stage is shared through a double-buffered LDS ring.
//  * Weight loads are coalesced.  Plain layout: one instruction covers 16 rows
//    x 64 contiguous bytes (two groups); the split kernel restores the
//    matrix-core layout in registers with v_permlane16_swap, the persistent
//    kernel reads it from an LDS slot that direct loads filled row by row.  Packed layout (w8inv_pack.hip): one instruction
//    reads 1 KB of whole cache lines already in the matrix-core lane order,
//    with the nontemporal cache policy (each byte is read once).
//  * Each group's 32 products per output are summed by two chained
//    v_mfma_f32_32x32x16_bf16 (A = activations, B = weights) into fp32 from
//    zero; int8 -> bf16 is exact (7 significant bits).
//  * The fp16 group scale is applied to that fp32 group sum in fp64 (the
//    product is exact there); the fp64 result is rounded once to bf16.
//  * Columns >= t are zeros and are never stored.  A padding column inside a
//    direct load's 8 columns loads as zeros without a memory access (an
//    offset past the activation buffer's range); a load whose 8 columns are
//    all padding is not issued at all, its LDS region zeroed once, and the
//    fp64 products of such columns are not formed (a 32-column tile with no
//    live column skips its MFMAs; at T_pad 48 or 64 with t <= 32 the one-tile
//    kernel runs, see kernel_width).  That is all t selects: how much padding
//    work is skipped.
//  * No atomics; the arithmetic of a column -- K plan, MFMA sequence,
//    roundings -- depends on neither t, its neighbours, N nor the device.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "w8inv_gemm_common.h"
#include "w8inv_internal.h"
#include "w8inv_math.h"

namespace w8i {

constexpr int kGemmThreads = 64 * kKSlices;
constexpr size_t kMaxGemmLds = 160 * 1024;  // LDS of one gfx950 workgroup
constexpr int kMinTilesPerCu = 2;            // persistent tiles need at least this many per CU

// ----------------------------------------------------------------------------
// Split-K: one workgroup = 32 output rows x all K, its 8 waves take the 8
// K-slices, the slice sums meet in LDS.  Activations are staged in LDS by
// direct loads (buffer_load ... lds).  Every wave re-reads its slice's
// activations from L2, and what that costs is the number of cache lines
// touched, not the bytes: each direct load covers 8 columns x 128 bytes (whole
// lines) and lands in a per-wave LDS ring of depth D, from which the
// matrix-core operands are read.  Plain layout: the strip's scales (rows
// n0 .. n0+31) are one contiguous block of 64 G bytes and are copied to LDS
// before the main loop when they fit beside the ring; otherwise each stage
// loads its scales with the weights.  Packed layout: each stage loads its
// scales as one 128-byte line.
// ----------------------------------------------------------------------------

// one ring slot (the stage of all 8 waves) for NT 32-column tiles
__host__ __device__ constexpr int split_lds_slot_bytes(int NT) { return kKSlices * NT * kXTileBytes; }

// LDS capacity left for the scales when the ring has D slots
__host__ __device__ constexpr int split_lds_scale_bytes(int NT, int D) {
    return (int)kMaxGemmLds - D * split_lds_slot_bytes(NT) - (4 - D) * 16;
}

// LS: the strip's scales are copied to LDS (when they fit beside the ring);
// otherwise every stage loads its two scales per row with the weights.
// EPI: what is stored (see LinearEpilogue): kEpiStore, kEpiAdd or kEpiSwiGLU.
// PK: W and S are in the packed layout (w8_pack): each stage's weights are two
// contiguous 1 KB blocks already in the matrix-core lane order, and its scales
// one 128-byte line, loaded with the stage.
// R: output rows per workgroup (8..32; 32 with the SwiGLU epilogue).  The
// matrix core always computes 32 rows; rows R..31 repeat row R - 1's loads
// (no extra memory traffic) and are not stored.
// EPI kEpiPair: the launch covers two projections of the same x, the first
// ep.wg1 workgroups the first (W, S, Y, N, ldy), the others the second (ep.W2,
// ...); each workgroup then runs exactly the single projection's code.
template <int TP16, int D, bool LS, int EPI, bool PK>  // TP16 = T_pad / 16 (1..4), D = ring depth (2..4)
__global__ __launch_bounds__(kGemmThreads) void gemm_w8g32_split_lds(
    const int8_t* __restrict__ W, const uint16_t* __restrict__ S, const uint16_t* __restrict__ X,
    uint16_t* __restrict__ Y, int64_t N, int64_t K, int t, int64_t ldx, int64_t ldy, LinearEpilogue ep, int R) {
    int bid = (int)blockIdx.x;
    if constexpr (EPI == kEpiPair) {
        if (bid >= ep.wg1) {
            W = ep.W2;
            S = ep.S2;
            Y = ep.Y2;
            N = ep.N2;
            ldy = ep.ldy2;
            bid -= ep.wg1;
        }
    }
    static_assert(TP16 >= 1 && TP16 <= 4, "T_pad 16..64");
    static_assert(D >= 2 && D <= 4, "ring depth");
    constexpr int NT = (TP16 + 1) / 2;                // 32-column tiles
    constexpr int kLastValues = (TP16 & 1) ? 8 : 16;  // real rows of the last tile's 16 per lane
    constexpr int kStageBytes = NT * kXTileBytes;     // one wave's activation stage
    constexpr int kSlotBytes = split_lds_slot_bytes(NT);
    constexpr int kScaleBytes = LS ? split_lds_scale_bytes(NT, D) : 16;
    constexpr int kXLoads = 4 * NT;                   // direct loads of 8 columns x 128 bytes per stage
    static_assert(!PK || !LS, "packed layout: scales come with each stage");
    static_assert(kScaleBytes > 0, "LDS");
    // one array per ring slot, so the compiler can wait for each slot's loads alone
    __shared__ __align__(16) unsigned char xr0[kSlotBytes];
    __shared__ __align__(16) unsigned char xr1[kSlotBytes];
    __shared__ __align__(16) unsigned char xr2[D > 2 ? kSlotBytes : 16];
    __shared__ __align__(16) unsigned char xr3[D > 3 ? kSlotBytes : 16];
    __shared__ __align__(16) unsigned char s_raw[kScaleBytes];
    const uint16_t* s_lds = reinterpret_cast<const uint16_t*>(s_raw);

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int G = (int)(K / kGroup);
    const int64_t n0 = (int64_t)bid * R;
    // The workgroup's rows: n0 .. n0 + R - 1, or with the SwiGLU epilogue the
    // 16 gate rows h0 .. h0 + 15 followed by the 16 matching up rows
    // F + h0 .. F + h0 + 15.  Rows past the end read the last valid row (valid
    // memory; their results are never stored).
    const int64_t h0 = (int64_t)bid * (kRows / 2);
    auto row_of = [&](int rho) -> int64_t {
        if constexpr (EPI == kEpiSwiGLU) {
            const int64_t h = h0 + (rho & 15);
            return (rho < 16 ? 0 : ep.F) + (h < ep.F ? h : ep.F - 1);
        } else {
            const int64_t n = n0 + (rho < R ? rho : R - 1);
            return n < N ? n : N - 1;
        }
    };
    const int g_begin = __builtin_amdgcn_readfirstlane((int)kslice_begin(G, wave));
    const int g_end = __builtin_amdgcn_readfirstlane((int)kslice_begin(G, wave + 1));

    // Rows past N read row N-1 (valid memory, results never stored); padding
    // columns (j >= t) load as zeros without a memory access (kPadColumnOffset);
    // the descriptors' ranges bound every access.
    // packed layout: whole strips of P = ceil(G/2) stage blocks (2 KB of codes, 128 bytes of scales)
    const int64_t P = (G + 1) / 2;
    const int64_t strips = (N + kRows - 1) / kRows;
    const __amdgpu_buffer_rsrc_t w_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t*>(W), (short)0, (int)(uint32_t)(PK ? strips * P * 2048 : N * K), 0x00020000);
    const __amdgpu_buffer_rsrc_t x_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(X), (short)0, (int)(uint32_t)(((int64_t)(t - 1) * ldx + K) * 2), 0x00020000);
    // The range is rounded up to whole 16-byte pieces: a piece that straddles
    // the end would otherwise come back as zeros, scales of the last row
    // included.  S is 16-byte aligned here, so the rounded piece lies in the
    // same aligned 16 bytes (and page) as the last scales.
    const __amdgpu_buffer_rsrc_t s_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(S), (short)0,
        (int)(PK ? (uint32_t)(strips * P * 128) : ((uint32_t)(N * G * 2) + 15u) & ~15u), 0x00020000);

    // the strip's scales -> LDS, issued first so the wait below can leave the
    // activation ring in flight
    // (SwiGLU: the gate rows' and the up rows' scales are two blocks of 32 G
    // bytes, each copied to its own LDS region of whole 1 KB pieces)
    const int s_block = LS ? (EPI == kEpiSwiGLU ? 32 * G : 64 * G) : 0;
    const int s_pieces = (s_block + kLdsDmaBytes - 1) / kLdsDmaBytes;
    const int s_loads = EPI == kEpiSwiGLU ? 2 * s_pieces : s_pieces;
    for (int k = wave; k < s_loads; k += kKSlices) {
        const int blk = EPI == kEpiSwiGLU && k >= s_pieces ? 1 : 0;
        const int piece = k - blk * s_pieces;
        const int64_t first_row = EPI == kEpiSwiGLU ? blk * ep.F + h0 : n0;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(s_rsrc, W8I_LDS(s_raw + k * kLdsDmaBytes), 16, 16u * lane,
                                                 (uint32_t)(first_row * G * 2) + (uint32_t)(piece * kLdsDmaBytes),
                                                 0, 0);
    }

    uint32_t w_off[2];     // this lane's weight piece in group 0 of the stage
    uint32_t w_off_gs[2];  // ... in the group it carries, (lane >> 4) & 1
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        w_off[i] = (uint32_t)(row_of(16 * i + (lane & 15)) * K) + 16u * (lane >> 5);
        w_off_gs[i] = w_off[i] + 32u * ((lane >> 4) & 1);
    }
    // packed: lane (r, c) takes the 16 bytes of its row's K half c in each 1 KB
    // half-block of its row's strip (for a plain strip: bytes 16 l .. 16 l + 15
    // of the workgroup's own blocks), and the 4 bytes of its row's two scales
    const int64_t pk_row = row_of(lane & 31);
    const uint32_t pk_w = (uint32_t)((pk_row / kRows) * P * 2048) + 512u * (lane >> 5) + 16u * (uint32_t)(pk_row % kRows);
    const uint32_t pk_s = (uint32_t)((pk_row / kRows) * P * 128) + 4u * (uint32_t)(pk_row % kRows);
    // direct load i of a stage: columns 8 i .. 8 i + 7 (sized for two tiles: an
    // array whose size depends on the template arguments, captured by the
    // lambdas below, made the host pass drop the kernel stubs)
    uint32_t xd_off[8];
#pragma unroll
    for (int i = 0; i < kXLoads; ++i) {
        const int a = 8 * i + (lane >> 3);
        xd_off[i] = (a < t ? (uint32_t)(a * ldx) * 2u : kPadColumnOffset) + 16u * xs_piece(a, lane);
    }
    const int r = lane & 31;  // weight row of this lane after the swaps (B column, D column)
    const int c = lane >> 5;
    // matrix-core A operand of tile tt: lane (r, c) takes K [16 c, 16 c + 16)
    // of group gs of column 32 tt + r = pieces 4 gs + 2 c (first MFMA) and
    // 4 gs + 2 c + 1 (second)
    uint32_t xa_off[NT][2][2];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
        for (int gs = 0; gs < 2; ++gs)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                xa_off[tt][gs][h] = (uint32_t)(wave * kStageBytes) + xs_off(32 * tt + r, 4 * gs + 2 * c + h);

    double acc[NT][16];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[tt][v] = 0.0;

    const int len = g_end - g_begin;
    const int full = len >> 1;
    const int odd = len & 1;

    // this lane's row of scales (per-stage scale loads), and its place in LDS
    const uint32_t s_row_off = (uint32_t)(row_of(r) * G) * 2u;
    const int s_row_lds = EPI == kEpiSwiGLU ? (r >> 4) * (s_pieces * kLdsDmaBytes / 2) + (r & 15) * G : r * G;

    auto slot = [&](int u) -> unsigned char* { return u == 0 ? xr0 : u == 1 ? xr1 : u == 2 ? xr2 : xr3; };
    // stage starting at group g; `single` loads group g alone in position 0
    // (the odd last group)
    // (packed: the stage block of group g, both groups, and its scale line)
    // (XLc: the number of direct activation loads issued, see `run` below)
    auto load_stage = [&](auto XLc, int g, u32x4 (&w)[2], uint16_t (&sc)[2], uint32_t& sp, unsigned char* xs,
                          bool single) {
        constexpr int XL = decltype(XLc)::value;
        if constexpr (PK) {
            sp = __builtin_amdgcn_raw_buffer_load_b32(s_rsrc, pk_s, g * 64, kStreamOnce);
        } else if constexpr (!LS) {
            sc[0] = __builtin_amdgcn_raw_buffer_load_b16(s_rsrc, s_row_off + 2u * g, 0, 0);
            sc[1] = __builtin_amdgcn_raw_buffer_load_b16(s_rsrc, s_row_off + 2u * (single ? g : g + 1), 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
            w[i] = __builtin_bit_cast(
                u32x4, PK ? __builtin_amdgcn_raw_buffer_load_b128(w_rsrc, pk_w + 1024u * i, g * 1024, kStreamOnce)
                          : __builtin_amdgcn_raw_buffer_load_b128(w_rsrc, single ? w_off[i] : w_off_gs[i], g * kGroup,
                                                                  0));
#pragma unroll
        for (int i = 0; i < XL; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(x_rsrc, W8I_LDS(xs + wave * kStageBytes + i * kLdsDmaBytes), 16,
                                                     xd_off[i], g * (2 * kGroup), 0, 0);
    };
    // group gs of the stage (weights already swapped), acc += s * D_g in fp64,
    // for the values of the column groups below XL = XLc (value v of tile tt
    // holds columns of group 4 tt + v / 4); the other values are padding
    // columns, never stored, so their products are not formed, and a tile
    // with no live value is skipped whole
    auto step = [&](auto XLc, const u32x4 (&w)[2], const uint16_t (&ss)[2], uint32_t sp, const unsigned char* xs,
                    int gs, int g) {
        constexpr int XL = decltype(XLc)::value;
        const bf16x8 b_lo = dequant8(w[gs].x, w[gs].y);
        const bf16x8 b_hi = dequant8(w[gs].z, w[gs].w);
        const uint16_t s16 = PK ? (uint16_t)(sp >> (16 * gs)) : LS ? s_lds[s_row_lds + g] : ss[gs];
        const double sc = (double)(float)__builtin_bit_cast(_Float16, s16);
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            const int nv = tile_live_values(tt, XL, (tt == NT - 1) ? kLastValues : 16);
            if (nv == 0) continue;
            const u32x4 a0 = *reinterpret_cast<const u32x4*>(xs + xa_off[tt][gs][0]);
            const u32x4 a1 = *reinterpret_cast<const u32x4*>(xs + xa_off[tt][gs][1]);
            const f32x16 zero = {};
            f32x16 d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a0), b_lo, zero, 0, 0, 0);
            d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a1), b_hi, d, 0, 0, 0);
#pragma unroll
            for (int v = 0; v < nv; ++v) acc[tt][v] = __builtin_fma(sc, (double)d[v], acc[tt][v]);
        }
    };

    // Both groups of a full stage at once, ordered for latency as in the
    // persistent kernel: the A operands are read from LDS first, the two
    // groups' MFMA chains are interleaved, group 0's fp64 epilogue runs under
    // group 1's.  Per output the operations and their order are those of
    // step(0) then step(1).
    auto step2 = [&](auto XLc, const u32x4 (&w)[2], const uint16_t (&ss)[2], uint32_t sp, const unsigned char* xs,
                     int g) {
        constexpr int XL = decltype(XLc)::value;
        u32x4 a[2][NT][2];
#pragma unroll
        for (int gs = 0; gs < 2; ++gs)
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                if (tile_live_values(tt, XL, (tt == NT - 1) ? kLastValues : 16) == 0) continue;
#pragma unroll
                for (int h = 0; h < 2; ++h) a[gs][tt][h] = *reinterpret_cast<const u32x4*>(xs + xa_off[tt][gs][h]);
            }
        bf16x8 b_lo[2], b_hi[2];
        double sc[2];
#pragma unroll
        for (int gs = 0; gs < 2; ++gs) {
            b_lo[gs] = dequant8(w[gs].x, w[gs].y);
            b_hi[gs] = dequant8(w[gs].z, w[gs].w);
            const uint16_t s16 = PK ? (uint16_t)(sp >> (16 * gs)) : LS ? s_lds[s_row_lds + g + gs] : ss[gs];
            sc[gs] = (double)(float)__builtin_bit_cast(_Float16, s16);
        }
        f32x16 d[2][NT];
        const f32x16 zero = {};
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            if (tile_live_values(tt, XL, (tt == NT - 1) ? kLastValues : 16) == 0) continue;
#pragma unroll
            for (int gs = 0; gs < 2; ++gs)
                d[gs][tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[gs][tt][0]), b_lo[gs],
                                                                    zero, 0, 0, 0);
#pragma unroll
            for (int gs = 0; gs < 2; ++gs)
                d[gs][tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[gs][tt][1]), b_hi[gs],
                                                                    d[gs][tt], 0, 0, 0);
        }
#pragma unroll
        for (int gs = 0; gs < 2; ++gs)
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                const int nv = tile_live_values(tt, XL, (tt == NT - 1) ? kLastValues : 16);
#pragma unroll
                for (int v = 0; v < nv; ++v) acc[tt][v] = __builtin_fma(sc[gs], (double)d[gs][tt][v], acc[tt][v]);
            }
    };

    // The stages' loads, for XL = XLc direct activation loads per stage.  A
    // direct load covers 8 columns; those whose 8 columns are all padding
    // (j >= t) are not issued, and their LDS regions are zeroed once here, so
    // the matrix core sees the same zeros for padding columns as it would
    // from loads (and, as for every padding column, nothing of them is
    // stored).  What is computed for the live columns -- the K plan, every
    // MFMA and every rounding -- does not depend on XL; the choice only
    // spares the memory pipeline 1 KB per skipped load (at t = 1, three of
    // every four activation loads) and the VALU the padding columns'
    // products (in `step`).
    auto run = [&](auto XLc) {
        constexpr int XL = decltype(XLc)::value;
        constexpr int kLPS = 2 + XL + (PK ? 1 : LS ? 0 : 2);  // loads per stage
        if constexpr (XL < kXLoads) {
#pragma unroll
            for (int u = 0; u < D; ++u)
#pragma unroll
                for (int i = XL; i < kXLoads; ++i)
                    *reinterpret_cast<u32x4*>(slot(u) + wave * kStageBytes + i * kLdsDmaBytes + 16 * lane) =
                        u32x4{0u, 0u, 0u, 0u};
        }
        u32x4 ring[D][2];
        uint16_t sring[D][2];
        uint32_t pring[D];
        using I0 = std::integral_constant<int, 0>;
        using I1 = std::integral_constant<int, 1>;
        using I2 = std::integral_constant<int, 2>;
        using I3 = std::integral_constant<int, 3>;
        using ID = std::integral_constant<int, D>;
        // (LS) the strip's scales must be in LDS before the first stage: wait for
        // this wave's scale loads (issued before the ring: only the `after`
        // loads issued since may stay pending), then a plain barrier --
        // __syncthreads() would also wait for the ring's loads (its release
        // fence covers all pending LDS writes); the signal fences keep the
        // compiler from moving LDS accesses across it.
        auto scales_ready = [&](auto After) {
            if constexpr (LS) {
                wait_vm<decltype(After)::value>();
                __atomic_signal_fence(__ATOMIC_SEQ_CST);
                __builtin_amdgcn_s_barrier();
                __atomic_signal_fence(__ATOMIC_SEQ_CST);
            }
        };
        int g = g_begin;
        // the stage in ring slot u (its loads have landed)
        auto compute = [&](auto U) {
            constexpr int u = decltype(U)::value;
            if constexpr (!PK) swap16(ring[u][0], ring[u][1]);
            step2(XLc, ring[u], sring[u], pring[u], slot(u), g);
        };
        // Only real stages are loaded: the first min(D, full) up front, then
        // stage q + D right after stage q is computed, while q + D < full.
        // Stage q's loads are complete once only the loads of the stages
        // after it that have been issued are pending (D - 1 of them while
        // the ring is full).  The waits are explicit: the compiler's own
        // tracking of direct-to-LDS loads is not relied on.  Every stage body
        // below is a separate, sequential copy (alternative copies of the same
        // stages in switch cases made the compiler merge them and double the
        // live registers).
        auto wait_stages = [&](int pending) {  // s_waitcnt takes an immediate
            switch (pending) {
                case 0: wait_vm<0>(); break;
                case 1: wait_vm<kLPS>(); break;
                case 2: if constexpr (D > 2) wait_vm<kLPS * 2>(); break;
                default: if constexpr (D > 3) wait_vm<kLPS * 3>(); break;
            }
        };
        auto prefetching = [&](auto U) {
            constexpr int u = decltype(U)::value;
            wait_vm<kLPS * (D - 1)>();
            compute(U);
            __builtin_amdgcn_sched_barrier(0);
            load_stage(XLc, g + 2 * D, ring[u], sring[u], pring[u], slot(u), false);
            __builtin_amdgcn_sched_barrier(0);
            g += 2;
        };
        // the last n stages, the first of them in slot s0
        auto last_one = [&](auto S0, auto Nn, auto Ii) {
            constexpr int n = decltype(Nn)::value, i = decltype(Ii)::value;
            if constexpr (i < n) {
                wait_vm<kLPS * (n - 1 - i)>();
                compute(std::integral_constant<int, (decltype(S0)::value + i) % D>{});
                __builtin_amdgcn_sched_barrier(0);
                g += 2;
            }
        };
        auto last = [&](auto S0, auto Nn) {
            last_one(S0, Nn, I0{});
            last_one(S0, Nn, I1{});
            last_one(S0, Nn, I2{});
            last_one(S0, Nn, I3{});
        };
        // the final full ring: D stages in slots 0..D-1, of which the first r
        // still prefetch (stage u then has D - 1 stages pending after it, the
        // others D - 1 - u + r)
        auto final_one = [&](auto U, int r) {
            constexpr int u = decltype(U)::value;
            if constexpr (u < D) {
                wait_stages(u < r ? D - 1 : D - 1 - u + r);
                compute(U);
                __builtin_amdgcn_sched_barrier(0);
                if (u < r) load_stage(XLc, g + 2 * D, ring[u], sring[u], pring[u], slot(u), false);
                __builtin_amdgcn_sched_barrier(0);
                g += 2;
            }
        };
        // then the r < D stages those prefetched, in slots 0..r-1
        auto after_one = [&](auto U, int r) {
            constexpr int u = decltype(U)::value;
            if constexpr (u < D - 1) {
                if (u < r) {
                    wait_stages(r - 1 - u);
                    compute(U);
                    __builtin_amdgcn_sched_barrier(0);
                    g += 2;
                }
            }
        };
        if (full >= D) {
#pragma unroll
            for (int u = 0; u < D; ++u) load_stage(XLc, g_begin + 2 * u, ring[u], sring[u], pring[u], slot(u), false);
            scales_ready(std::integral_constant<int, kLPS * D>{});
            const int pre = full - D;  // stages followed by a prefetch
            const int nblocks = pre / D;
            for (int blk = 0; blk < nblocks; ++blk) {
                prefetching(I0{});
                prefetching(I1{});
                if constexpr (D > 2) prefetching(I2{});
                if constexpr (D > 3) prefetching(I3{});
            }
            const int r = pre - nblocks * D;
            final_one(I0{}, r);
            final_one(I1{}, r);
            final_one(I2{}, r);
            final_one(I3{}, r);
            after_one(I0{}, r);
            after_one(I1{}, r);
            after_one(I2{}, r);
        } else {
            // fewer full stages than the ring holds (short slices of small K)
            switch (full) {
                case 1:
                    load_stage(XLc, g_begin, ring[0], sring[0], pring[0], slot(0), false);
                    scales_ready(I0{});
                    last(I0{}, I1{});
                    break;
                case 2:
                    if constexpr (D > 2) {
                        load_stage(XLc, g_begin, ring[0], sring[0], pring[0], slot(0), false);
                        load_stage(XLc, g_begin + 2, ring[1], sring[1], pring[1], slot(1), false);
                        scales_ready(I0{});
                        last(I0{}, I2{});
                    }
                    break;
                case 3:
                    if constexpr (D > 3) {
                        load_stage(XLc, g_begin, ring[0], sring[0], pring[0], slot(0), false);
                        load_stage(XLc, g_begin + 2, ring[1], sring[1], pring[1], slot(1), false);
                        load_stage(XLc, g_begin + 4, ring[2], sring[2], pring[2], slot(2), false);
                        scales_ready(I0{});
                        last(I0{}, I3{});
                    }
                    break;
                default: scales_ready(I0{}); break;
            }
        }
        if (odd) {
            // the row's last group (slice 7 when K/32 is odd); the ring is drained
            // and slot 0's region of this wave is free
            // (packed: the block of the last pair, whose second group is padding)
            u32x4 w1[2];
            uint16_t s1[2];
            uint32_t p1;
            load_stage(XLc, g_end - 1, w1, s1, p1, xr0, true);
            wait_vm<0>();
            if constexpr (!PK) swap16(w1[0], w1[1]);
            step(XLc, w1, s1, p1, xr0, 0, g_end - 1);
        }
    };
    // one uniform branch per launch: XL = the column groups holding a live
    // column (two-tile kernels run for t > 32, so theirs start at 4: the first
    // tile whole)
    const int live_groups = (t + 7) / 8;
    if constexpr (kXLoads == 4) {
        switch (live_groups) {
            case 1: run(std::integral_constant<int, 1>{}); break;
            case 2: run(std::integral_constant<int, 2>{}); break;
            case 3: run(std::integral_constant<int, 3>{}); break;
            default: run(std::integral_constant<int, 4>{}); break;
        }
    } else {
        switch (live_groups) {
            case 5: run(std::integral_constant<int, 5>{}); break;
            case 6: run(std::integral_constant<int, 6>{}); break;
            case 7: run(std::integral_constant<int, 7>{}); break;
            case 8: run(std::integral_constant<int, 8>{}); break;
            default: run(std::integral_constant<int, 4>{}); break;
        }
    }

    // Left fold of the 8 slice sums, ((((((s0 + s1) + s2) + s3) + s4) + s5) + s6) + s7,
    // shared by the waves.  Each wave's loads have all landed (the wait below
    // only guards that: its direct loads write its ring regions), then it writes
    // its slice sum into its own regions of ring slots 0 and 1 (values 16 tt + v,
    // the first NT * 8 in slot 0, the rest in slot 1), so only one barrier
    // stands between the last wave's finish and the fold; then wave w folds
    // and stores values V = w, w + 8, ... (V = 16 tt + v) of every lane.
    wait_vm<0>();
    auto part = [&](int w, int V) {
        constexpr int kHalf = NT * 8;
        return reinterpret_cast<double*>((V < kHalf ? xr0 : xr1) + w * kStageBytes) + (V % kHalf) * 64 + lane;
    };
    // (only values of live column groups: the others were not computed)
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
        for (int v = 0; v < ((tt == NT - 1) ? kLastValues : 16); ++v)
            if (4 * tt + (v >> 2) < live_groups) *part(wave, tt * 16 + v) = acc[tt][v];
    __syncthreads();
    const int64_t n = n0 + r;
#pragma unroll
    for (int k = 0; k < 2 * NT; ++k) {
        const int V = wave + kKSlices * k;
        const int tt = V >> 4, v = V & 15;
        if (v >= ((tt == NT - 1) ? kLastValues : 16) || 4 * tt + (v >> 2) >= live_groups) continue;
        double sum = *part(0, V);
#pragma unroll
        for (int w = 1; w < kKSlices; ++w) sum = sum + *part(w, V);
        // MFMA 32x32 result layout: lane holds column (= weight row) lane % 32
        // and rows 8*(v/4) + 4*(lane/32) + v%4 (= activation columns) of tile tt
        const int j = 32 * tt + 8 * (v >> 2) + 4 * c + (v & 3);
        const uint16_t b = f64_to_bf16(sum);
        if constexpr (EPI == kEpiSwiGLU) {
            // lane r < 16 holds gate row h0 + r, lane r + 16 the up row of the
            // same h, both for column j
            const uint16_t up = (uint16_t)__shfl_xor((int)b, 16);
            const int64_t h = h0 + r;
            if (r < 16 && h < ep.F && j < t) Y[(int64_t)j * ldy + h] = swiglu_bf16(b, up);
        } else if constexpr (EPI == kEpiAdd) {
            // the residual element is read before its own output is written
            // (y may be the residual itself)
            if (r < R && n < N && j < t) Y[(int64_t)j * ldy + n] = add_bf16(b, ep.r[(int64_t)j * ep.ldr + n]);
        } else {
            if (r < R && n < N && j < t) Y[(int64_t)j * ldy + n] = b;
        }
    }
}

// ----------------------------------------------------------------------------
// Large N: persistent tiles.  One workgroup per CU streams tiles of 8 strips
// (256 rows); wave w owns strip w of the tile and walks all of K, keeping the
// current slice's sum and the left fold of the finished slices in registers,
// so every output gets exactly the bits of the split-K kernel above.
//
// Work goes in blocks of BS stages (4 with the plain layout, whose SC scale
// loads carry 8 groups; 8 with the packed one, which halves the barriers and
// measured 2-4% faster on a 248320 x 5120 head); a tile is padded to whole
// blocks with phantom stages, whose loads use zero-range descriptors (no
// memory traffic) and whose compute is skipped.  Per block:
//  * the activations of the next block (32 columns x 2 BS groups) are copied to
//    a double-buffered LDS ring by direct loads, 1/8 by each wave, and one
//    barrier publishes them -- one barrier per block, not per stage;
//  * with SC (K/32 % 8 == 0 and 16-byte aligned scales) each lane loads its
//    row's 8 scales of the next block with one 16-byte load; otherwise every
//    stage loads its two scales per row (two 2-byte loads per lane);
//  * weights run one block (BS stages) ahead: in a register ring with the
//    packed layout (its 1 KB loads are already in matrix-core lane order);
//    with the plain layout in a per-wave LDS ring filled by direct loads, the
//    16-byte slot of each piece XOR-swizzled by the row so that the
//    matrix-core reads are free of bank conflicts: with SC, 4 KB slots of two
//    stages, each refilled after its second stage by loads of 8 rows x 128
//    bytes (whole lines: a bare read of the head with 64 bytes per row per
//    load ran at 4.9 TB/s, with 128 at 7.0); otherwise 2 KB stage slots, 4
//    lanes per row's 64 bytes (register loads of 16 rows x 64 bytes, one row
//    per lane, took 4x the L1 accesses and ran 10% slower).
// The loads are issued in a fixed order, so every wait is a constant count.
// ----------------------------------------------------------------------------
constexpr int kTileStrips = kKSlices;  // 8 waves, one 32-row strip each

// a raw buffer descriptor of p with the given range in bytes (0: every load returns zeros
// with no memory access)
template <typename T>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t range_rsrc(const T* p, int range) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(p), (short)0, range, 0x00020000);
}

// DPP controls (GFX9 encoding) for the max epilogue's cross-lane reduction
constexpr int kDppIdentity = 0xE4;       // quad_perm [0, 1, 2, 3]
constexpr int kDppQuadSwap1 = 0xB1;      // quad_perm [1, 0, 3, 2]
constexpr int kDppQuadSwap2 = 0x4E;      // quad_perm [2, 3, 0, 1]
constexpr int kDppRowHalfMirror = 0x141;  // lane i of each 8 takes lane 7 - i
constexpr int kDppRowMirror = 0x140;      // lane i of each 16 takes lane 15 - i
constexpr int kDppRowBcast15 = 0x142;     // lane 15 of each row to every lane of the next row

// Order key of a stored bf16 value for the max epilogue: the fp32 bit pattern
// with the magnitude bits of negative values flipped, so that a signed-integer
// comparison orders numbers as floats do (-0 below +0: either zero may be the
// maximum of a tie); NaN takes the largest key, so any NaN wins, and rows past
// the last (valid false) the key of -inf.
constexpr int kKeyNaN = 0x7FFFFFFF;
constexpr int kKeyNegInf = (int)0x807FFFFFu;
__device__ __forceinline__ int mx_key(uint16_t b, bool valid) {
    const int bits = (int)((uint32_t)b << 16);
    const int k = (b & 0x7FFF) > 0x7F80 ? kKeyNaN : bits ^ ((bits >> 31) & 0x7FFFFFFF);
    return valid ? k : kKeyNegInf;
}
// the float a key stands for (the canonical NaN for the NaN key)
__device__ __forceinline__ float mx_value(int k) {
    return k == kKeyNaN ? __builtin_nanf("") : __builtin_bit_cast(float, k ^ ((k >> 31) & 0x7FFFFFFF));
}

// PK: packed layout (w8_pack): each stage's weights are the strip's 2 KB block
// and its scales one 128-byte line, loaded with the stage.
// MX: the logprob's max epilogue (the head projection fused with the first
// step of the blockwise logprob): besides storing the outputs, the workgroup
// writes, for every live column j, the maximum over the rows n < N of all its
// tiles of the stored values (bf16 widened exactly to fp32), or NaN if one of
// them is NaN, to M[j * ldm + workgroup].  A maximum is exact in any order, so
// the row maximum the logprob takes from these per-workgroup maxima is the one
// it would take from the logits.
template <int TP16, bool SC, bool PK, bool MX = false>
__global__ __launch_bounds__(kGemmThreads) void gemm_w8g32_tiles(
    const int8_t* __restrict__ W, const uint16_t* __restrict__ S, const uint16_t* __restrict__ X,
    uint16_t* __restrict__ Y, int64_t N, int64_t K, int t, int64_t ldx, int64_t ldy, int ntiles,
    float* __restrict__ M, int64_t ldm) {
    constexpr int NT = (TP16 + 1) / 2;
    constexpr int kLastValues = (TP16 & 1) ? 8 : 16;
    constexpr int kBlockStages = PK ? 8 : 4;                      // stages per block (BS)
    constexpr int kStageBytes = NT * kXTileBytes;                 // one stage's activations
    constexpr int kBlockBytes = kBlockStages * kStageBytes;       // one block's
    constexpr int kXLoads = kBlockBytes / kLdsDmaBytes / kTileStrips;  // direct loads per wave per block
    static_assert(!(SC && PK), "packed scales come with each stage");
    static_assert(!SC || kBlockStages == 4, "an SC scale load holds the 8 groups of a 4-stage block");
    static_assert(kXLoads * kTileStrips * kLdsDmaBytes == kBlockBytes && kXLoads <= 4,
                  "a block's activations split evenly, at most 4 direct loads per wave");
    constexpr int LW = SC ? 2 : PK ? 3 : 4;                       // loads per stage (weights [+ scales])
    constexpr int LS = SC ? 1 : 0;                                // scale-chunk loads per block
    // one array per buffer, so each buffer's direct loads are told apart
    __shared__ __align__(16) unsigned char xb0[kBlockBytes];
    __shared__ __align__(16) unsigned char xb1[kBlockBytes];
    // MX: the workgroup's running column maxima (order keys), per 32-column tile
    __shared__ int skey[MX ? 32 * NT : 1];
    // plain layout: each wave's weight stages, one 2 KB slot per stage of a block
    __shared__ __align__(16) unsigned char wl[PK ? 16 : kTileStrips * kBlockStages * 2048];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int G = (int)(K / kGroup);
    const int nst = (G + 1) >> 1;                                 // real stages per tile
    const int nbt = (nst + kBlockStages - 1) / kBlockStages;      // blocks per tile
    const int my_tiles = (ntiles - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
    const int nb = my_tiles * nbt;                                // blocks of this workgroup
    const int r = lane & 31, c = lane >> 5;
    if constexpr (MX) {
        if (wave == 0 && lane < 32)
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) skey[tt * 32 + lane] = kKeyNegInf;
        __syncthreads();
    }

    // packed layout: whole strips of P = ceil(G/2) stage blocks (2 KB of codes, 128 bytes of scales)
    const int64_t P = (G + 1) / 2;
    const int64_t strips = (N + kRows - 1) / kRows;
    // the buffers' ranges in bytes: a load goes through a descriptor with its buffer's
    // range, or with range 0 (phantom stages, blocks past the last), which returns zeros
    // with no memory access; only the range word differs, so one scalar select picks it
    const int w_range = (int)(uint32_t)(PK ? strips * P * 2048 : N * K);
    const int s_range = (int)(uint32_t)(PK ? strips * P * 128 : N * G * 2);
    const int x_range = (int)(uint32_t)(((int64_t)(t - 1) * ldx + K) * 2);

    // direct load i of this wave covers load m = kXLoads * wave + i of the
    // block: stage m / (4 NT), tile (m / 4) % NT, columns 8 (m % 4) .. + 7
    // (sized for two tiles: see xd_off in the split kernel)
    uint32_t xg_off[4];
    uint32_t xl_off[4];
#pragma unroll
    for (int i = 0; i < kXLoads; ++i) {
        const int m = kXLoads * wave + i;
        const int st = m / (4 * NT), tt = (m / 4) % NT;
        const int a = 32 * tt + 8 * (m % 4) + (lane >> 3);
        xg_off[i] = (a < t ? (uint32_t)(a * ldx) * 2u : kPadColumnOffset) + (uint32_t)st * 64u * 2u +
                    16u * xs_piece(a, lane);
        xl_off[i] = (uint32_t)(st * kStageBytes + tt * kXTileBytes + (8 * (m % 4)) * 128);
    }

    // plain layout with 8-scale loads: this lane's offset within pair load i (row
    // 8 i + l / 8 of the strip, its swizzled 16-byte piece, see load_stage); the
    // strip's and the pair's offsets are added per load
    uint32_t wl_off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int rl = 8 * i + (lane >> 3);
        wl_off[i] = (uint32_t)(rl * K) + 16u * (uint32_t)((lane & 7) ^ ((rl >> 1) & 7));
    }

    // tile of block b, first group of block b (wave-uniform)
    auto tile_of = [&](int b) { return (int)blockIdx.x + (b / nbt) * (int)gridDim.x; };
    auto strip_row = [&](int b) { return (int64_t)tile_of(b) * (kTileStrips * kRows) + (int64_t)wave * kRows; };
    auto block_g = [&](int b) { return kBlockStages * 2 * (b % nbt); };

    struct WStage {
        u32x4 w[2];
        uint16_t s[2];
        uint32_t sp;  // packed: the row's two scales
    };
    // Packed layout: where block b's stages start in this wave's strip, worked
    // out once per block (stage u of the block is the strip's stage block
    // block_g(b) / 2 + u, 2 KB of codes and 128 bytes of scales further on),
    // and how many of its stages lie inside K (the others are phantoms).
    // Strips past the last read the last one: valid memory, never stored.
    struct BlockBase {
        uint32_t w, s;  // byte offsets of stage 0's codes and scales
        int nlive;      // stages of the block with g < G (0 past the last block)
    };
    auto block_base = [&](int b) -> BlockBase {
        BlockBase bb{0u, 0u, 0};
        if constexpr (PK) {
            const int bc = b < nb ? b : nb - 1;
            int64_t strip = (int64_t)tile_of(bc) * kTileStrips + wave;
            strip = strip < strips ? strip : strips - 1;
            const int p0 = block_g(bc) >> 1;
            const uint32_t blk = (uint32_t)(strip * P + p0);
            bb.w = blk * 2048u;
            bb.s = blk * 128u;
            bb.nlive = b < nb ? (nst - p0 < kBlockStages ? nst - p0 : kBlockStages) : 0;
        }
        return bb;
    };
    // weights (and per-stage scales) of stage u of block b (bb = block_base(b))
    auto load_stage = [&](int b, int u, WStage& st, const BlockBase& bb) {
        if constexpr (PK) {
            // lane l takes bytes 16 l .. 16 l + 15 of each 1 KB half and its
            // row's scale pair; the stage's offset is a scalar operand
            const bool live = u < bb.nlive;
            const __amdgpu_buffer_rsrc_t wr = range_rsrc(W, live ? w_range : 0);
#pragma unroll
            for (int i = 0; i < 2; ++i)
                st.w[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                        wr, 1024u * i + 16u * lane, bb.w + 2048u * u, kStreamOnce));
            st.sp = __builtin_amdgcn_raw_buffer_load_b32(range_rsrc(S, live ? s_range : 0), 4u * r, bb.s + 128u * u, kStreamOnce);
            return;
        }
        if constexpr (SC) {
            // pairs of stages: after the second stage of pair u / 2 its slot takes
            // the pair of block b, 4 loads of 8 rows x 128 bytes (whole lines: reading
            // 64 bytes per row per load ran the same weights at 4.9 against 7.0 TB/s).
            // Lane l of load i: row 8 i + l / 8 of the strip, into slot l % 8 of that
            // row's 128 bytes in the pair's 4 KB LDS slot; slot s holds the row's piece
            // s ^ (row / 2 % 8) (piece q: stage q / 4 of the pair, group q / 2 % 2,
            // 16-byte half q % 2), so one LDS pass of 16 rows reads 16 bank groups.
            // Past K (odd G, phantom stages) the loads bring bytes that are not used.
            if ((u & 1) == 0) return;
            const int pr = u >> 1;
            const int gp = block_g(b) + 4 * pr;  // first group of the pair
            const bool live = b < nb && gp < G;
            const __amdgpu_buffer_rsrc_t wr = range_rsrc(W, live ? w_range : 0);
            // rows past N (the last strip of a ragged N) lie past the range: their
            // loads bring zeros without a memory access, and they are never stored
            const uint32_t base = (uint32_t)(strip_row(b < nb ? b : nb - 1) * K) + (uint32_t)gp * kGroup;
            unsigned char* slot = wl + (wave * (kBlockStages / 2) + pr) * 4096;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, W8I_LDS(slot + 1024 * i), 16, wl_off[i] + base, 0, 0, 0);
            return;
        }
        const int g = block_g(b) + 2 * u;
        const bool live = b < nb && g < G;
        const __amdgpu_buffer_rsrc_t wr = range_rsrc(W, live ? w_range : 0);
        const int g1 = g + 1 < G ? g + 1 : g;  // odd G: the last stage repeats its group
        const int64_t row0 = strip_row(b < nb ? b : nb - 1);
        {
            // lane l: row 16 i + l / 4 of the strip, into slot l % 4 of that row's 64 bytes in
            // the stage's LDS slot; the slot holds piece (l % 4) ^ (l / 16) (piece p: group
            // p / 2 of the stage, 16-byte half p % 2)
            const int k = lane >> 2;
            const int piece = (lane & 3) ^ ((k >> 2) & 3);
            const int gl = (piece >> 1) ? g1 : g;
            unsigned char* slot = wl + (wave * kBlockStages + u) * 2048;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                int64_t row = row0 + 16 * i + k;
                row = row < N ? row : N - 1;
                const uint32_t off = (uint32_t)(row * K) + (uint32_t)gl * kGroup + 16u * (uint32_t)(piece & 1);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, W8I_LDS(slot + 1024 * i), 16, off, 0, 0, 0);
            }
        }
        if constexpr (!SC) {
            const __amdgpu_buffer_rsrc_t sr = range_rsrc(S, live ? s_range : 0);
            int64_t row = row0 + r;
            row = row < N ? row : N - 1;
            const uint32_t off = (uint32_t)(row * G) * 2u;
            st.s[0] = __builtin_amdgcn_raw_buffer_load_b16(sr, off + 2u * g, 0, 0);
            st.s[1] = __builtin_amdgcn_raw_buffer_load_b16(sr, off + 2u * g1, 0, 0);
        }
    };
    // this lane's row's 8 scales of block b (SC)
    auto load_scales = [&](int b) -> u32x4 {
        const bool live = b < nb;
        int64_t row = strip_row(live ? b : nb - 1) + r;
        row = row < N ? row : N - 1;
        const uint32_t off = (uint32_t)(row * G + block_g(b < nb ? b : nb - 1)) * 2u;
        return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(range_rsrc(S, live ? s_range : 0), off, 0, 0));
    };
    // this wave's share of block b's activations, into buffer xb (its first
    // XL = XLc direct loads)
    auto load_x = [&](auto XLc, int b, unsigned char* xb) {
        constexpr int XL = decltype(XLc)::value;
        const bool live = b < nb;
        const uint32_t g_off = (uint32_t)block_g(live ? b : nb - 1) * 64u;
#pragma unroll
        for (int i = 0; i < XL; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(range_rsrc(X, live ? x_range : 0), W8I_LDS(xb + xl_off[i]), 16,
                                                     xg_off[i] + g_off, 0, 0, 0);
    };

    double acc[NT][16], total[NT][16];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[tt][v] = total[tt][v] = 0.0;

    // `slice` is the slice the next group belongs to; a slice is folded into
    // the running total as soon as the groups before the next stage are done
    // (empty slices, possible when K < 512, fold a +0 sum like any other).
    int slice = 0;
    int next_bound = (int)kslice_begin(G, 1);  // first group of slice `slice + 1`
    auto fold_slice = [&]() {
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                total[tt][v] = slice == 0 ? acc[tt][v] : total[tt][v] + acc[tt][v];
                acc[tt][v] = 0.0;
            }
        ++slice;
        next_bound = (int)kslice_begin(G, slice + 1);
    };

    // The loop, for XL = XLc direct activation loads per wave per block.  With
    // the packed layout, wave w's loads are the 4 column groups of stage w of
    // the block, so every wave has the same XL live ones; loads whose 8
    // columns are all padding are not issued and their LDS regions are
    // zeroed once at entry (the same zeros the loads would bring; what is
    // computed for live columns does not depend on XL).  The plain layout's
    // 4-stage blocks give a stage's column groups to two waves, so it always
    // loads them all.
    // Only the values of the first XG column groups of 8 are computed (with
    // the packed layout the XL groups loaded, otherwise all): the others are
    // padding columns, never stored.
    auto run = [&](auto XLc, auto XGc) {
        constexpr int XL = decltype(XLc)::value;
        constexpr int XG = decltype(XGc)::value;
        // a stage's weights have landed once only the loads issued after them are
        // pending: the block's later stages, the next block's activations (and
        // scales) and the next block's stages already reloaded -- the same count for
        // every stage.  With pairs of stages (SC) that is the other pair's 4 loads:
        // before the first pair's stages the block's second pair, before the second
        // pair's the next block's first pair.
        constexpr int kStageWait = SC ? 4 + XL + LS : (kBlockStages - 1) * LW + XL + LS;
        if constexpr (XL < kXLoads) {
#pragma unroll
            for (int i = XL; i < kXLoads; ++i) {
                *reinterpret_cast<u32x4*>(xb0 + xl_off[i] + 16 * lane) = u32x4{0u, 0u, 0u, 0u};
                *reinterpret_cast<u32x4*>(xb1 + xl_off[i] + 16 * lane) = u32x4{0u, 0u, 0u, 0u};
            }
            __syncthreads();  // (no loads are in flight yet)
        }
        WStage ring[kBlockStages];
        u32x4 sc0 = {}, sc1 = {};
        // prologue: block 0's activations, scales and weights, in this order (the
        // wait counts below depend on it; the scheduling barriers keep it)
        load_x(XLc, 0, xb0);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (SC) sc0 = load_scales(0);
        __builtin_amdgcn_sched_barrier(0);
        {
            const BlockBase bb0 = block_base(0);
#pragma unroll
            for (int u = 0; u < kBlockStages; ++u) {
                load_stage(0, u, ring[u], bb0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }

        // block b: activations in xs, scales in sc; block b + 1 is loaded into
        // xn and sn.  Blocks go in pairs so that buffers and scale registers are
        // named statically; a phantom block pads an odd count.
        auto block = [&](int b, const unsigned char* xs, unsigned char* xn, const u32x4& sc, u32x4& sn) {
            // this wave's direct loads of block b have landed once only the loads
            // issued after them are pending; the barrier publishes all waves'
            wait_vm<LS + kBlockStages * LW>();
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            __builtin_amdgcn_s_barrier();
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            // every wave is past block b - 1, so its buffer takes block b + 1
            __builtin_amdgcn_sched_barrier(0);
            load_x(XLc, b + 1, xn);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (SC) sn = load_scales(b + 1);
            __builtin_amdgcn_sched_barrier(0);
            const bool live = b < nb;
            const int g0 = block_g(b);
            const BlockBase nbb = block_base(b + 1);
            // A one-stage software pipeline.  fetch(u) reads stage u's matrix-core
            // A operands from LDS (the block's activations are all there since the
            // barrier), dequantises its weights from the register ring and decodes
            // its two scales; stage u's MFMAs are issued, its ring slot is reloaded
            // with the next block's stage u, stage u + 1 is fetched under those
            // MFMAs, and only then does stage u's fp64 epilogue run.  Per output the
            // operations and their order are unchanged: group g's two MFMAs from
            // zero, then acc = fma(s_g, D_g, acc) for g and then for g + 1 (odd G:
            // the tile's last stage has one group; its second chain runs on the
            // zero or repeated group the loads bring and is not accumulated).
            struct StageOps {
                u32x4 a[2][NT][2];
                bf16x8 lo[2], hi[2];
                double s[2];
            };
            auto fetch = [&](int u, StageOps& o) {
                WStage& cur = ring[u];
#pragma unroll
                for (int gs = 0; gs < 2; ++gs)
#pragma unroll
                    for (int tt = 0; tt < NT; ++tt) {
                        if (tile_live_values(tt, XG, 16) == 0) continue;
                        const unsigned char* xt = xs + u * kStageBytes + tt * kXTileBytes;
#pragma unroll
                        for (int h = 0; h < 2; ++h)
                            o.a[gs][tt][h] = *reinterpret_cast<const u32x4*>(xt + xs_off(r, 4 * gs + 2 * c + h));
                    }
#pragma unroll
                for (int gs = 0; gs < 2; ++gs) {
                    u32x4 wv;
                    if constexpr (PK) {
                        wv = cur.w[gs];
                    } else if constexpr (SC) {
                        // row r, piece 4 (u % 2) + 2 gs + c of pair u / 2, from its swizzled slot
                        const int q = 4 * (u & 1) + 2 * gs + c;
                        wv = *reinterpret_cast<const u32x4*>(wl + (wave * (kBlockStages / 2) + (u >> 1)) * 4096 +
                                                             r * 128 + 16 * (q ^ ((r >> 1) & 7)));
                    } else {
                        // row r, piece 2 gs + c of the stage, from its swizzled slot: the 16
                        // lanes of one LDS pass (rows 16 i .. 16 i + 15) hit 16 bank groups
                        const int rr = r & 15, q = 2 * gs + c;
                        wv = *reinterpret_cast<const u32x4*>(wl + (wave * kBlockStages + u) * 2048 + (r >> 4) * 1024 +
                                                             rr * 64 + 16 * (q ^ ((rr >> 2) & 3)));
                    }
                    o.lo[gs] = dequant8(wv.x, wv.y);
                    o.hi[gs] = dequant8(wv.z, wv.w);
                    uint16_t s16;
                    if constexpr (SC)
                        s16 = (uint16_t)(sc[u] >> (16 * gs));  // dword u: groups g0 + 2u, g0 + 2u + 1
                    else if constexpr (PK)
                        s16 = (uint16_t)(cur.sp >> (16 * gs));
                    else
                        s16 = cur.s[gs];
                    o.s[gs] = (double)(float)__builtin_bit_cast(_Float16, s16);
                }
            };
            StageOps ops[2];
            // stage 0's loads have landed once only the loads issued after them
            // are pending: the block's other stages, the next block's activations
            // (and scales)
            wait_vm<kStageWait>();
            fetch(0, ops[0]);
#pragma unroll
            for (int u = 0; u < kBlockStages; ++u) {
                StageOps& o = ops[u & 1];
                const int g = g0 + 2 * u;
                const bool work = live && g < G;
                f32x16 d[2][NT];
                if (work) {
                    while (next_bound <= g) fold_slice();
                    const f32x16 zero = {};
#pragma unroll
                    for (int tt = 0; tt < NT; ++tt) {
                        if (tile_live_values(tt, XG, 16) == 0) continue;
#pragma unroll
                        for (int gs = 0; gs < 2; ++gs)
                            d[gs][tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                                __builtin_bit_cast(bf16x8, o.a[gs][tt][0]), o.lo[gs], zero, 0, 0, 0);
#pragma unroll
                        for (int gs = 0; gs < 2; ++gs)
                            d[gs][tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                                __builtin_bit_cast(bf16x8, o.a[gs][tt][1]), o.hi[gs], d[gs][tt], 0, 0, 0);
                    }
                }
                // the loads keep their issue order (the waits count on it); other
                // work may move across
                __builtin_amdgcn_sched_barrier(kKeepVmemOrder);
                load_stage(b + 1, u, ring[u], nbb);
                __builtin_amdgcn_sched_barrier(kKeepVmemOrder);
                if (u + 1 < kBlockStages) {
                    // stage u + 1's loads: after them are pending the block's later
                    // stages, the next block's activations (and scales) and its
                    // stages 0..u -- the same count as for stage 0
                    wait_vm<kStageWait>();
                    fetch(u + 1, ops[(u + 1) & 1]);
                }
                if (work) {
                    const int ngs = g + 1 < G ? 2 : 1;
#pragma unroll
                    for (int gs = 0; gs < 2; ++gs) {
                        if (gs >= ngs) break;
#pragma unroll
                        for (int tt = 0; tt < NT; ++tt) {
                            const int nv = tile_live_values(tt, XG, (tt == NT - 1) ? kLastValues : 16);
#pragma unroll
                            for (int v = 0; v < nv; ++v)
                                acc[tt][v] = __builtin_fma(o.s[gs], (double)d[gs][tt][v], acc[tt][v]);
                        }
                    }
                }
            }
            if (live && b % nbt == nbt - 1) {
                // the tile's last block: fold the remaining slices, store this strip
                while (slice < kKSlices) fold_slice();
                const int64_t n = strip_row(b) + r;
                uint16_t bv[NT][16];
#pragma unroll
                for (int tt = 0; tt < NT; ++tt)
#pragma unroll
                    for (int v = 0; v < ((tt == NT - 1) ? kLastValues : 16); ++v) bv[tt][v] = f64_to_bf16(total[tt][v]);
                if (n < N) {
                    // the lane's column half through an identity DPP move here: a convergent
                    // operation, which the compiler keeps inside this branch, so the store
                    // addresses are formed at the stores instead of being held in registers
                    // across the loop
                    const int ce = __builtin_amdgcn_mov_dpp(c, kDppIdentity, 0xF, 0xF, false);
#pragma unroll
                    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
                        for (int v = 0; v < ((tt == NT - 1) ? kLastValues : 16); ++v) {
                            const int j = 32 * tt + 8 * (v >> 2) + 4 * ce + (v & 3);
                            if (j < t) Y[(int64_t)j * ldy + n] = bv[tt][v];
                        }
                }
                if constexpr (MX) {
                    // lane (r, c) holds row r of the strip for columns 8 (v / 4) + 4 c + v % 4.
                    // Each stored value becomes an order key (mx_key: a signed-integer max
                    // of keys is the float max; NaN has the largest key, rows past N the key
                    // of -inf), and the keys are reduced over the 32 lanes of each half with
                    // DPP moves: within each row of 16 lanes (quad swaps, half-row and row
                    // mirrors), then row 0 into row 1 and row 2 into row 3 (row_bcast:15),
                    // so lanes 16 and 48 hold the strip's column maxima, which join the
                    // workgroup's running maxima in LDS (atomic max)
                    int key[NT][16];
#pragma unroll
                    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
                        for (int v = 0; v < tile_live_values(tt, XG, (tt == NT - 1) ? kLastValues : 16); ++v)
                            key[tt][v] = mx_key(bv[tt][v], n < N);
                    // one DPP step over every key at a time (independent moves back to back);
                    // the last step writes rows 1 and 3 only, the others are not read
                    auto reduce_step = [&](auto ctrl, auto row_mask) {
#pragma unroll
                        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
                            for (int v = 0; v < tile_live_values(tt, XG, (tt == NT - 1) ? kLastValues : 16); ++v)
                                key[tt][v] = max(key[tt][v], __builtin_amdgcn_mov_dpp(key[tt][v], decltype(ctrl)::value,
                                                                                      decltype(row_mask)::value, 0xF, true));
                    };
                    using RowsAll = std::integral_constant<int, 0xF>;
                    reduce_step(std::integral_constant<int, kDppQuadSwap1>{}, RowsAll{});
                    reduce_step(std::integral_constant<int, kDppQuadSwap2>{}, RowsAll{});
                    reduce_step(std::integral_constant<int, kDppRowHalfMirror>{}, RowsAll{});
                    reduce_step(std::integral_constant<int, kDppRowMirror>{}, RowsAll{});
                    reduce_step(std::integral_constant<int, kDppRowBcast15>{}, std::integral_constant<int, 0xA>{});
                    if (r == 16) {
#pragma unroll
                        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
                            for (int v = 0; v < tile_live_values(tt, XG, (tt == NT - 1) ? kLastValues : 16); ++v)
                                atomicMax(&skey[tt * 32 + 8 * (v >> 2) + 4 * c + (v & 3)], key[tt][v]);
                    }
                }
                slice = 0;
                next_bound = (int)kslice_begin(G, 1);
            }
        };
        for (int b = 0; b < nb; b += 2) {
            block(b, xb0, xb1, sc0, sc1);
            block(b + 1, xb1, xb0, sc1, sc0);
        }
        // the phantom block's loads are still in flight: drain them before exit
        wait_vm<0>();
        if constexpr (MX) {
            // every wave's last tile has met the running maxima: wave 0 writes them
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            if (wave == 0 && lane < 32)
#pragma unroll
                for (int tt = 0; tt < NT; ++tt)
                    if (32 * tt + lane < t)
                        M[(int64_t)(32 * tt + lane) * ldm + (int)blockIdx.x] = mx_value(skey[tt * 32 + lane]);
        }
    };
    using G1 = std::integral_constant<int, 1>;
    using G2 = std::integral_constant<int, 2>;
    using G3 = std::integral_constant<int, 3>;
    using GAll = std::integral_constant<int, 4 * NT>;
    if constexpr (PK) {
        switch ((t + 7) / 8) {
            case 1: run(G1{}, G1{}); break;
            case 2: run(G2{}, G2{}); break;
            case 3: run(std::integral_constant<int, kXLoads < 3 ? kXLoads : 3>{}, G3{}); break;
            default: run(std::integral_constant<int, kXLoads>{}, GAll{}); break;
        }
    } else {
        using XAll = std::integral_constant<int, kXLoads>;
        switch ((t + 7) / 8) {
            case 1: run(XAll{}, G1{}); break;
            case 2: run(XAll{}, G2{}); break;
            case 3: run(XAll{}, G3{}); break;
            default: run(XAll{}, GAll{}); break;
        }
    }
}

// Tiles of the persistent kernel; it is used when there are enough of them
// to keep every CU busy for several tiles.
static int tile_count(int64_t N) { return (int)((N + kTileStrips * kRows - 1) / (kTileStrips * kRows)); }

// scales: 0 per-stage 2-byte loads, 1 eight scales per 16-byte load (SC), 2 packed layout (PK)
// M != nullptr: the max epilogue (MX), per-workgroup column maxima into M [t][ldm = workgroups],
// the number of workgroups into *nm
static int launch_tiles(const int8_t* W, const uint16_t* S, const uint16_t* X, int t, int T_pad, uint16_t* Y,
                        int64_t N, int64_t K, int64_t ldx, int64_t ldy, int scales, hipStream_t stream,
                        float* M = nullptr, int* nm = nullptr) {
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return W8I_EHIP;
    const int ntiles = tile_count(N);
    const dim3 grid((unsigned)(ntiles < ncu ? ntiles : ncu)), block(kGemmThreads);
    if (nm) *nm = (int)grid.x;
#define W8I_TILES_LAUNCH(TP, SCV, PKV)                                                                            \
    if (M)                                                                                                        \
        hipLaunchKernelGGL((gemm_w8g32_tiles<TP, SCV, PKV, true>), grid, block, 0, stream, W, S, X, Y, N, K, t, ldx, \
                           ldy, ntiles, M, (int64_t)grid.x);                                                      \
    else                                                                                                          \
        hipLaunchKernelGGL((gemm_w8g32_tiles<TP, SCV, PKV>), grid, block, 0, stream, W, S, X, Y, N, K, t, ldx, ldy, \
                           ntiles, nullptr, (int64_t)0)
    switch (T_pad / 16 * 4 + scales) {
        case 4: W8I_TILES_LAUNCH(1, false, false); break;
        case 5: W8I_TILES_LAUNCH(1, true, false); break;
        case 6: W8I_TILES_LAUNCH(1, false, true); break;
        case 8: W8I_TILES_LAUNCH(2, false, false); break;
        case 9: W8I_TILES_LAUNCH(2, true, false); break;
        case 10: W8I_TILES_LAUNCH(2, false, true); break;
        default: return W8I_ET;
    }
#undef W8I_TILES_LAUNCH
    return hipGetLastError() == hipSuccess ? W8I_OK : W8I_EHIP;
}

// The kernel a call runs: a function of (N, K, T_pad) and of the scales'
// 16-byte alignment, never of t.  All kernels share the K plan, so the choice
// changes no bit of the result.
enum class LinearKernel { kTiles, kSplitLds };
struct LinearPlan {
    LinearKernel kind;
    int tp16;         // T_pad / 16
    int depth;        // ring depth of the LDS-staged split kernel
    bool lds_scales;  // ... and whether it copies the scales to LDS; for the
                      // tiles kernel: whether it loads the scales by blocks
    int rows = kRows; // output rows per workgroup of the split kernel
};

// Plain layout: rows per workgroup so that the workgroups cover every CU
// where 32-row ones would not (N < 256 x 32): ceil(N / 256) rounded up to a
// multiple of 8 (a whole 128-byte line of the packed layout's rows; the
// plain layout's loads are by row anyway).  The packed layout keeps 32: its
// stream reaches the HBM rate from 192 CUs and more workgroups only added
// contention (6144x5120 t = 1: 9.1 -> 9.9 us), while the plain layout gained
// on every shape (6144x5120 t = 32: 16.7 -> 15.6 us, 1024x5120 T_pad 16:
// 12.8 -> 9.9 us).
static int plain_rows_per_workgroup(int64_t N) {
    const int64_t need = (N + 255) / 256;
    return need >= kRows ? kRows : (int)((need + 7) / 8 * 8);
}

// The LDS-staged variant: the deepest ring (3 or 2 stages for one 32-column
// tile, 2 for two) whose LDS leaves room for the strip's scales when they can
// be copied as 16-byte pieces (s_bytes: the scale bytes the strip needs in
// LDS, 0 when they cannot be copied); otherwise the deepest ring with the
// scales loaded per stage.  (A depth of 3 measured faster than 4 at T_pad:
// more loads in flight only queue longer.)
static LinearPlan plan_split(int tp16, int64_t s_bytes) {
    const int nt = (tp16 + 1) / 2;
    const int dmax = nt == 1 ? 3 : 2;
    if (s_bytes > 0) {
        for (int D = dmax; D >= 2; --D)
            if (s_bytes <= split_lds_scale_bytes(nt, D)) return {LinearKernel::kSplitLds, tp16, D, true};
    }
    return {LinearKernel::kSplitLds, tp16, dmax, false};
}

static int64_t round_dma(int64_t bytes) { return (bytes + kLdsDmaBytes - 1) / kLdsDmaBytes * kLdsDmaBytes; }

static LinearPlan plan_linear(int64_t N, int64_t K, int T_pad, const void* S) {
    const int tp16 = T_pad / 16;
    const bool s16 = (reinterpret_cast<uintptr_t>(S) & 15) == 0;
    if (T_pad <= 32 && tile_count(N) >= kMinTilesPerCu * 256) {
        const bool sc = (K / kGroup) % 8 == 0 && s16;
        return {LinearKernel::kTiles, tp16, 0, sc};
    }
    LinearPlan p = plan_split(tp16, s16 ? round_dma(64 * (K / kGroup)) : 0);
    p.rows = plain_rows_per_workgroup(N);
    return p;
}

// SwiGLU rows: two scale blocks of 32 G bytes; the up rows' block starts at
// byte 2 F G, which the 16-byte pieces need 16-byte aligned
static LinearPlan plan_epilogue(int epi, int64_t N, int64_t K, int T_pad, const void* S) {
    const int64_t G = K / kGroup;
    const bool s16 = (reinterpret_cast<uintptr_t>(S) & 15) == 0;
    if (epi == kEpiSwiGLU) return plan_split(T_pad / 16, s16 && ((N / 2) * G) % 8 == 0 ? 2 * round_dma(32 * G) : 0);
    LinearPlan p = plan_split(T_pad / 16, s16 ? round_dma(64 * G) : 0);
    p.rows = plain_rows_per_workgroup(N);
    return p;
}

const char* linear_kernel_name(int64_t N, int64_t K, int T_pad, const void* S) {
    static const char* const tiles[2][2] = {
        {"gemm_w8g32_tiles<1, false, false>", "gemm_w8g32_tiles<1, true, false>"},
        {"gemm_w8g32_tiles<2, false, false>", "gemm_w8g32_tiles<2, true, false>"}};
    static const char* const split_lds[4][3] = {
        {"gemm_w8g32_split_lds<1, 2, true, 0, false>", "gemm_w8g32_split_lds<1, 3, true, 0, false>", ""},
        {"gemm_w8g32_split_lds<2, 2, true, 0, false>", "gemm_w8g32_split_lds<2, 3, true, 0, false>", ""},
        {"gemm_w8g32_split_lds<3, 2, true, 0, false>", "", ""},
        {"gemm_w8g32_split_lds<4, 2, true, 0, false>", "", ""}};
    static const char* const split_lds_gs[4] = {
        "gemm_w8g32_split_lds<1, 3, false, 0, false>", "gemm_w8g32_split_lds<2, 3, false, 0, false>",
        "gemm_w8g32_split_lds<3, 2, false, 0, false>", "gemm_w8g32_split_lds<4, 2, false, 0, false>"};
    if (T_pad != 16 && T_pad != 32 && T_pad != 48 && T_pad != 64) return "";
    const LinearPlan p = plan_linear(N, K, T_pad, S);
    switch (p.kind) {
        case LinearKernel::kTiles: return tiles[p.tp16 - 1][p.lds_scales ? 1 : 0];
        case LinearKernel::kSplitLds:
            return p.lds_scales ? split_lds[p.tp16 - 1][p.depth - 2] : split_lds_gs[p.tp16 - 1];
        default: return "";
    }
}

// Packed layout (scales come with each stage, no LDS for them): the split
// kernel's ring is the only LDS, so with one 32-column tile and a ring of two
// stages (64 KB) two workgroups fit on a CU, one streaming while the other
// starts or folds.  That pays once there are workgroups to spare (at least two
// per CU: 512 row groups of 32); below it the deeper ring of three is faster.
constexpr int64_t kPackedTwoPerCuRows = 512 * 32;

static LinearPlan plan_packed(int tp16, int64_t row_groups) {
    LinearPlan p = plan_split(tp16, 0);
    if ((tp16 + 1) / 2 == 1 && row_groups * kRows >= kPackedTwoPerCuRows) p.depth = 2;
    return p;
}

const char* linear_packed_kernel_name(int64_t N, int64_t K, int T_pad) {
    static const char* const tiles[2] = {"gemm_w8g32_tiles<1, false, true>", "gemm_w8g32_tiles<2, false, true>"};
    static const char* const split[4][2] = {
        {"gemm_w8g32_split_lds<1, 2, false, 0, true>", "gemm_w8g32_split_lds<1, 3, false, 0, true>"},
        {"gemm_w8g32_split_lds<2, 2, false, 0, true>", "gemm_w8g32_split_lds<2, 3, false, 0, true>"},
        {"gemm_w8g32_split_lds<3, 2, false, 0, true>", ""},
        {"gemm_w8g32_split_lds<4, 2, false, 0, true>", ""}};
    (void)K;
    if (T_pad != 16 && T_pad != 32 && T_pad != 48 && T_pad != 64) return "";
    if (T_pad <= 32 && tile_count(N) >= kMinTilesPerCu * 256) return tiles[T_pad / 16 - 1];
    const LinearPlan p = plan_packed(T_pad / 16, (N + kRows - 1) / kRows);
    return split[T_pad / 16 - 1][p.depth - 2];
}

template <int EPI, bool PK = false>
static int launch_split(const LinearPlan& p, const int8_t* W, const uint16_t* S, const uint16_t* X, int t,
                        uint16_t* Y, int64_t N, int64_t K, int64_t ldx, int64_t ldy, LinearEpilogue ep,
                        hipStream_t stream) {
    const int R = EPI == kEpiSwiGLU ? kRows : p.rows;
    if constexpr (EPI == kEpiPair) ep.wg1 = (int)((N + R - 1) / R);
    const int64_t wgs = EPI == kEpiSwiGLU ? (ep.F + kRows / 2 - 1) / (kRows / 2)
                        : EPI == kEpiPair ? ep.wg1 + (ep.N2 + R - 1) / R
                                          : (N + R - 1) / R;
    const dim3 grid((unsigned)wgs);
    const dim3 block(kGemmThreads);
#define W8I_SPLIT_LAUNCH(TP, D, LS)                                                                     \
    case TP * 16 + D * 2 + LS:                                                                          \
        if constexpr (!(PK && LS))                                                                      \
            hipLaunchKernelGGL((gemm_w8g32_split_lds<TP, D, LS, EPI, PK>), grid, block, 0, stream, W, S, X, Y, N, \
                               K, t, ldx, ldy, ep, R);                                                  \
        break;
    switch (p.tp16 * 16 + p.depth * 2 + (p.lds_scales ? 1 : 0)) {
        W8I_SPLIT_LAUNCH(1, 2, true)
        W8I_SPLIT_LAUNCH(1, 3, true)
        W8I_SPLIT_LAUNCH(2, 2, true)
        W8I_SPLIT_LAUNCH(2, 3, true)
        W8I_SPLIT_LAUNCH(3, 2, true)
        W8I_SPLIT_LAUNCH(4, 2, true)
        W8I_SPLIT_LAUNCH(1, 3, false)
        W8I_SPLIT_LAUNCH(2, 3, false)
        W8I_SPLIT_LAUNCH(1, 2, false)
        W8I_SPLIT_LAUNCH(2, 2, false)
        W8I_SPLIT_LAUNCH(3, 2, false)
        W8I_SPLIT_LAUNCH(4, 2, false)
        default:
            return W8I_ET;
    }
#undef W8I_SPLIT_LAUNCH
    return hipGetLastError() == hipSuccess ? W8I_OK : W8I_EHIP;
}

// The width the kernels run at: T_pad, or 32 when T_pad is 48 or 64 and t <= 32.
// Then the second 32-column tile holds padding columns only, and the one-tile
// kernels give every live column the same bits: a column's K plan, MFMAs and
// roundings do not depend on T_pad (nor on which kernel runs it).  Like the
// skipped activation loads, this only decides how much padding is processed.
static int kernel_width(int t, int T_pad) { return T_pad > 32 && t <= 32 ? 32 : T_pad; }

// the K-slice kernels need kKSlices fp64 sums per live output in the workspace
static bool kslice_fits(const void* ws, size_t ws_bytes, int t, int64_t N) {
    return ws && ws_bytes >= (size_t)kKSlices * (size_t)t * (size_t)N * sizeof(double);
}

int launch_linear(const int8_t* W, const uint16_t* S, const uint16_t* X, int t, int T_pad, uint16_t* Y,
                  int64_t N, int64_t K, int64_t ldx, int64_t ldy, hipStream_t stream, void* ws, size_t ws_bytes) {
    T_pad = kernel_width(t, T_pad);
    if (kslice_applies(N, T_pad) && kslice_fits(ws, ws_bytes, t, N))
        return launch_kslice(false, W, S, X, t, T_pad, Y, N, K, ldx, ldy, ws, stream);
    const LinearPlan p = plan_linear(N, K, T_pad, S);
    switch (p.kind) {
        case LinearKernel::kTiles:
            return launch_tiles(W, S, X, t, T_pad, Y, N, K, ldx, ldy, p.lds_scales ? 1 : 0, stream);
        case LinearKernel::kSplitLds:
            return launch_split<kEpiStore>(p, W, S, X, t, Y, N, K, ldx, ldy, LinearEpilogue{nullptr, 0, 0}, stream);
        default:
            return W8I_ESHAPE;
    }
}

int launch_linear_packed(const int8_t* Wp, const uint16_t* Sp, const uint16_t* X, int t, int T_pad, uint16_t* Y,
                         int64_t N, int64_t K, int64_t ldx, int64_t ldy, hipStream_t stream, void* ws,
                         size_t ws_bytes) {
    // the K-slice kernels for small N when the workspace holds their sums, the
    // persistent kernel where it runs the plain layout, else the split kernel
    T_pad = kernel_width(t, T_pad);
    if (kslice_applies(N, T_pad) && kslice_fits(ws, ws_bytes, t, N))
        return launch_kslice(true, Wp, Sp, X, t, T_pad, Y, N, K, ldx, ldy, ws, stream);
    if (T_pad <= 32 && tile_count(N) >= kMinTilesPerCu * 256)
        return launch_tiles(Wp, Sp, X, t, T_pad, Y, N, K, ldx, ldy, 2, stream);
    const LinearPlan p = plan_packed(T_pad / 16, (N + kRows - 1) / kRows);
    return launch_split<kEpiStore, true>(p, Wp, Sp, X, t, Y, N, K, ldx, ldy, LinearEpilogue{nullptr, 0, 0}, stream);
}

int tiles_of(int64_t N) { return tile_count(N); }

// the head projection on the persistent kernel with the max epilogue: y as w8_linear_invariant
// (or _packed) gives it, and M [t][*nm] the column maxima of each of its *nm <= tiles_of(N)
// workgroups; T_pad <= 32 (or 48 / 64 with t <= 32)
int launch_linear_max(bool packed, const int8_t* W, const uint16_t* S, const uint16_t* X, int t, int T_pad,
                      uint16_t* Y, int64_t N, int64_t K, int64_t ldx, int64_t ldy, float* M, int* nm,
                      hipStream_t stream) {
    T_pad = kernel_width(t, T_pad);
    if (T_pad > 32) return W8I_ET;
    const bool s16 = (reinterpret_cast<uintptr_t>(S) & 15) == 0;
    const int scales = packed ? 2 : ((K / kGroup) % 8 == 0 && s16 ? 1 : 0);
    return launch_tiles(W, S, X, t, T_pad, Y, N, K, ldx, ldy, scales, stream, M, nm);
}

int launch_linear_pair(bool packed, const int8_t* W, const uint16_t* S, const uint16_t* X, int t, int T_pad,
                       uint16_t* Y, int64_t N, int64_t K, int64_t ldx, int64_t ldy, LinearEpilogue ep,
                       hipStream_t stream) {
    // the split kernel, planned for the two projections together: rows per
    // workgroup from their total rows; scales staged in LDS only when both
    // scale arrays allow it
    T_pad = kernel_width(t, T_pad);
    if (packed) {
        const LinearPlan p = plan_packed(T_pad / 16, (N + kRows - 1) / kRows + (ep.N2 + kRows - 1) / kRows);
        return launch_split<kEpiPair, true>(p, W, S, X, t, Y, N, K, ldx, ldy, ep, stream);
    }
    const bool s16 = (reinterpret_cast<uintptr_t>(S) & 15) == 0 && (reinterpret_cast<uintptr_t>(ep.S2) & 15) == 0;
    LinearPlan p = plan_split(T_pad / 16, s16 ? round_dma(64 * (K / kGroup)) : 0);
    p.rows = plain_rows_per_workgroup(N + ep.N2);
    return launch_split<kEpiPair>(p, W, S, X, t, Y, N, K, ldx, ldy, ep, stream);
}

int launch_linear_epilogue(int epi, bool packed, const int8_t* W, const uint16_t* S, const uint16_t* X, int t,
                           int T_pad, uint16_t* Y, int64_t N, int64_t K, int64_t ldx, int64_t ldy, LinearEpilogue ep,
                           hipStream_t stream) {
    // (SwiGLU: a workgroup covers 16 gate and 16 up rows, one row group of 32)
    T_pad = kernel_width(t, T_pad);
    const LinearPlan p = packed ? plan_packed(T_pad / 16, epi == kEpiSwiGLU ? (N / 2 + 15) / 16 : (N + kRows - 1) / kRows)
                                : plan_epilogue(epi, N, K, T_pad, S);
    switch (epi * 2 + (packed ? 1 : 0)) {
        case kEpiAdd * 2: return launch_split<kEpiAdd>(p, W, S, X, t, Y, N, K, ldx, ldy, ep, stream);
        case kEpiAdd * 2 + 1: return launch_split<kEpiAdd, true>(p, W, S, X, t, Y, N, K, ldx, ldy, ep, stream);
        case kEpiSwiGLU * 2: return launch_split<kEpiSwiGLU>(p, W, S, X, t, Y, N, K, ldx, ldy, ep, stream);
        case kEpiSwiGLU * 2 + 1:
            return launch_split<kEpiSwiGLU, true>(p, W, S, X, t, Y, N, K, ldx, ldy, ep, stream);
        default: return W8I_ESHAPE;
    }
}

}  // namespace w8i
