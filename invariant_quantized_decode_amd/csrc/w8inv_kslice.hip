// w8inv_kslice.hip -- the projection for small N, its K-slices on separate
// workgroups, folded by a second launch.
//
// The K plan gives every output 8 slices (kslice_begin).  The split kernel
// runs the 8 slices of a 32-row strip on the 8 waves of one workgroup, so a
// projection of N rows runs N/32 workgroups: 32 for 1024 rows, an eighth of
// the chip, each wave walking up to 15 stages through a ring of 2-3.  Given
// the caller's optional workspace, workgroup (slice i, strip s) here computes
// slice i's sum of the strip's 32 x t outputs and parks it, in fp64, in the
// workspace; kslice_fold then
// folds each output's 8 slice sums left to right and rounds once.  Every
// output gets the bits of the split kernel: the same stages, the same two
// chained MFMAs per group from zero, the same fma(s, D, acc) sequence from +0
// in ascending group order, the same left fold and the same rounding; only
// where each step runs differs.
//
// Inside the workgroup the slice's stages are dealt to 4 waves (stage q to
// wave q % 4) in chunks of 4 * DR stages, all of a chunk's loads in flight at
// once: each wave forms its stages' fp32 group sums with the matrix cores and
// parks them, with the group scales, in LDS; after a barrier each thread
// accumulates its 4 outputs over the chunk's groups in ascending order.  The
// fp32 group sums, not fp64 partial sums, are what crosses between waves, so
// the fp64 sequence of every output stays the single ascending chain.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "w8inv_gemm_common.h"
#include "w8inv_internal.h"
#include "w8inv_math.h"

namespace w8i {

constexpr int kKsWaves = 4;
constexpr int kKsThreads = 64 * kKsWaves;
constexpr int kFoldThreads = 256;

// The workspace query offers the K-slice kernels where a strip count this
// small leaves most of the chip idle under the split kernel (N <= 2048 rows)
// and the width is one 32-column tile; they run when the caller passes it.
// (Measured on MI355X at 1024 x 5120: 8.2 us against the one-launch kernel's
// 7.1 at t = 1, 11.0 against 11.7 at t = 32 -- the fold launch and the
// kernel's own round trip cost what the extra workgroups save, so the
// workspace stays optional.)
constexpr int64_t kKsliceMaxStrips = 64;

bool kslice_applies(int64_t N, int T_pad) { return T_pad <= 32 && (N + kRows - 1) / kRows <= kKsliceMaxStrips; }

// fp64 slice sums [8][t][N] for the largest t of a call at this T_pad
size_t kslice_workspace_bytes(int64_t N, int T_pad) {
    const int width = T_pad < 32 ? T_pad : 32;
    return kslice_applies(N, width) ? (size_t)kKSlices * (size_t)width * (size_t)N * sizeof(double) : 0;
}

// TP16 = T_pad / 16 (1 or 2): one 32-column tile, of which a lane holds
// kValues values (8 at T_pad 16: columns 0..15).  PK: packed layout.
// Workgroup b: slice b / strips, strip b % strips (the long slices 0..3 are
// dispatched first).  P: fp64 [8][t][N], slice i's sum of output (j, n) at
// (i * t + j) * N + n.
template <int TP16, bool PK>
__global__ __launch_bounds__(kKsThreads) void gemm_w8g32_kslice(const int8_t* __restrict__ W,
                                                                const uint16_t* __restrict__ S,
                                                                const uint16_t* __restrict__ X,
                                                                double* __restrict__ P, int64_t N, int64_t K, int t,
                                                                int64_t ldx, int strips) {
    static_assert(TP16 == 1 || TP16 == 2, "one 32-column tile");
    constexpr int kValues = TP16 == 1 ? 8 : 16;
    constexpr int DR = TP16 == 1 ? 4 : 3;  // stages per wave per chunk
    constexpr int CS = kKsWaves * DR;      // stages per chunk
    constexpr int kXLoads = 4;             // direct loads of 8 columns per stage
    // activation stages (one region per wave and chunk slot), the chunk's fp32
    // group sums [group][value][lane] and scales [group][row]
    __shared__ __align__(16) unsigned char xs[kKsWaves * DR * kXTileBytes];
    __shared__ __align__(16) float dsum[2 * CS * kValues * 64];
    __shared__ uint16_t ssc[2 * CS * kRows];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int slice = __builtin_amdgcn_readfirstlane((int)blockIdx.x / strips);
    const int strip = (int)blockIdx.x - slice * strips;
    const int G = (int)(K / kGroup);
    const int gb = __builtin_amdgcn_readfirstlane((int)kslice_begin(G, slice));
    const int ge = __builtin_amdgcn_readfirstlane((int)kslice_begin(G, slice + 1));
    const int len = ge - gb;
    const int ns = (len + 1) / 2;  // stages; the last holds one group when len is odd
    const int64_t n0 = (int64_t)strip * kRows;
    // rows past N read row N - 1 (valid memory; their sums are never stored)
    auto row_of = [&](int rho) -> int64_t {
        const int64_t n = n0 + rho;
        return n < N ? n : N - 1;
    };
    const int r = lane & 31;
    const int c = lane >> 5;

    const int64_t PP = (G + 1) / 2;  // stage blocks per strip of the packed layout
    const __amdgpu_buffer_rsrc_t w_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t*>(W), (short)0, (int)(uint32_t)(PK ? (int64_t)strips * PP * 2048 : N * K), 0x00020000);
    const __amdgpu_buffer_rsrc_t x_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(X), (short)0, (int)(uint32_t)(((int64_t)(t - 1) * ldx + K) * 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t s_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(S), (short)0,
        (int)(uint32_t)(PK ? (int64_t)strips * PP * 128 : N * (int64_t)G * 2), 0x00020000);

    // plain layout: the weight-load lanes of the split kernel (16 rows x 64
    // bytes per instruction, then swap16), per-element scale loads
    uint32_t w_off[2], w_off_gs[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        w_off[i] = (uint32_t)(row_of(16 * i + (lane & 15)) * K) + 16u * (lane >> 5);
        w_off_gs[i] = w_off[i] + 32u * ((lane >> 4) & 1);
    }
    const uint32_t s_row_off = (uint32_t)(row_of(r) * G) * 2u;
    // packed layout: lane (r, c) takes the 16 bytes of its row's K half c in
    // each 1 KB half-block, and the 4 bytes of its row's two scales
    const int64_t pk_row = row_of(r);
    const uint32_t pk_w = (uint32_t)((pk_row / kRows) * PP * 2048) + 512u * (uint32_t)c + 16u * (uint32_t)(pk_row % kRows);
    const uint32_t pk_s = (uint32_t)((pk_row / kRows) * PP * 128) + 4u * (uint32_t)(pk_row % kRows);
    // direct activation load i: columns 8 i .. 8 i + 7, piece xs_piece of each
    uint32_t xd_off[kXLoads];
#pragma unroll
    for (int i = 0; i < kXLoads; ++i) {
        const int a = 8 * i + (lane >> 3);
        xd_off[i] = (a < t ? (uint32_t)(a * ldx) * 2u : kPadColumnOffset) + 16u * xs_piece(a, lane);
    }
    // matrix-core A operand: lane (r, c) takes pieces 4 gs + 2 c (first MFMA)
    // and 4 gs + 2 c + 1 (second) of column r
    uint32_t xa_off[2][2];
#pragma unroll
    for (int gs = 0; gs < 2; ++gs)
#pragma unroll
        for (int h = 0; h < 2; ++h) xa_off[gs][h] = xs_off(r, 4 * gs + 2 * c + h);
    auto slot = [&](int k) -> unsigned char* { return xs + (wave * DR + k) * kXTileBytes; };

    // Phase-two ownership: thread (kq, al) accumulates values 4 kq .. 4 kq + 3
    // of lane al's 32x32 result: row al % 32, columns 8 kq + 4 (al / 32) + u.
    const int al = threadIdx.x & 63;
    const int kq = threadIdx.x >> 6;
    double acc[4] = {0.0, 0.0, 0.0, 0.0};

    auto run = [&](auto XLc) {
        constexpr int XL = decltype(XLc)::value;                      // live column groups of 8
        constexpr int NVL = tile_live_values(0, XL, kValues);         // live values per lane
        constexpr int kLPS = 2 + XL + (PK ? 1 : 2);                   // loads per stage
        // regions of loads that are not issued (all 8 columns padding) hold zeros
        if constexpr (XL < kXLoads) {
#pragma unroll
            for (int k = 0; k < DR; ++k)
#pragma unroll
                for (int i = XL; i < kXLoads; ++i)
                    *reinterpret_cast<u32x4*>(slot(k) + i * kLdsDmaBytes + 16 * lane) = u32x4{0u, 0u, 0u, 0u};
        }
        for (int c0 = 0; c0 < ns; c0 += CS) {
            // this wave's stages of the chunk: q = c0 + wave + 4 k, k < nk
            const int nk = __builtin_amdgcn_readfirstlane(
                c0 + wave >= ns ? 0 : (ns - 1 - c0 - wave) / kKsWaves + 1 < DR ? (ns - 1 - c0 - wave) / kKsWaves + 1 : DR);
            u32x4 wr[DR][2];
            uint16_t sr[DR][2];
            uint32_t pr[DR];
#pragma unroll
            for (int k = 0; k < DR; ++k) {
                if (k < nk) {
                    const int g = gb + 2 * (c0 + wave + kKsWaves * k);
                    const bool single = g + 1 == ge;
                    if constexpr (PK) {
                        pr[k] = __builtin_amdgcn_raw_buffer_load_b32(s_rsrc, pk_s, g * 64, kStreamOnce);
                    } else {
                        sr[k][0] = __builtin_amdgcn_raw_buffer_load_b16(s_rsrc, s_row_off + 2u * g, 0, 0);
                        sr[k][1] = __builtin_amdgcn_raw_buffer_load_b16(s_rsrc, s_row_off + 2u * (single ? g : g + 1),
                                                                        0, 0);
                    }
#pragma unroll
                    for (int i = 0; i < 2; ++i)
                        wr[k][i] = __builtin_bit_cast(
                            u32x4, PK ? __builtin_amdgcn_raw_buffer_load_b128(w_rsrc, pk_w + 1024u * i, g * 1024,
                                                                              kStreamOnce)
                                      : __builtin_amdgcn_raw_buffer_load_b128(
                                            w_rsrc, single ? w_off[i] : w_off_gs[i], g * kGroup, 0));
#pragma unroll
                    for (int i = 0; i < XL; ++i)
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(x_rsrc, W8I_LDS(slot(k) + i * kLdsDmaBytes), 16,
                                                                 xd_off[i], g * (2 * kGroup), 0, 0);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < DR; ++k) {
                if (k < nk) {
                    // stage k has landed once only the later stages' loads are pending
                    switch (nk - 1 - k) {
                        case 0: wait_vm<0>(); break;
                        case 1: wait_vm<kLPS>(); break;
                        case 2: wait_vm<2 * kLPS>(); break;
                        default: wait_vm<3 * kLPS>(); break;
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    const int q = c0 + wave + kKsWaves * k;
                    const int g = gb + 2 * q;
                    const int ng = g + 1 == ge ? 1 : 2;
                    if constexpr (!PK) swap16(wr[k][0], wr[k][1]);
                    const f32x16 zero = {};
#pragma unroll
                    for (int gs = 0; gs < 2; ++gs) {
                        if (gs < ng) {
                            const u32x4 a0 = *reinterpret_cast<const u32x4*>(slot(k) + xa_off[gs][0]);
                            const u32x4 a1 = *reinterpret_cast<const u32x4*>(slot(k) + xa_off[gs][1]);
                            f32x16 d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                                __builtin_bit_cast(bf16x8, a0), dequant8(wr[k][gs].x, wr[k][gs].y), zero, 0, 0, 0);
                            d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                                __builtin_bit_cast(bf16x8, a1), dequant8(wr[k][gs].z, wr[k][gs].w), d, 0, 0, 0);
                            const int gi = 2 * (q - c0) + gs;
#pragma unroll
                            for (int v = 0; v < NVL; ++v) dsum[(gi * kValues + v) * 64 + lane] = d[v];
                            const uint16_t s16 = PK ? (uint16_t)(pr[k] >> (16 * gs)) : sr[k][gs];
                            if (c == 0) ssc[gi * kRows + r] = s16;
                        }
                    }
                }
            }
            __syncthreads();
            // ascending groups of the chunk: acc = fma(s_g, D_g, acc).  Eight
            // groups' LDS reads are issued before their fmas (indices past the
            // chunk's last group repeat it and are not used), so the chain waits
            // on the fp64 latency, not on one LDS round trip per group.
            if (4 * kq < NVL) {
                const int ngc = len - 2 * c0 < 2 * CS ? len - 2 * c0 : 2 * CS;
                for (int g0 = 0; g0 < ngc; g0 += 8) {
                    uint16_t sv[8];
                    float dv[8][4];
#pragma unroll
                    for (int k = 0; k < 8; ++k) {
                        const int gi = g0 + k < ngc ? g0 + k : ngc - 1;
                        sv[k] = ssc[gi * kRows + (al & 31)];
#pragma unroll
                        for (int u = 0; u < 4; ++u) dv[k][u] = dsum[(gi * kValues + 4 * kq + u) * 64 + al];
                    }
#pragma unroll
                    for (int k = 0; k < 8; ++k) {
                        if (g0 + k < ngc) {
                            const double sc = (double)(float)__builtin_bit_cast(_Float16, sv[k]);
#pragma unroll
                            for (int u = 0; u < 4; ++u) acc[u] = __builtin_fma(sc, (double)dv[k][u], acc[u]);
                        }
                    }
                }
            }
            __syncthreads();
        }
        if (4 * kq < NVL) {
            const int64_t n = n0 + (al & 31);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int j = 8 * kq + 4 * (al >> 5) + u;
                if (j < t && n < N) P[((int64_t)slice * t + j) * N + n] = acc[u];
            }
        }
    };
    const int live_groups = (t + 7) / 8;
    if constexpr (TP16 == 1) {
        if (live_groups == 1)
            run(std::integral_constant<int, 1>{});
        else
            run(std::integral_constant<int, 2>{});
    } else {
        switch (live_groups) {
            case 1: run(std::integral_constant<int, 1>{}); break;
            case 2: run(std::integral_constant<int, 2>{}); break;
            case 3: run(std::integral_constant<int, 3>{}); break;
            default: run(std::integral_constant<int, 4>{}); break;
        }
    }
}

// y[j, n] = bf16(((((((P0 + P1) + P2) + P3) + P4) + P5) + P6) + P7), the left
// fold of output (j, n)'s slice sums, rounded once
__global__ __launch_bounds__(kFoldThreads) void kslice_fold(const double* __restrict__ P, uint16_t* __restrict__ Y,
                                                            int64_t N, int t, int64_t ldy) {
    const int64_t n = (int64_t)blockIdx.x * kFoldThreads + threadIdx.x;
    const int j = (int)blockIdx.y;
    if (n >= N) return;
    const int64_t stride = (int64_t)t * N;
    const double* p = P + (int64_t)j * N + n;
    double sum = p[0];
#pragma unroll
    for (int w = 1; w < kKSlices; ++w) sum = sum + p[w * stride];
    Y[(int64_t)j * ldy + n] = f64_to_bf16(sum);
}

// T_pad here is the width the kernels run at (16 or 32); the caller checked
// kslice_applies and that ws holds kKSlices * t * N doubles
int launch_kslice(bool packed, const int8_t* W, const uint16_t* S, const uint16_t* X, int t, int T_pad, uint16_t* Y,
                  int64_t N, int64_t K, int64_t ldx, int64_t ldy, void* ws, hipStream_t stream) {
    const int strips = (int)((N + kRows - 1) / kRows);
    double* P = static_cast<double*>(ws);
    const dim3 grid((unsigned)(strips * kKSlices));
    const dim3 block(kKsThreads);
    if (T_pad <= 16) {
        if (packed)
            hipLaunchKernelGGL((gemm_w8g32_kslice<1, true>), grid, block, 0, stream, W, S, X, P, N, K, t, ldx, strips);
        else
            hipLaunchKernelGGL((gemm_w8g32_kslice<1, false>), grid, block, 0, stream, W, S, X, P, N, K, t, ldx, strips);
    } else {
        if (packed)
            hipLaunchKernelGGL((gemm_w8g32_kslice<2, true>), grid, block, 0, stream, W, S, X, P, N, K, t, ldx, strips);
        else
            hipLaunchKernelGGL((gemm_w8g32_kslice<2, false>), grid, block, 0, stream, W, S, X, P, N, K, t, ldx, strips);
    }
    const dim3 fgrid((unsigned)((N + kFoldThreads - 1) / kFoldThreads), (unsigned)t);
    hipLaunchKernelGGL(kslice_fold, fgrid, dim3(kFoldThreads), 0, stream, P, Y, N, t, ldy);
    return hipGetLastError() == hipSuccess ? W8I_OK : W8I_EHIP;
}

}  // namespace w8i
