// w8inv_gemm.hip -- the W8A16 (int8 group-32, fp16 scales, bf16 activations)
// decode projection at a fixed width T_pad, with one reduction schedule for
// every t.
//
// Method: the ninfer issue on t-dependent kernel dispatch (GitHub issue 80),
// "Proposal: opt-in fixed decode width" -- the kernel and its internal
// schedule are the same for every real t <= T_pad, padded columns are zero
// and ignored, columns never mix.  Format: table "Where t selects
// arithmetic", row "ops::linear W8G32".
//
// Design for gfx950 (CDNA4):
//  * One workgroup = one strip of 32 output rows x all K.  Its 8 waves take
//    the 8 fixed K-slices (slice i = groups [G*i/8, G*(i+1)/8), G = K/32).
//  * Per 32-element group, each lane loads 16 contiguous weight bytes of its
//    row (row = lane % 32, half = lane / 32) with one 128-bit load; the two
//    8-byte halves feed the B operand of two chained
//    v_mfma_f32_32x32x16_bf16 (A = activations, B = weights), so one group's
//    32 products per output are summed by the matrix core into fp32 from
//    zero.  The same K permutation is applied to the activations.
//  * int8 -> bf16 is exact (7 significant bits); the fp16 group scale is
//    applied afterwards in fp64 (the product is exact there) and the groups
//    are accumulated in fp64 in ascending order inside each slice.
//  * The 8 slice sums meet in LDS in the fixed tree ((0+1)+(2+3))+((4+5)+(6+7)),
//    then wave 0 rounds to bf16 once and stores the real columns.
//  * Every one of the T_pad columns goes through the matrix core for every t;
//    columns >= t are zero registers, never loaded and never stored.
//  * No atomics; nothing depends on t, T_pad, N or the device.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "w8inv_internal.h"
#include "w8inv_math.h"

namespace w8i {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRows = 32;             // output rows per workgroup (MFMA 32x32 tile)
constexpr int kGemmThreads = 64 * kKSlices;
constexpr int kBatch = 4;             // groups whose loads are issued together

// two int8 codes (bytes 2i and 2i+1 of q) -> two bf16 in one dword, exact
__device__ __forceinline__ uint32_t dequant2(uint32_t q, int i) {
    const f32x2 a = {(float)(int8_t)(q >> (16 * i)), (float)(int8_t)(q >> (16 * i + 8))};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(a, bf16x2));
}

// eight int8 codes -> bf16x8 operand (element p = byte p)
__device__ __forceinline__ bf16x8 dequant8(uint32_t q0, uint32_t q1) {
    const u32x4 r = {dequant2(q0, 0), dequant2(q0, 1), dequant2(q1, 0), dequant2(q1, 1)};
    return __builtin_bit_cast(bf16x8, r);
}

template <int NT>  // NT = number of 32-column tiles = ceil(T_pad / 32)
__global__ __launch_bounds__(kGemmThreads) void gemm_w8g32_fixed_width(
    const int8_t* __restrict__ W, const uint16_t* __restrict__ S, const uint16_t* __restrict__ X,
    uint16_t* __restrict__ Y, int64_t N, int64_t K, int t, int64_t ldx, int64_t ldy) {
    // slice partials travel through LDS: slot x tile-value x lane
    __shared__ double red[kKSlices / 2][NT * 16][64];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r = lane & 31;  // B column (weight row) and A row (activation column)
    const int c = lane >> 5;  // which 16-byte half of each 32-byte group
    const int64_t G = K / kGroup;
    const int64_t g_begin = kslice_begin(G, wave);
    const int64_t g_end = kslice_begin(G, wave + 1);

    const int64_t n = (int64_t)blockIdx.x * kRows + r;
    const bool row_ok = n < N;
    const int8_t* wp = W + (row_ok ? n : 0) * K + 16 * c;
    const uint16_t* sp = S + (row_ok ? n : 0) * G;

    const uint16_t* xp[NT];
    bool col_ok[NT];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
        const int j = 32 * tt + r;
        col_ok[tt] = j < t;
        xp[tt] = X + (col_ok[tt] ? j : 0) * ldx + 16 * c;
    }

    double acc[NT][16];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[tt][v] = 0.0;

    for (int64_t g = g_begin; g < g_end; g += kBatch) {
        u32x4 wv[kBatch];
        uint32_t sv[kBatch];
        u32x4 xv[kBatch][NT][2];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int64_t gg = g + u;
            const bool ok = gg < g_end;
            const u32x4 zero = {0u, 0u, 0u, 0u};
            wv[u] = (ok && row_ok) ? *reinterpret_cast<const u32x4*>(wp + kGroup * gg) : zero;
            sv[u] = (ok && row_ok) ? (uint32_t)sp[gg] : 0u;
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    xv[u][tt][h] = (ok && col_ok[tt])
                                       ? *reinterpret_cast<const u32x4*>(xp[tt] + kGroup * gg + 8 * h)
                                       : zero;
            }
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            if (g + u >= g_end) break;  // uniform across the workgroup's wave
            const bf16x8 b_lo = dequant8(wv[u].x, wv[u].y);
            const bf16x8 b_hi = dequant8(wv[u].z, wv[u].w);
            const double s = f16_to_f64(sv[u]);
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                f32x16 d = {};
                d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, xv[u][tt][0]), b_lo, d,
                                                            0, 0, 0);
                d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, xv[u][tt][1]), b_hi, d,
                                                            0, 0, 0);
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[tt][v] = __builtin_fma(s, (double)d[v], acc[tt][v]);
            }
        }
    }

    // fixed tree over the 8 slice sums: level L pairs wave w (left, receives)
    // with wave w + 2^L (right, sends), for w a multiple of 2^(L+1).
#pragma unroll
    for (int level = 0; level < 3; ++level) {
        const int span = 1 << level;
        const bool sender = (wave & (2 * span - 1)) == span;
        const bool receiver = (wave & (2 * span - 1)) == 0;
        const int slot = wave >> (level + 1);
        if (sender) {
#pragma unroll
            for (int tt = 0; tt < NT; ++tt)
#pragma unroll
                for (int v = 0; v < 16; ++v) red[slot][tt * 16 + v][lane] = acc[tt][v];
        }
        __syncthreads();
        if (receiver) {
#pragma unroll
            for (int tt = 0; tt < NT; ++tt)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[tt][v] = acc[tt][v] + red[slot][tt * 16 + v][lane];
        }
        __syncthreads();
    }

    if (wave == 0 && row_ok) {
        // MFMA 32x32 result layout: lane holds column (= weight row) lane % 32
        // and rows 8*(v/4) + 4*(lane/32) + v%4 (= activation columns) of the tile
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int j = 32 * tt + 8 * (v >> 2) + 4 * c + (v & 3);
                if (j < t) Y[(int64_t)j * ldy + n] = f64_to_bf16(acc[tt][v]);
            }
    }
}

int launch_linear(const int8_t* W, const uint16_t* S, const uint16_t* X, int t, int T_pad, uint16_t* Y,
                  int64_t N, int64_t K, int64_t ldx, int64_t ldy, hipStream_t stream) {
    const dim3 grid((unsigned)((N + kRows - 1) / kRows));
    const dim3 block(kGemmThreads);
    const int NT = (T_pad + 31) / 32;
    switch (NT) {
        case 1:
            hipLaunchKernelGGL(gemm_w8g32_fixed_width<1>, grid, block, 0, stream, W, S, X, Y, N, K, t, ldx, ldy);
            break;
        case 2:
            hipLaunchKernelGGL(gemm_w8g32_fixed_width<2>, grid, block, 0, stream, W, S, X, Y, N, K, t, ldx, ldy);
            break;
        default:
            return W8I_ET;
    }
    return hipGetLastError() == hipSuccess ? W8I_OK : W8I_EHIP;
}

}  // namespace w8i
