// w8inv_glue.hip -- column-local glue between the projections of one decode
// layer: RMSNorm, SwiGLU and the residual add.  The ninfer issue's table
// "Where t selects arithmetic" notes that norms and other per-lane ops are
// invariant; here each column (token) is reduced and transformed on its own,
// with a fixed order, so its bits never depend on the other columns.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "w8inv_internal.h"
#include "w8inv_math.h"

namespace w8i {

constexpr int kNormThreads = 1024;
constexpr int kNormWaves = kNormThreads / 64;

// One workgroup per column.  The sum of squares is the balanced pairwise fp32
// tree over the H features zero-padded to E*1024 (a power of two; padding
// with +0 leaves every partial sum unchanged): thread i owns features
// [i*E, (i+1)*E) and reduces them pairwise, xor butterflies complete each
// wave's 64-thread subtree, and the 16 wave sums are combined pairwise.
// The features stay in registers for the scaling pass.  VEC: the row and the
// weight are 16-byte aligned and E >= 8, so each thread reads 16-byte pieces.
template <int E, bool VEC>
__global__ __launch_bounds__(kNormThreads) void rmsnorm_kernel(const uint16_t* __restrict__ x,
                                                               const uint16_t* __restrict__ w, float eps,
                                                               uint16_t* __restrict__ y, int64_t H, int64_t ldx,
                                                               int64_t ldy) {
    __shared__ float wsum[kNormWaves];
    __shared__ float s_denom;
    const int j = blockIdx.x;
    const uint16_t* xr = x + (int64_t)j * ldx;
    const int64_t base = (int64_t)threadIdx.x * E;
    uint16_t xv[E];
    if (VEC && base + E <= H) {
#pragma unroll
        for (int i = 0; i < E; i += 8) *reinterpret_cast<uint4*>(&xv[i]) = *reinterpret_cast<const uint4*>(xr + base + i);
    } else {
#pragma unroll
        for (int i = 0; i < E; ++i) xv[i] = (base + i < H) ? xr[base + i] : (uint16_t)0;
    }
    float sq[E];
#pragma unroll
    for (int i = 0; i < E; ++i) {
        const float v = bf16_to_f32(xv[i]);
        sq[i] = v * v;
    }
#pragma unroll
    for (int s = 1; s < E; s *= 2)
#pragma unroll
        for (int i = 0; i < E; i += 2 * s) sq[i] = sq[i] + sq[i + s];
    float acc = sq[0];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) acc = acc + __shfl_xor(acc, off);
    if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        float p[kNormWaves];
#pragma unroll
        for (int i = 0; i < kNormWaves; ++i) p[i] = wsum[i];
#pragma unroll
        for (int s = 1; s < kNormWaves; s *= 2)
#pragma unroll
            for (int i = 0; i < kNormWaves; i += 2 * s) p[i] = p[i] + p[i + s];
        const float mean = p[0] / (float)H;
        s_denom = __builtin_sqrtf(mean + eps);
    }
    __syncthreads();
    const float d = s_denom;
    if (base >= H) return;
    uint16_t wv[E];
    if (VEC && base + E <= H) {
        if (w) {
#pragma unroll
            for (int i = 0; i < E; i += 8) *reinterpret_cast<uint4*>(&wv[i]) = *reinterpret_cast<const uint4*>(w + base + i);
        }
        uint16_t yv[E];
#pragma unroll
        for (int i = 0; i < E; ++i) {
            float v = bf16_to_f32(xv[i]) / d;
            if (w) v = v * bf16_to_f32(wv[i]);
            yv[i] = f32_to_bf16(v);
        }
        uint16_t* yr = y + (int64_t)j * ldy + base;
        if (((uintptr_t)yr & 15) == 0) {
#pragma unroll
            for (int i = 0; i < E; i += 8) *reinterpret_cast<uint4*>(yr + i) = *reinterpret_cast<const uint4*>(&yv[i]);
        } else {
#pragma unroll
            for (int i = 0; i < E; ++i) yr[i] = yv[i];
        }
    } else {
        uint16_t* yr = y + (int64_t)j * ldy;
#pragma unroll
        for (int i = 0; i < E; ++i) {
            if (base + i < H) {
                float v = bf16_to_f32(xv[i]) / d;
                if (w) v = v * bf16_to_f32(w[base + i]);
                yr[base + i] = f32_to_bf16(v);
            }
        }
    }
}

__global__ void swiglu_kernel(const uint16_t* __restrict__ gu, uint16_t* __restrict__ y, int64_t F, int64_t ldg,
                              int64_t ldy) {
    const int j = blockIdx.y;
    const int64_t h = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (h >= F) return;
    y[(int64_t)j * ldy + h] = swiglu_bf16(gu[(int64_t)j * ldg + h], gu[(int64_t)j * ldg + F + h]);
}

__global__ void residual_add_kernel(const uint16_t* a, const uint16_t* b, uint16_t* y, int64_t H, int64_t lda,
                                    int64_t ldb, int64_t ldy) {
    const int j = blockIdx.y;
    const int64_t h = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (h >= H) return;
    y[(int64_t)j * ldy + h] = add_bf16(a[(int64_t)j * lda + h], b[(int64_t)j * ldb + h]);
}

int launch_rmsnorm(const uint16_t* x, const uint16_t* w, float eps, uint16_t* y, int t, int64_t H, int64_t ldx,
                   int64_t ldy, hipStream_t stream) {
    int64_t P = 1;
    while (P < H) P *= 2;
    const int64_t E = P <= kNormThreads ? 1 : P / kNormThreads;
    const bool vec = E >= 8 && ((uintptr_t)x & 15) == 0 && ldx % 8 == 0 && (w == nullptr || ((uintptr_t)w & 15) == 0);
    const dim3 grid(t), block(kNormThreads);
#define W8I_NORM(EV)                                                                                            \
    case EV:                                                                                                    \
        if (vec)                                                                                                \
            hipLaunchKernelGGL((rmsnorm_kernel<EV, true>), grid, block, 0, stream, x, w, eps, y, H, ldx, ldy);  \
        else                                                                                                    \
            hipLaunchKernelGGL((rmsnorm_kernel<EV, false>), grid, block, 0, stream, x, w, eps, y, H, ldx, ldy); \
        break;
    switch (E) {
        W8I_NORM(1)
        W8I_NORM(2)
        W8I_NORM(4)
        W8I_NORM(8)
        W8I_NORM(16)
        W8I_NORM(32)
        W8I_NORM(64)
        default: return W8I_ESHAPE;
    }
#undef W8I_NORM
    return hipGetLastError() == hipSuccess ? W8I_OK : W8I_EHIP;
}

int launch_swiglu(const uint16_t* gu, uint16_t* y, int t, int64_t F, int64_t ldg, int64_t ldy, hipStream_t stream) {
    hipLaunchKernelGGL(swiglu_kernel, dim3((unsigned)((F + 255) / 256), t), dim3(256), 0, stream, gu, y, F, ldg, ldy);
    return hipGetLastError() == hipSuccess ? W8I_OK : W8I_EHIP;
}

int launch_residual_add(const uint16_t* a, const uint16_t* b, uint16_t* y, int t, int64_t H, int64_t lda,
                        int64_t ldb, int64_t ldy, hipStream_t stream) {
    hipLaunchKernelGGL(residual_add_kernel, dim3((unsigned)((H + 255) / 256), t), dim3(256), 0, stream, a, b, y, H,
                       lda, ldb, ldy);
    return hipGetLastError() == hipSuccess ? W8I_OK : W8I_EHIP;
}

}  // namespace w8i
