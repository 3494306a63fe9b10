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

constexpr int kNormThreads = 256;

// One workgroup per column.  The sum of squares is the balanced pairwise fp32
// tree over the H features zero-padded to E*256 (a power of two): thread i
// owns features [i*E, (i+1)*E), reduces them pairwise, then xor butterflies
// and (w0 + w1) + (w2 + w3) complete the tree.
template <int E>
__global__ __launch_bounds__(kNormThreads) void rmsnorm_kernel(const uint16_t* __restrict__ x,
                                                               const uint16_t* __restrict__ w, float eps,
                                                               uint16_t* __restrict__ y, int64_t H, int64_t ldx,
                                                               int64_t ldy) {
    __shared__ float wsum[kNormThreads / 64];
    __shared__ float s_denom;
    const int j = blockIdx.x;
    const uint16_t* xr = x + (int64_t)j * ldx;
    const int64_t base = (int64_t)threadIdx.x * E;
    float sq[E];
#pragma unroll
    for (int i = 0; i < E; ++i) {
        const float v = (base + i < H) ? bf16_to_f32(xr[base + i]) : 0.0f;
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
        const float total = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
        const float mean = total / (float)H;
        s_denom = __builtin_sqrtf(mean + eps);
    }
    __syncthreads();
    const float d = s_denom;
    uint16_t* yr = y + (int64_t)j * ldy;
    for (int64_t h = threadIdx.x; h < H; h += kNormThreads) {
        float v = bf16_to_f32(xr[h]) / d;
        if (w) v = v * bf16_to_f32(w[h]);
        yr[h] = f32_to_bf16(v);
    }
}

__global__ void swiglu_kernel(const uint16_t* __restrict__ gu, uint16_t* __restrict__ y, int64_t F, int64_t ldg,
                              int64_t ldy) {
    const int j = blockIdx.y;
    const int64_t h = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (h >= F) return;
    // fp64: e^-g of any bf16 gate is finite or its silu is below bf16's range,
    // so the only rounding that matters is the final one to bf16 (in fp32,
    // e^-g overflows for g < -88.7 while g e^g u can still be a normal bf16)
    const double g = (double)bf16_to_f32(gu[(int64_t)j * ldg + h]);
    const double u = (double)bf16_to_f32(gu[(int64_t)j * ldg + F + h]);
    const double silu = g / (1.0 + ::exp(-g));
    y[(int64_t)j * ldy + h] = f64_to_bf16(silu * u);
}

__global__ void residual_add_kernel(const uint16_t* a, const uint16_t* b, uint16_t* y, int64_t H, int64_t lda,
                                    int64_t ldb, int64_t ldy) {
    const int j = blockIdx.y;
    const int64_t h = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (h >= H) return;
    const float s = bf16_to_f32(a[(int64_t)j * lda + h]) + bf16_to_f32(b[(int64_t)j * ldb + h]);
    y[(int64_t)j * ldy + h] = f32_to_bf16(s);
}

int launch_rmsnorm(const uint16_t* x, const uint16_t* w, float eps, uint16_t* y, int t, int64_t H, int64_t ldx,
                   int64_t ldy, hipStream_t stream) {
    int64_t P = 1;
    while (P < H) P *= 2;
    const int64_t E = P <= kNormThreads ? 1 : P / kNormThreads;
    const dim3 grid(t), block(kNormThreads);
    switch (E) {
        case 1: hipLaunchKernelGGL(rmsnorm_kernel<1>, grid, block, 0, stream, x, w, eps, y, H, ldx, ldy); break;
        case 2: hipLaunchKernelGGL(rmsnorm_kernel<2>, grid, block, 0, stream, x, w, eps, y, H, ldx, ldy); break;
        case 4: hipLaunchKernelGGL(rmsnorm_kernel<4>, grid, block, 0, stream, x, w, eps, y, H, ldx, ldy); break;
        case 8: hipLaunchKernelGGL(rmsnorm_kernel<8>, grid, block, 0, stream, x, w, eps, y, H, ldx, ldy); break;
        case 16: hipLaunchKernelGGL(rmsnorm_kernel<16>, grid, block, 0, stream, x, w, eps, y, H, ldx, ldy); break;
        case 32: hipLaunchKernelGGL(rmsnorm_kernel<32>, grid, block, 0, stream, x, w, eps, y, H, ldx, ldy); break;
        case 64: hipLaunchKernelGGL(rmsnorm_kernel<64>, grid, block, 0, stream, x, w, eps, y, H, ldx, ldy); break;
        case 128: hipLaunchKernelGGL(rmsnorm_kernel<128>, grid, block, 0, stream, x, w, eps, y, H, ldx, ldy); break;
        case 256: hipLaunchKernelGGL(rmsnorm_kernel<256>, grid, block, 0, stream, x, w, eps, y, H, ldx, ldy); break;
        default: return W8I_ESHAPE;
    }
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
