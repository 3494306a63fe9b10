// w8inv_argmax.hip -- canonical greedy argmax of each column of bf16 logits
// (LM-head epilogue): the maximum, and among equal values the lowest index,
// with -0 and +0 equal.  Method: tokenspeed "Numerics envelopes", "Logprobs"
// section (the vocabulary-parallel argmax packs the maximum and its global
// index into one integer key reduced with MAX, one canonical key for signed
// zeros).  A NaN ranks above every number, and the lowest-index NaN wins.
//
// No floating-point arithmetic: every element becomes a 64-bit key whose high
// half orders the values and whose low half is the complement of the index,
// so the largest key is the answer, and MAX is exact in any order.  Pass 1:
// one workgroup per 4096-entry block and column takes the block's largest key;
// pass 2: one wave per column takes the largest of the block keys.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "w8inv_internal.h"

namespace w8i {

constexpr int kArgThreads = 256;
constexpr int kArgE = kArgmaxBlock / kArgThreads;  // 16 entries per thread

// bf16 bits -> 16-bit code in the order of the values: NaNs become one code
// above +inf, -0 the code of +0, negatives below positives.
__device__ __forceinline__ uint32_t order_code(uint32_t b) {
    if ((b & 0x7fffu) > 0x7f80u) return 0xffffu;  // any NaN
    if (b == 0x8000u) b = 0u;                      // -0 -> +0
    return (b & 0x8000u) ? (~b & 0xffffu) : (b | 0x8000u);
}

__device__ __forceinline__ uint64_t arg_key(uint32_t bits, int64_t v) {
    return ((uint64_t)order_code(bits) << 32) | (uint64_t)(0xffffffffu - (uint32_t)v);
}

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint64_t wave_max(uint64_t k) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) k = max_u64(k, __shfl_xor(k, off));
    return k;
}

// VEC: rows 16-byte aligned (ldl % 8 == 0): 16-byte loads of 8 entries
template <bool VEC>
__global__ __launch_bounds__(kArgThreads) void argmax_block(const uint16_t* __restrict__ L, int64_t V, int64_t ldl,
                                                             int nb, uint64_t* __restrict__ keys) {
    __shared__ uint64_t wk[kArgThreads / 64];
    const int b = blockIdx.x, j = blockIdx.y;
    const uint16_t* row = L + (int64_t)j * ldl;
    const int64_t v0 = (int64_t)b * kArgmaxBlock + (int64_t)threadIdx.x * kArgE;
    uint64_t k = 0;  // below every real key (the smallest real code is that of -inf, 0x007f)
    if (VEC && v0 + kArgE <= V) {
#pragma unroll
        for (int i = 0; i < kArgE; i += 8) {
            const uint4 q = *reinterpret_cast<const uint4*>(row + v0 + i);
            const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int h = 0; h < 8; ++h)
                k = max_u64(k, arg_key((w[h >> 1] >> (16 * (h & 1))) & 0xffffu, v0 + i + h));
        }
    } else {
#pragma unroll
        for (int i = 0; i < kArgE; ++i)
            if (v0 + i < V) k = max_u64(k, arg_key(row[v0 + i], v0 + i));
    }
    k = wave_max(k);
    if ((threadIdx.x & 63) == 0) wk[threadIdx.x >> 6] = k;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint64_t m = wk[0];
#pragma unroll
        for (int w = 1; w < kArgThreads / 64; ++w) m = max_u64(m, wk[w]);
        keys[(int64_t)j * nb + b] = m;
    }
}

__global__ __launch_bounds__(64) void argmax_fold(const uint64_t* __restrict__ keys, int nb,
                                                  int64_t* __restrict__ out) {
    const int j = blockIdx.x;
    uint64_t k = 0;
    for (int b = threadIdx.x; b < nb; b += 64) k = max_u64(k, keys[(int64_t)j * nb + b]);
    k = wave_max(k);
    if (threadIdx.x == 0) out[j] = (int64_t)(0xffffffffu - (uint32_t)(k & 0xffffffffu));
}

size_t argmax_workspace_bytes(int t, int64_t V) {
    const int64_t nb = (V + kArgmaxBlock - 1) / kArgmaxBlock;
    return (size_t)((int64_t)t * nb * 8);
}

int launch_argmax(const uint16_t* L, int64_t* out, int t, int64_t V, int64_t ldl, void* ws, hipStream_t stream) {
    const int64_t nb = (V + kArgmaxBlock - 1) / kArgmaxBlock;
    uint64_t* keys = static_cast<uint64_t*>(ws);
    const bool vec = (reinterpret_cast<uintptr_t>(L) % 16 == 0) && (ldl % 8 == 0);
    const dim3 grid((unsigned)nb, (unsigned)t);
    if (vec)
        hipLaunchKernelGGL(argmax_block<true>, grid, dim3(kArgThreads), 0, stream, L, V, ldl, (int)nb, keys);
    else
        hipLaunchKernelGGL(argmax_block<false>, grid, dim3(kArgThreads), 0, stream, L, V, ldl, (int)nb, keys);
    hipLaunchKernelGGL(argmax_fold, dim3(t), dim3(64), 0, stream, keys, (int)nb, out);
    return hipGetLastError() == hipSuccess ? W8I_OK : W8I_EHIP;
}

}  // namespace w8i
