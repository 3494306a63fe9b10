// w8calib.hip -- calibration kernels (libw8calib.so): the practical read
// ceiling of one launch and the dense bf16 matrix-core rate of the device.
// They frame the decode projection's roofline figures; no decode result
// depends on them.  Interface and conventions: include/w8calib.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "w8calib.h"
#include "w8inv.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kReadThreads = 512;
constexpr int kReadUnroll = 8;      // 16-byte loads in flight per thread
constexpr uint32_t kNever = 0x9E3779B9u;  // the sink is written only on this XOR value

// Workgroup b reads 16-byte words [b * per, min((b + 1) * per, n16)).
__global__ __launch_bounds__(kReadThreads) void stream_read(const u32x4* __restrict__ p, int64_t n16, int64_t per,
                                                            uint32_t* __restrict__ sink) {
    const int64_t begin = (int64_t)blockIdx.x * per;
    const int64_t end = begin + per < n16 ? begin + per : n16;
    uint32_t x = 0;
    for (int64_t i = begin + threadIdx.x; i < end; i += kReadThreads * kReadUnroll) {
        u32x4 v[kReadUnroll];
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) {
            const int64_t j = i + (int64_t)kReadThreads * u;
            v[u] = j < end ? __builtin_nontemporal_load(p + j) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (x == kNever) sink[(int64_t)blockIdx.x * kReadThreads + threadIdx.x] = x;
}

// The persistent projection's decomposition over the packed layout: workgroup b takes tiles
// b, b + gridDim.x, ... of 8 strips, wave w strip w of the tile; a strip is `pairs` blocks of
// 2048 code bytes (two 1 KB loads) and 128 scale bytes (a 4-byte load per lane of the first 32),
// read in order with kStripDepth blocks in flight per wave.  Every access goes through a buffer
// descriptor of exactly strips * pairs * 2048 (codes) and strips * pairs * 128 (scales) bytes.
constexpr int kStripDepth = 8;
__global__ __launch_bounds__(kReadThreads) void strip_read(const uint8_t* __restrict__ codes,
                                                          const uint8_t* __restrict__ scales, int strips, int pairs,
                                                          uint32_t* __restrict__ sink) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const __amdgpu_buffer_rsrc_t cr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(codes), (short)0, (int)(uint32_t)((int64_t)strips * pairs * 2048), 0x00020000);
    const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(scales), (short)0, (int)(uint32_t)((int64_t)strips * pairs * 128), 0x00020000);
    const int tiles = (strips + 7) / 8;
    uint32_t x = 0;
    for (int tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
        int s = tile * 8 + wave;
        s = s < strips ? s : strips - 1;
        for (int p0 = 0; p0 < pairs; p0 += kStripDepth) {
            u32x4 v[kStripDepth][2];
            uint32_t sv[kStripDepth];
#pragma unroll
            for (int d = 0; d < kStripDepth; ++d) {
                const int p = p0 + d < pairs ? p0 + d : pairs - 1;
                const uint32_t blk = (uint32_t)s * (uint32_t)pairs + (uint32_t)p;
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    v[d][i] = __builtin_bit_cast(
                        u32x4, __builtin_amdgcn_raw_buffer_load_b128(cr, 1024u * i + 16u * lane, blk * 2048u, 2));
                sv[d] = __builtin_amdgcn_raw_buffer_load_b32(sr, 4u * (uint32_t)(lane & 31), blk * 128u, 2);
            }
#pragma unroll
            for (int d = 0; d < kStripDepth; ++d)
#pragma unroll
                for (int i = 0; i < 2; ++i) x ^= v[d][i].x ^ v[d][i].y ^ v[d][i].z ^ v[d][i].w ^ sv[d];
        }
    }
    if (x == kNever) sink[(int64_t)blockIdx.x * kReadThreads + threadIdx.x] = x;
}

constexpr int kMfmaThreads = 256;  // 4 waves
constexpr int kChains = 4;         // independent accumulators per wave

__global__ __launch_bounds__(kMfmaThreads) void mfma_bf16(int iters, float* __restrict__ sink) {
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)(float)((lane + e) & 7);
        b[e] = (__bf16)(float)((lane * 3 + e) & 7);
    }
    f32x16 c[kChains];
#pragma unroll
    for (int k = 0; k < kChains; ++k) c[k] = f32x16{};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int k = 0; k < kChains; ++k) c[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[k], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < kChains; ++k)
#pragma unroll
        for (int v = 0; v < 16; ++v) s += c[k][v];
    if (__builtin_bit_cast(uint32_t, s) == kNever) sink[(int64_t)blockIdx.x * kMfmaThreads + threadIdx.x] = s;
}

int launch_status() { return hipGetLastError() == hipSuccess ? W8I_OK : W8I_EHIP; }

}  // namespace

extern "C" int w8c_stream_read(const void* buf, int64_t bytes, int32_t workgroups, void* sink, size_t sink_bytes,
                               void* stream) {
    if (buf == nullptr || sink == nullptr) return W8I_ENULL;
    if (bytes <= 0 || bytes % 16 != 0 || workgroups < 1 || workgroups > 65536) return W8I_ESHAPE;
    if ((reinterpret_cast<uintptr_t>(buf) & 15) != 0 || (reinterpret_cast<uintptr_t>(sink) & 3) != 0)
        return W8I_EALIGN;
    if (sink_bytes < (size_t)workgroups * kReadThreads * sizeof(uint32_t)) return W8I_EWORKSPACE;
    const int64_t n16 = bytes / 16;
    const int64_t per = (n16 + workgroups - 1) / workgroups;
    hipLaunchKernelGGL(stream_read, dim3((unsigned)workgroups), dim3(kReadThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4*>(buf), n16, per,
                       static_cast<uint32_t*>(sink));
    return launch_status();
}

extern "C" int w8c_strip_read(const void* codes, const void* scales, int32_t strips, int32_t pairs,
                              int32_t workgroups, void* sink, size_t sink_bytes, void* stream) {
    if (codes == nullptr || scales == nullptr || sink == nullptr) return W8I_ENULL;
    if (strips < 1 || pairs < 1 || (int64_t)strips * pairs * 2048 >= ((int64_t)1 << 32) || workgroups < 1 ||
        workgroups > 65536)
        return W8I_ESHAPE;
    if ((reinterpret_cast<uintptr_t>(codes) & 15) != 0 || (reinterpret_cast<uintptr_t>(scales) & 3) != 0 ||
        (reinterpret_cast<uintptr_t>(sink) & 3) != 0)
        return W8I_EALIGN;
    if (sink_bytes < (size_t)workgroups * kReadThreads * sizeof(uint32_t)) return W8I_EWORKSPACE;
    hipLaunchKernelGGL(strip_read, dim3((unsigned)workgroups), dim3(kReadThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const uint8_t*>(codes),
                       static_cast<const uint8_t*>(scales), strips, pairs, static_cast<uint32_t*>(sink));
    return launch_status();
}

extern "C" int w8c_mfma_bf16(int32_t workgroups, int32_t iters, void* sink, size_t sink_bytes, void* stream) {
    if (sink == nullptr) return W8I_ENULL;
    if (workgroups < 1 || workgroups > 65536 || iters < 1 || iters > (1 << 20)) return W8I_ESHAPE;
    if ((reinterpret_cast<uintptr_t>(sink) & 3) != 0) return W8I_EALIGN;
    if (sink_bytes < (size_t)workgroups * kMfmaThreads * sizeof(float)) return W8I_EWORKSPACE;
    hipLaunchKernelGGL(mfma_bf16, dim3((unsigned)workgroups), dim3(kMfmaThreads), 0, static_cast<hipStream_t>(stream),
                       iters, static_cast<float*>(sink));
    return launch_status();
}
