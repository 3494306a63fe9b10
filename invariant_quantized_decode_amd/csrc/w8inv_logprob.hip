// w8inv_logprob.hip -- target-token logprob by fixed-width vocabulary blocks.
//
// Method: the tokenspeed "Numerics envelopes" page, alignment.trainer table
// row "--logprob-order blockwise", the "Logprobs" section and the
// block_sumexp leaf contract paragraph: row max, shift by it, sum of exps per
// fixed-width vocabulary block with each block in its own fixed tree, block
// partials in vocabulary order folded left to right in fp32, then
// out = -(log(sum) - (target - max)).
//
// Three launches on the caller's stream:
//  1. block_max    grid (nb, t): exact max (and NaN flag) of each block.
//  2. block_sumexp grid (nb, t): row max from the block maxima (exact), then
//     the block partial in the canonical pairwise tree: thread i owns the E
//     contiguous elements [i*E, (i+1)*E) and reduces them pairwise in
//     registers, the wave combines lanes with xor-1 .. xor-32 butterflies
//     (each step adds two adjacent subtrees; fp32 addition is commutative, so
//     both lanes of a pair hold the same bits), and the four waves' subtrees
//     are added as (w0 + w1) + (w2 + w3).  Every step is a node of
//     T(i,2w) = T(i,w) + T(i+w,w) over the block.
//  3. fold         one thread per column: S = ((P0 + P1) + P2) + ...,
//     LOG32(S), target gather, final subtraction and negation.
// Logits are bf16, widened exactly in registers.  Indices >= V are virtual
// -inf logits: they contribute +0 to a block and nothing to the max.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "w8inv_internal.h"
#include "w8inv_math.h"

namespace w8i {

constexpr int kLpThreads = 256;

template <int C, bool VEC>
__device__ __forceinline__ void load_chunk(const uint16_t* row, int64_t v0, int64_t V, float (&x)[C],
                                           bool (&ok)[C]) {
    if constexpr (VEC && C == 8) {
        if (v0 + 8 <= V) {
            const uint4 q = *reinterpret_cast<const uint4*>(row + v0);
            const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[2 * i] = __uint_as_float(w[i] << 16);
                x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
                ok[2 * i] = ok[2 * i + 1] = true;
            }
            return;
        }
    }
#pragma unroll
    for (int i = 0; i < C; ++i) {
        ok[i] = v0 + i < V;
        x[i] = ok[i] ? bf16_to_f32(row[v0 + i]) : 0.0f;
    }
}

template <int E, bool VEC>
__global__ __launch_bounds__(kLpThreads) void lp_block_max(const uint16_t* __restrict__ L, int64_t V, int64_t ldl,
                                                           int nb, float* __restrict__ M) {
    constexpr int C = E < 8 ? E : 8;
    __shared__ float wmax[kLpThreads / 64];
    __shared__ int wnan[kLpThreads / 64];
    const int b = blockIdx.x, j = blockIdx.y;
    const uint16_t* row = L + (int64_t)j * ldl;
    const int64_t base = (int64_t)b * (E * kLpThreads) + (int64_t)threadIdx.x * E;
    float m = -__builtin_inff();
    int nan = 0;
#pragma unroll
    for (int ci = 0; ci < E / C; ++ci) {
        float x[C];
        bool ok[C];
        load_chunk<C, VEC>(row, base + ci * C, V, x, ok);
#pragma unroll
        for (int i = 0; i < C; ++i) {
            if (ok[i]) {
                if (x[i] != x[i]) nan = 1;
                else m = __builtin_fmaxf(m, x[i]);
            }
        }
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        m = __builtin_fmaxf(m, __shfl_xor(m, off));
        nan |= __shfl_xor(nan, off);
    }
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        wmax[wave] = m;
        wnan[wave] = nan;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float mm = wmax[0];
        int nn = wnan[0];
#pragma unroll
        for (int w = 1; w < kLpThreads / 64; ++w) {
            mm = __builtin_fmaxf(mm, wmax[w]);
            nn |= wnan[w];
        }
        M[(int64_t)j * nb + b] = nn ? __builtin_nanf("") : mm;
    }
}

// max over the block maxima of column j (NaN if any block saw a NaN)
// Row max of column j from its nb block maxima, by all threads of the
// workgroup (NTH threads, NTH / 64 waves) at once: a max is exact in any
// order.  (A +0 / -0 tie may resolve either way; no output bit depends on
// it: the max only enters through l - m, and its sign could matter only for
// a unique maximum.)  nan is set when any block max is NaN.
template <int NTH>
__device__ __forceinline__ float row_max_from_blocks(const float* M, int nb, int j, bool& nan) {
    __shared__ float wmax[NTH / 64];
    __shared__ int wnan[NTH / 64];
    float m = -__builtin_inff();
    int n = 0;
    for (int i = threadIdx.x; i < nb; i += NTH) {
        const float v = M[(int64_t)j * nb + i];
        if (v != v) n = 1;
        else m = __builtin_fmaxf(m, v);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        m = __builtin_fmaxf(m, __shfl_xor(m, off));
        n |= __shfl_xor(n, off);
    }
    if constexpr (NTH > 64) {
        if ((threadIdx.x & 63) == 0) {
            wmax[threadIdx.x >> 6] = m;
            wnan[threadIdx.x >> 6] = n;
        }
        __syncthreads();
#pragma unroll
        for (int w = 0; w < NTH / 64; ++w) {
            m = __builtin_fmaxf(m, wmax[w]);
            n |= wnan[w];
        }
    }
    nan = n != 0;
    return m;
}

// M holds nm partial maxima per column (the nb block maxima, or the head
// projection's per-workgroup maxima when it ran with the max epilogue).
template <int E, bool VEC>
__global__ __launch_bounds__(kLpThreads) void lp_block_sumexp(const uint16_t* __restrict__ L, int64_t V,
                                                              int64_t ldl, int nb, const float* __restrict__ M,
                                                              int nm, float* __restrict__ P) {
    constexpr int C = E < 8 ? E : 8;
    constexpr int NC = E / C;
    __shared__ float wsum[kLpThreads / 64];
    const int b = blockIdx.x, j = blockIdx.y;
    bool nan;
    const float m = row_max_from_blocks<kLpThreads>(M, nm, j, nan);
    if (nan) {
        if (threadIdx.x == 0) P[(int64_t)j * nb + b] = __builtin_nanf("");
        return;
    }
    const uint16_t* row = L + (int64_t)j * ldl;
    const int64_t base = (int64_t)b * (E * kLpThreads) + (int64_t)threadIdx.x * E;

    float cs[NC];
#pragma unroll
    for (int ci = 0; ci < NC; ++ci) {
        float x[C];
        bool ok[C];
        load_chunk<C, VEC>(row, base + ci * C, V, x, ok);
        float e[C];
#pragma unroll
        for (int i = 0; i < C; ++i) {
            const float shifted = x[i] - m;
            e[i] = ok[i] ? exp32(shifted) : 0.0f;
        }
#pragma unroll
        for (int w = 1; w < C; w *= 2)
#pragma unroll
            for (int i = 0; i < C; i += 2 * w) e[i] = e[i] + e[i + w];
        cs[ci] = e[0];
    }
#pragma unroll
    for (int w = 1; w < NC; w *= 2)
#pragma unroll
        for (int i = 0; i < NC; i += 2 * w) cs[i] = cs[i] + cs[i + w];
    float s = cs[0];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) s = s + __shfl_xor(s, off);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) wsum[wave] = s;
    __syncthreads();
    if (threadIdx.x == 0) P[(int64_t)j * nb + b] = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
}

// One wave per column: the block partials are staged in LDS by all lanes
// (their loads in flight together), then lane 0 folds them left to right.
constexpr int kFoldChunk = 1024;  // partials staged per pass
// DIRECT: the blockwise-direct form st - Lg (+0.0 for a certain token) instead
// of the blockwise -(Lg - st) (-0.0); tokenspeed numerics, "Logprobs".
template <bool DIRECT>
__global__ __launch_bounds__(64) void lp_fold(const uint16_t* __restrict__ L, int64_t V, int64_t ldl,
                                               const int64_t* __restrict__ targets, int nb,
                                               const float* __restrict__ M, int nm, const float* __restrict__ P,
                                               float* __restrict__ out) {
    __shared__ __align__(16) float part[kFoldChunk];
    const int j = blockIdx.x;
    const int lane = threadIdx.x;
    bool nan;
    const float m = row_max_from_blocks<64>(M, nm, j, nan);
    float S = 0.0f;
    for (int b0 = 0; b0 < nb; b0 += kFoldChunk) {
        const int n = nb - b0 < kFoldChunk ? nb - b0 : kFoldChunk;
        for (int i = lane; i < n; i += 64) part[i] = P[(int64_t)j * nb + b0 + i];
        __syncthreads();
        if (lane == 0) {
            // S = ((P_0 + P_1) + P_2) + ... in vocabulary order
            int i = 0;
            if (b0 == 0) S = part[i++];
            for (; i + 4 <= n; i += 4) {  // four reads in flight, adds in order
                const float p0 = part[i], p1 = part[i + 1], p2 = part[i + 2], p3 = part[i + 3];
                S = S + p0;
                S = S + p1;
                S = S + p2;
                S = S + p3;
            }
            for (; i < n; ++i) S = S + part[i];
        }
        __syncthreads();
    }
    if (lane != 0) return;
    const int64_t tg = targets[j];
    if (nan || tg < 0 || tg >= V) {
        out[j] = __builtin_nanf("");
        return;
    }
    const float Lg = log32(S);
    const float st = bf16_to_f32(L[(int64_t)j * ldl + tg]) - m;
    if constexpr (DIRECT) {
        out[j] = st - Lg;
    } else {
        const float d = Lg - st;
        out[j] = -d;
    }
}

static int64_t round_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

size_t logprob_workspace_bytes(int t, int64_t V, int block) {
    const int64_t nb = (V + block - 1) / block;
    return (size_t)(2 * round_up((int64_t)t * nb * (int64_t)sizeof(float), 256));
}

// with_max: the block-max pass first (M receives the nb block maxima); otherwise M already holds nm
// partial maxima per column
template <int E>
static void launch_lp_e(const uint16_t* L, int64_t V, int64_t ldl, int nb, int t, float* M, int nm, float* P,
                        bool vec, bool with_max, hipStream_t stream) {
    const dim3 grid(nb, t), block(kLpThreads);
    if constexpr (E >= 8) {
        if (vec) {
            if (with_max) hipLaunchKernelGGL((lp_block_max<E, true>), grid, block, 0, stream, L, V, ldl, nb, M);
            hipLaunchKernelGGL((lp_block_sumexp<E, true>), grid, block, 0, stream, L, V, ldl, nb, M, nm, P);
            return;
        }
    }
    if (with_max) hipLaunchKernelGGL((lp_block_max<E, false>), grid, block, 0, stream, L, V, ldl, nb, M);
    hipLaunchKernelGGL((lp_block_sumexp<E, false>), grid, block, 0, stream, L, V, ldl, nb, M, nm, P);
}

static int launch_lp(const uint16_t* L, const int64_t* targets, int block, float* out, int t, int64_t V, int64_t ldl,
                     float* M, int nm, float* P, bool with_max, bool direct, hipStream_t stream) {
    const int nb = (int)((V + block - 1) / block);
    const bool vec = (reinterpret_cast<uintptr_t>(L) % 16 == 0) && (ldl % 8 == 0);
    switch (block / kLpThreads) {
        case 1: launch_lp_e<1>(L, V, ldl, nb, t, M, nm, P, vec, with_max, stream); break;
        case 2: launch_lp_e<2>(L, V, ldl, nb, t, M, nm, P, vec, with_max, stream); break;
        case 4: launch_lp_e<4>(L, V, ldl, nb, t, M, nm, P, vec, with_max, stream); break;
        case 8: launch_lp_e<8>(L, V, ldl, nb, t, M, nm, P, vec, with_max, stream); break;
        case 16: launch_lp_e<16>(L, V, ldl, nb, t, M, nm, P, vec, with_max, stream); break;
        case 32: launch_lp_e<32>(L, V, ldl, nb, t, M, nm, P, vec, with_max, stream); break;
        case 64: launch_lp_e<64>(L, V, ldl, nb, t, M, nm, P, vec, with_max, stream); break;
        case 128: launch_lp_e<128>(L, V, ldl, nb, t, M, nm, P, vec, with_max, stream); break;
        default: return W8I_EBLOCK;
    }
    if (direct)
        hipLaunchKernelGGL(lp_fold<true>, dim3(t), dim3(64), 0, stream, L, V, ldl, targets, nb, M, nm, P, out);
    else
        hipLaunchKernelGGL(lp_fold<false>, dim3(t), dim3(64), 0, stream, L, V, ldl, targets, nb, M, nm, P, out);
    return hipGetLastError() == hipSuccess ? W8I_OK : W8I_EHIP;
}

int launch_logprob(const uint16_t* L, const int64_t* targets, int block, float* out, int t, int64_t V, int64_t ldl,
                   void* ws, bool direct, hipStream_t stream) {
    const int64_t nb = (V + block - 1) / block;
    float* M = static_cast<float*>(ws);
    float* P = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                        round_up((int64_t)t * nb * (int64_t)sizeof(float), 256));
    return launch_lp(L, targets, block, out, t, V, ldl, M, (int)nb, P, true, direct, stream);
}

size_t logprob_from_max_workspace_bytes(int t, int64_t V, int block, int nm) {
    const int64_t nb = (V + block - 1) / block;
    return (size_t)(round_up((int64_t)t * nm * (int64_t)sizeof(float), 256) +
                    round_up((int64_t)t * nb * (int64_t)sizeof(float), 256));
}

int launch_logprob_from_max(const uint16_t* L, const int64_t* targets, int block, float* out, int t, int64_t V,
                            int64_t ldl, void* ws, int nm, hipStream_t stream) {
    float* M = static_cast<float*>(ws);
    float* P = reinterpret_cast<float*>(static_cast<char*>(ws) + round_up((int64_t)t * nm * (int64_t)sizeof(float), 256));
    return launch_lp(L, targets, block, out, t, V, ldl, M, nm, P, false, false, stream);
}

// ------------------------------------------- scratch of the no-alloc entry point
// vocab_block_logprob_noalloc keeps its block maxima and partials here instead
// of in a caller's workspace.  Every GPU the library runs on holds its own copy
// of this array, at its own address, until the process ends.  In host code the
// array's name is not a device address: it is looked up once per device with
// hipGetSymbolAddress (that device current), and only that address is ever
// passed to kernels.
static __device__ __align__(256) unsigned char scratch[W8I_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex scratch_mutex;
void* scratch_ptr[kMaxScratchDevices] = {};
}  // namespace

int noalloc_scratch(void** ptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return W8I_EHIP;
    std::lock_guard<std::mutex> lock(scratch_mutex);
    if (!scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return W8I_EHIP;
        scratch_ptr[dev] = p;
    }
    *ptr = scratch_ptr[dev];
    return W8I_OK;
}

// ------------------------------------------------------- verification hooks

__global__ void exp32_kernel(const float* __restrict__ x, float* __restrict__ y, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) y[i] = exp32(x[i]);
}

__global__ void log32_kernel(const float* __restrict__ x, float* __restrict__ y, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) y[i] = log32(x[i]);
}

int launch_exp32(const float* x, float* y, int64_t n, hipStream_t stream) {
    hipLaunchKernelGGL(exp32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, x, y, n);
    return hipGetLastError() == hipSuccess ? W8I_OK : W8I_EHIP;
}

int launch_log32(const float* x, float* y, int64_t n, hipStream_t stream) {
    hipLaunchKernelGGL(log32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, x, y, n);
    return hipGetLastError() == hipSuccess ? W8I_OK : W8I_EHIP;
}

}  // namespace w8i
