// w8inv_internal.h -- declarations shared by the library's translation units
// (not part of the public ABI; the public header is include/w8inv.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "w8inv.h"

namespace w8i {

constexpr int kGroup = 32;   // K elements per fp16 scale (W8G32)
constexpr int kKSlices = 8;  // fixed number of K-slices per output, for every shape

// First group of K-slice i when K holds G groups.  Slices are made of whole
// pairs of groups, slices 0..3 three times as long as slices 4..7: with P =
// G/2 pairs and cumulative weights c_i = 0, 3, 6, 9, 12, 13, 14, 15, 16,
// slice i covers pairs [floor(P*c_i/16), floor(P*c_{i+1}/16)), and when G is
// odd the row's last group closes slice 7.  The whole K-reduction plan is
// this function of K alone.  (Why unequal: the split kernel gives slice i to
// wave i, and waves 0..3 -- the older wave on each SIMD -- stream their loads
// ahead of waves 4..7, whose first loads queue behind theirs; with equal
// slices the younger waves finished ~2.5 us later, alone on their SIMDs.)
__host__ __device__ __forceinline__ int64_t kslice_begin(int64_t G, int i) {
    if (i >= kKSlices) return G;
    const int64_t c = i <= 4 ? 3 * i : 8 + i;
    return 2 * (((G / 2) * c) / 16);
}

// What the projection kernel stores for output (j, n).
constexpr int kEpiStore = 0;   // y = bf16(W x)
constexpr int kEpiAdd = 1;     // y = residual add of bf16(W x) and r (the glue's w8i_residual_add)
constexpr int kEpiSwiGLU = 2;  // rows [0, F) gate, [F, 2F) up; y[:, h] = SwiGLU(gate h, up h) (w8i_swiglu)
constexpr int kEpiPair = 3;    // two projections of one x: workgroups [0, wg1) the first, the rest the second
struct LinearEpilogue {
    const uint16_t* r = nullptr;  // kEpiAdd: residual, bf16 [t, ldr]
    int64_t ldr = 0;
    int64_t F = 0;                // kEpiSwiGLU: gate rows (the projection has 2F rows)
    // kEpiPair: the second projection (weights, scales, output, rows, output stride) and the
    // number of workgroups of the first (set by the launcher)
    const int8_t* W2 = nullptr;
    const uint16_t* S2 = nullptr;
    uint16_t* Y2 = nullptr;
    int64_t N2 = 0;
    int64_t ldy2 = 0;
    int wg1 = 0;
};

// ws: the caller's workspace (may be null); with at least kKSlices * t * N doubles
// and a small N (kslice_applies) the K-slice kernels run, with the same bits
int launch_linear(const int8_t* W, const uint16_t* S, const uint16_t* X, int t, int T_pad, uint16_t* Y,
                  int64_t N, int64_t K, int64_t ldx, int64_t ldy, hipStream_t stream, void* ws = nullptr,
                  size_t ws_bytes = 0);
// the projection over weights and scales in the packed layout (w8_pack)
int launch_linear_packed(const int8_t* Wp, const uint16_t* Sp, const uint16_t* X, int t, int T_pad, uint16_t* Y,
                         int64_t N, int64_t K, int64_t ldx, int64_t ldy, hipStream_t stream, void* ws = nullptr,
                         size_t ws_bytes = 0);
// Small N (w8inv_kslice.hip): the 8 K-slices of each strip on separate workgroups, their fp64
// sums in a workspace [8][t][N], then the left fold; T_pad is the width the kernels run at.
bool kslice_applies(int64_t N, int T_pad);
size_t kslice_workspace_bytes(int64_t N, int T_pad);  // 0 where the K-slice kernels do not run
int launch_kslice(bool packed, const int8_t* W, const uint16_t* S, const uint16_t* X, int t, int T_pad, uint16_t* Y,
                  int64_t N, int64_t K, int64_t ldx, int64_t ldy, void* ws, hipStream_t stream);
// bytes of the packed layout of an [N, K] projection: 32-row strips x ceil(K/64) blocks
inline int64_t packed_weight_bytes(int64_t N, int64_t K) { return (N + 31) / 32 * ((K / kGroup + 1) / 2) * 2048; }
inline int64_t packed_scale_bytes(int64_t N, int64_t K) { return (N + 31) / 32 * ((K / kGroup + 1) / 2) * 128; }
int launch_pack(const int8_t* W, const uint16_t* S, int64_t N, int64_t K, int8_t* Wp, uint16_t* Sp,
                hipStream_t stream);
// the projection with a fused epilogue (always the LDS-staged split kernel;
// `packed`: W and S in the packed layout);
// for kEpiSwiGLU, N is the projection's 2F rows and y has F columns
int launch_linear_epilogue(int epi, bool packed, const int8_t* W, const uint16_t* S, const uint16_t* X, int t,
                           int T_pad, uint16_t* Y, int64_t N, int64_t K, int64_t ldx, int64_t ldy, LinearEpilogue ep,
                           hipStream_t stream);
// two projections of one x in one launch (the split kernel, kEpiPair): ep carries the second
// projection (W2, S2, Y2, N2, ldy2); `packed`: both in the packed layout
int launch_linear_pair(bool packed, const int8_t* W, const uint16_t* S, const uint16_t* X, int t, int T_pad,
                       uint16_t* Y, int64_t N, int64_t K, int64_t ldx, int64_t ldy, LinearEpilogue ep,
                       hipStream_t stream);
const char* linear_kernel_name(int64_t N, int64_t K, int T_pad, const void* S);
const char* linear_packed_kernel_name(int64_t N, int64_t K, int T_pad);

size_t logprob_workspace_bytes(int t, int64_t V, int block);
int launch_logprob(const uint16_t* L, const int64_t* targets, int block, float* out, int t, int64_t V,
                   int64_t ldl, void* ws, bool direct, hipStream_t stream);
// the logprob whose row maxima come from nm partial maxima per column already in the workspace's
// first part (M [t][nm], then the block partials): the head projection's max epilogue wrote them
size_t logprob_from_max_workspace_bytes(int t, int64_t V, int block, int nm);
int launch_logprob_from_max(const uint16_t* L, const int64_t* targets, int block, float* out, int t, int64_t V,
                            int64_t ldl, void* ws, int nm, hipStream_t stream);
// the persistent projection with the max epilogue: per-workgroup column maxima into M [t][*nm],
// *nm (the number of workgroups) at most tiles_of(N)
int tiles_of(int64_t N);
int launch_linear_max(bool packed, const int8_t* W, const uint16_t* S, const uint16_t* X, int t, int T_pad,
                      uint16_t* Y, int64_t N, int64_t K, int64_t ldx, int64_t ldy, float* M, int* nm,
                      hipStream_t stream);
// device address of the current device's fixed scratch array (W8I_NOALLOC_SCRATCH_BYTES bytes),
// looked up once per device; allocates nothing
int noalloc_scratch(void** ptr);

constexpr int kArgmaxBlock = 4096;  // vocabulary entries per workgroup of the argmax's first pass
size_t argmax_workspace_bytes(int t, int64_t V);
int launch_argmax(const uint16_t* L, int64_t* out, int t, int64_t V, int64_t ldl, void* ws, hipStream_t stream);

int launch_rmsnorm(const uint16_t* x, const uint16_t* w, float eps, uint16_t* y, int t, int64_t H, int64_t ldx,
                   int64_t ldy, hipStream_t stream);
int launch_swiglu(const uint16_t* gu, uint16_t* y, int t, int64_t F, int64_t ldg, int64_t ldy,
                  hipStream_t stream);
int launch_residual_add(const uint16_t* a, const uint16_t* b, uint16_t* y, int t, int64_t H, int64_t lda,
                        int64_t ldb, int64_t ldy, hipStream_t stream);
int launch_exp32(const float* x, float* y, int64_t n, hipStream_t stream);
int launch_log32(const float* x, float* y, int64_t n, hipStream_t stream);

}  // namespace w8i
