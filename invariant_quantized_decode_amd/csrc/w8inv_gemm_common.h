// w8inv_gemm_common.h -- device helpers shared by the projection kernels
// (w8inv_gemm.hip, w8inv_kslice.hip): operand types, int8 -> bf16 operands,
// the weight-load lane exchange, the activation stage's LDS swizzle, the
// padding-column offset and the explicit vector-memory waits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "w8inv_internal.h"

namespace w8i {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRows = 32;             // output rows per workgroup (MFMA 32x32 tile)

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

// ----------------------------------------------------------------------------
// Weight loads.  A stage is two consecutive groups.  One load instruction
// covers 16 rows x 64 contiguous bytes: lane l of instruction i reads row
// 16 i + (l & 15), group (l >> 4) & 1 of the stage, 16-byte half l >> 5.  The
// matrix-core layout (lane = row + 32 * half) is then restored in registers
// with v_permlane16_swap, which exchanges lane bit 4 with the index of the
// register pair: afterwards register slot 0 / 1 holds group 0 / 1.
// ----------------------------------------------------------------------------

__device__ __forceinline__ void swap16(u32x4& a, u32x4& b) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const auto r = __builtin_amdgcn_permlane16_swap(a[q], b[q], false, false);
        a[q] = r[0];
        b[q] = r[1];
    }
}

#define W8I_LDS(p) ((__attribute__((address_space(3))) void*)(p))

constexpr int kXTileBytes = 32 * 128;  // 32 columns x one stage of bf16
constexpr int kLdsDmaBytes = 1024;     // bytes of one wave-wide 16-byte direct load

// Cache policy of the packed layout's weight and scale loads: nontemporal.
// Every packed byte is read once, by one load of whole lines, so nothing is
// gained by keeping it in L2 (measured 2-7% faster across the decode shapes).
// The plain layout keeps the default policy: each of its weight loads covers
// half of a 128-byte line whose other half the next stage reads, from L2.
constexpr int kStreamOnce = 2;  // the nt bit of the buffer load's cache-policy operand

// Byte offset of 16-byte piece p (0..7) of column a inside a stage: XOR
// swizzle.  The LDS serves a 16-byte read of 16 lanes (256 bytes, 64 banks)
// per pass; 16 consecutive columns reading one piece land in 16 different
// bank groups because the slot is p ^ ((a >> 1) & 7) and a * 128 alternates
// the 128-byte halves.  (With p ^ (a & 7), columns a and a + 8 collided: the
// counters showed half of all LDS cycles as bank conflicts.)  A direct load
// whose lane l fills bytes 16 l .. 16 l + 15 of 8 columns therefore fetches
// piece xs_piece(a, l) of its column a.
__device__ __forceinline__ uint32_t xs_off(int a, int p) { return (uint32_t)(a * 128 + 16 * (p ^ ((a >> 1) & 7))); }
__device__ __forceinline__ uint32_t xs_piece(int a, int lane) { return (uint32_t)((lane & 7) ^ ((a >> 1) & 7)); }

// Of the nv values a lane holds for 32-column tile tt (value v: column
// 32 tt + 8 (v / 4) + 4 (lane / 32) + v % 4, i.e. column group 4 tt + v / 4),
// the leading ones that fall in the first xl groups of 8 columns.
__device__ __forceinline__ constexpr int tile_live_values(int tt, int xl, int nv) {
    return 4 * (xl - 4 * tt) <= 0 ? 0 : 4 * (xl - 4 * tt) < nv ? 4 * (xl - 4 * tt) : nv;
}

// Byte offset given to the activation loads of padding columns (j >= t): past
// the end of any activation buffer (t <= 64 rows of at most 2^24 bf16 is at
// most 2^31 bytes), so the buffer descriptor's range check returns zeros and
// no memory is read; the stage and piece offsets added to it stay below 2^32.
constexpr uint32_t kPadColumnOffset = 0x80000000u;

// Scheduling-barrier mask that lets every instruction class except the vector
// memory ones move across the barrier (ALU, VALU, SALU, MFMA, LDS, transcendental):
// the loads keep the issue order the explicit waits count on.
constexpr int kKeepVmemOrder = 0x078F;

// s_waitcnt that waits until at most N vector-memory operations are pending
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

}  // namespace w8i
