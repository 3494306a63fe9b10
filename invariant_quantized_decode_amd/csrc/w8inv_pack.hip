// w8inv_pack.hip -- the packed weight layout: an [N, K] W8G32 projection
// (int8 codes row-major, fp16 scales [N, K/32]) rearranged once so that the
// projection kernel streams it with whole-cache-line loads already in the
// matrix-core operand order.  A layout change only: every code and scale is
// copied bit for bit, and the projection over the packed layout gives the
// bits of the projection over the original one.
//
// Layout (32-row strip s, pair of groups p = 0 .. ceil(G/2) - 1, G = K/32):
//   codes  block (s, p) = 2048 bytes at ((s * P + p) * 2048):
//            byte 1024 gs + 512 c + 16 r + b = W[32 s + r][64 p + 32 gs + 16 c + b]
//   scales block (s, p) = 128 bytes at ((s * P + p) * 128):
//            fp16 at 4 r + 2 gs = S[32 s + r][2 p + gs]
// for r < 32, gs, c < 2, b < 16; rows past N and the group past an odd G are
// zero.  Lane l = r + 32 c of a 64-lane load then reads bytes 16 l .. 16 l + 15
// of a 1 KB half-block: row r's 16-byte K half c of group gs.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "w8inv_internal.h"

namespace w8i {

// one thread per 16-byte piece of codes: grid (strips * P * 128 / 256)
__global__ __launch_bounds__(256) void pack_codes(const int8_t* __restrict__ W, int8_t* __restrict__ Wp, int64_t N,
                                                  int64_t K, int64_t P, int64_t pieces) {
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (q >= pieces) return;
    const int64_t blk = q >> 7;  // 128 pieces per block
    const int in = (int)(q & 127);
    const int64_t s = blk / P, p = blk % P;
    const int gs = in >> 6, c = (in >> 5) & 1, r = in & 31;
    const int64_t n = 32 * s + r;
    const int64_t k = 64 * p + 32 * gs + 16 * c;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (n < N && k < K) v = *reinterpret_cast<const uint4*>(W + n * K + k);
    *reinterpret_cast<uint4*>(Wp + q * 16) = v;
}

// one thread per (strip, pair, row): its two scales
__global__ __launch_bounds__(256) void pack_scales(const uint16_t* __restrict__ S, uint16_t* __restrict__ Sp,
                                                   int64_t N, int64_t G, int64_t P, int64_t items) {
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (q >= items) return;
    const int64_t blk = q >> 5;
    const int r = (int)(q & 31);
    const int64_t s = blk / P, p = blk % P;
    const int64_t n = 32 * s + r;
    const uint16_t s0 = n < N ? S[n * G + 2 * p] : (uint16_t)0;
    const uint16_t s1 = n < N && 2 * p + 1 < G ? S[n * G + 2 * p + 1] : (uint16_t)0;
    Sp[2 * q] = s0;
    Sp[2 * q + 1] = s1;
}

int launch_pack(const int8_t* W, const uint16_t* S, int64_t N, int64_t K, int8_t* Wp, uint16_t* Sp,
                hipStream_t stream) {
    const int64_t G = K / kGroup, P = (G + 1) / 2, strips = (N + 31) / 32;
    const int64_t pieces = strips * P * 128, items = strips * P * 32;
    hipLaunchKernelGGL(pack_codes, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, stream, W, Wp, N, K, P,
                       pieces);
    hipLaunchKernelGGL(pack_scales, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, stream, S, Sp, N, G, P,
                       items);
    return hipGetLastError() == hipSuccess ? W8I_OK : W8I_EHIP;
}

}  // namespace w8i
