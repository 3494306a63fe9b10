// w8inv_api.hip -- the extern "C" entry points of libw8inv.so: argument
// validation on the host, then launches on the caller's stream.  Nothing
// here allocates, frees or synchronises.  The rules checked are the ones
// stated for each entry point in include/w8inv.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "w8inv.h"
#include "w8inv_internal.h"

using namespace w8i;

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

constexpr int64_t kMaxDim = (int64_t)1 << 40;

// checks shared by the projections: the W8 operands of an [N, K] projection
int check_projection(const int8_t* W_q, const uint16_t* scales, const uint16_t* x, int32_t t, int32_t T_pad,
                     const uint16_t* y, int64_t N, int64_t K, int64_t ldx, int64_t ldy, int64_t y_cols) {
    if (T_pad != 16 && T_pad != 32 && T_pad != 48 && T_pad != 64) return W8I_ET;
    if (t < 0 || t > T_pad) return W8I_ET;
    if (t == 0) return W8I_OK;
    if (!W_q || !scales || !x || !y) return W8I_ENULL;
    if (N < 1 || K < kGroup || K % kGroup != 0 || N > kMaxDim || K > kMaxDim) return W8I_ESHAPE;
    if (N * K >= ((int64_t)1 << 32)) return W8I_ESHAPE;
    if (ldx < K || ldy < y_cols || ldx > ((int64_t)1 << 24)) return W8I_ESHAPE;
    if (!aligned(W_q, 16) || !aligned(x, 16) || ldx % 8 != 0 || !aligned(scales, 2) || !aligned(y, 2))
        return W8I_EALIGN;
    if ((N + 31) / 32 > 0x7fffffffLL) return W8I_ESHAPE;
    return W8I_OK;
}

}  // namespace

extern "C" {

const char* w8i_status_string(int status) {
    switch (status) {
        case W8I_OK: return "W8I_OK";
        case W8I_ENULL: return "W8I_ENULL: a required pointer is NULL";
        case W8I_ESHAPE: return "W8I_ESHAPE: a size or leading dimension is out of range";
        case W8I_EALIGN: return "W8I_EALIGN: a pointer or leading dimension breaks an alignment rule";
        case W8I_ET: return "W8I_ET: t < 0, t > T_pad, or T_pad not supported";
        case W8I_EBLOCK: return "W8I_EBLOCK: block width not a power of two in [256, 32768]";
        case W8I_EWORKSPACE: return "W8I_EWORKSPACE: workspace NULL or too small";
        case W8I_EHIP: return "W8I_EHIP: the HIP runtime reported an error";
        case W8I_ESCRATCH: return "W8I_ESCRATCH: the call needs more than the library's fixed scratch";
        default: return "unknown w8i status";
    }
}

const char* w8i_version(void) { return "w8inv 0.1 (gfx950)"; }

size_t w8_linear_invariant_workspace_bytes(int64_t N, int64_t K, int32_t T_pad) {
    if (N < 1 || K < kGroup || K % kGroup != 0 || N > kMaxDim || K > kMaxDim) return 0;
    if (T_pad != 16 && T_pad != 32 && T_pad != 48 && T_pad != 64) return 0;
    return kslice_workspace_bytes(N, T_pad);
}

int w8_linear_invariant(const int8_t* W_q, const uint16_t* scales, const uint16_t* x, int32_t t, int32_t T_pad,
                        uint16_t* y, int64_t N, int64_t K, int64_t ldx, int64_t ldy, void* workspace,
                        size_t workspace_bytes, void* stream) {
    const int st = check_projection(W_q, scales, x, t, T_pad, y, N, K, ldx, ldy, N);
    if (st != W8I_OK || t == 0) return st;
    if (workspace && !aligned(workspace, 8)) return W8I_EALIGN;
    return launch_linear(W_q, scales, x, t, T_pad, y, N, K, ldx, ldy, as_stream(stream), workspace,
                         workspace_bytes);
}

const char* w8_linear_invariant_kernel(int64_t N, int64_t K, int32_t T_pad, const uint16_t* scales) {
    if (N < 1 || K < kGroup || K % kGroup != 0 || N > kMaxDim || K > kMaxDim) return "";
    return linear_kernel_name(N, K, T_pad, scales);
}

int w8_pack_bytes(int64_t N, int64_t K, size_t* wp_bytes, size_t* sp_bytes) {
    if (!wp_bytes || !sp_bytes) return W8I_ENULL;
    if (N < 1 || K < kGroup || K % kGroup != 0 || N > kMaxDim || K > kMaxDim) return W8I_ESHAPE;
    if (packed_weight_bytes(N, K) >= ((int64_t)1 << 32)) return W8I_ESHAPE;
    *wp_bytes = (size_t)packed_weight_bytes(N, K);
    *sp_bytes = (size_t)packed_scale_bytes(N, K);
    return W8I_OK;
}

int w8_pack(const int8_t* W_q, const uint16_t* scales, int64_t N, int64_t K, int8_t* Wp, uint16_t* Sp, void* stream) {
    if (!W_q || !scales || !Wp || !Sp) return W8I_ENULL;
    if (N < 1 || K < kGroup || K % kGroup != 0 || N > kMaxDim || K > kMaxDim) return W8I_ESHAPE;
    if (packed_weight_bytes(N, K) >= ((int64_t)1 << 32)) return W8I_ESHAPE;
    if (!aligned(W_q, 16) || !aligned(scales, 2) || !aligned(Wp, 16) || !aligned(Sp, 16)) return W8I_EALIGN;
    return launch_pack(W_q, scales, N, K, Wp, Sp, as_stream(stream));
}

size_t w8_linear_invariant_packed_workspace_bytes(int64_t N, int64_t K, int32_t T_pad) {
    return w8_linear_invariant_workspace_bytes(N, K, T_pad);
}

int w8_linear_invariant_packed(const int8_t* Wp, const uint16_t* Sp, const uint16_t* x, int32_t t, int32_t T_pad,
                               uint16_t* y, int64_t N, int64_t K, int64_t ldx, int64_t ldy, void* workspace,
                               size_t workspace_bytes, void* stream) {
    const int st = check_projection(Wp, Sp, x, t, T_pad, y, N, K, ldx, ldy, N);
    if (st != W8I_OK || t == 0) return st;
    if (packed_weight_bytes(N, K) >= ((int64_t)1 << 32)) return W8I_ESHAPE;
    if (!aligned(Sp, 16)) return W8I_EALIGN;
    if (workspace && !aligned(workspace, 8)) return W8I_EALIGN;
    return launch_linear_packed(Wp, Sp, x, t, T_pad, y, N, K, ldx, ldy, as_stream(stream), workspace,
                                workspace_bytes);
}

const char* w8_linear_invariant_packed_kernel(int64_t N, int64_t K, int32_t T_pad) {
    if (N < 1 || K < kGroup || K % kGroup != 0 || N > kMaxDim || K > kMaxDim) return "";
    return linear_packed_kernel_name(N, K, T_pad);
}

// y is the residual itself (same pointer and stride), or the two do not overlap
static bool residual_ok(const uint16_t* residual, const uint16_t* y, int32_t t, int64_t N, int64_t ldr, int64_t ldy) {
    const uintptr_t r0 = reinterpret_cast<uintptr_t>(residual), y0 = reinterpret_cast<uintptr_t>(y);
    const uintptr_t r1 = r0 + (uintptr_t)(((int64_t)(t - 1) * ldr + N) * 2);
    const uintptr_t y1 = y0 + (uintptr_t)(((int64_t)(t - 1) * ldy + N) * 2);
    return (r0 == y0 && ldr == ldy) || r1 <= y0 || y1 <= r0;
}

static int linear_add(bool packed, const int8_t* W, const uint16_t* S, const uint16_t* x, const uint16_t* residual,
                      int32_t t, int32_t T_pad, uint16_t* y, int64_t N, int64_t K, int64_t ldx, int64_t ldr,
                      int64_t ldy, void* stream) {
    const int st = check_projection(W, S, x, t, T_pad, y, N, K, ldx, ldy, N);
    if (st != W8I_OK || t == 0) return st;
    if (!residual) return W8I_ENULL;
    if (ldr < N) return W8I_ESHAPE;
    if (!aligned(residual, 2)) return W8I_EALIGN;
    if (!residual_ok(residual, y, t, N, ldr, ldy)) return W8I_ESHAPE;
    if (packed && packed_weight_bytes(N, K) >= ((int64_t)1 << 32)) return W8I_ESHAPE;
    if (packed && !aligned(S, 16)) return W8I_EALIGN;
    return launch_linear_epilogue(kEpiAdd, packed, W, S, x, t, T_pad, y, N, K, ldx, ldy,
                                  LinearEpilogue{residual, ldr, 0}, as_stream(stream));
}

static int linear_swiglu(bool packed, const int8_t* W, const uint16_t* S, const uint16_t* x, int32_t t,
                         int32_t T_pad, uint16_t* y, int64_t F, int64_t K, int64_t ldx, int64_t ldy, void* stream) {
    if (T_pad != 16 && T_pad != 32 && T_pad != 48 && T_pad != 64) return W8I_ET;
    if (t < 0 || t > T_pad) return W8I_ET;
    if (t == 0) return W8I_OK;
    if (F < 1 || F > kMaxDim) return W8I_ESHAPE;
    const int st = check_projection(W, S, x, t, T_pad, y, 2 * F, K, ldx, ldy, F);
    if (st != W8I_OK) return st;
    if (packed && packed_weight_bytes(2 * F, K) >= ((int64_t)1 << 32)) return W8I_ESHAPE;
    if (packed && !aligned(S, 16)) return W8I_EALIGN;
    return launch_linear_epilogue(kEpiSwiGLU, packed, W, S, x, t, T_pad, y, 2 * F, K, ldx, ldy,
                                  LinearEpilogue{nullptr, 0, F}, as_stream(stream));
}

int w8_linear_add_invariant(const int8_t* W_q, const uint16_t* scales, const uint16_t* x, const uint16_t* residual,
                            int32_t t, int32_t T_pad, uint16_t* y, int64_t N, int64_t K, int64_t ldx, int64_t ldr,
                            int64_t ldy, void* stream) {
    return linear_add(false, W_q, scales, x, residual, t, T_pad, y, N, K, ldx, ldr, ldy, stream);
}

int w8_linear_add_invariant_packed(const int8_t* Wp, const uint16_t* Sp, const uint16_t* x, const uint16_t* residual,
                                   int32_t t, int32_t T_pad, uint16_t* y, int64_t N, int64_t K, int64_t ldx,
                                   int64_t ldr, int64_t ldy, void* stream) {
    return linear_add(true, Wp, Sp, x, residual, t, T_pad, y, N, K, ldx, ldr, ldy, stream);
}

int w8_linear_swiglu_invariant(const int8_t* W_q, const uint16_t* scales, const uint16_t* x, int32_t t,
                               int32_t T_pad, uint16_t* y, int64_t F, int64_t K, int64_t ldx, int64_t ldy,
                               void* stream) {
    return linear_swiglu(false, W_q, scales, x, t, T_pad, y, F, K, ldx, ldy, stream);
}

int w8_linear_swiglu_invariant_packed(const int8_t* Wp, const uint16_t* Sp, const uint16_t* x, int32_t t,
                                      int32_t T_pad, uint16_t* y, int64_t F, int64_t K, int64_t ldx, int64_t ldy,
                                      void* stream) {
    return linear_swiglu(true, Wp, Sp, x, t, T_pad, y, F, K, ldx, ldy, stream);
}

static int linear_pair(bool packed, const int8_t* Wa, const uint16_t* Sa, const int8_t* Wb, const uint16_t* Sb,
                       const uint16_t* x, int32_t t, int32_t T_pad, uint16_t* ya, uint16_t* yb, int64_t Na, int64_t Nb,
                       int64_t K, int64_t ldx, int64_t ldya, int64_t ldyb, void* stream) {
    int st = check_projection(Wa, Sa, x, t, T_pad, ya, Na, K, ldx, ldya, Na);
    if (st != W8I_OK || t == 0) return st;
    st = check_projection(Wb, Sb, x, t, T_pad, yb, Nb, K, ldx, ldyb, Nb);
    if (st != W8I_OK) return st;
    if (packed && (packed_weight_bytes(Na, K) >= ((int64_t)1 << 32) || packed_weight_bytes(Nb, K) >= ((int64_t)1 << 32)))
        return W8I_ESHAPE;
    if (packed && (!aligned(Sa, 16) || !aligned(Sb, 16))) return W8I_EALIGN;
    LinearEpilogue ep;
    ep.W2 = Wb;
    ep.S2 = Sb;
    ep.Y2 = yb;
    ep.N2 = Nb;
    ep.ldy2 = ldyb;
    return launch_linear_pair(packed, Wa, Sa, x, t, T_pad, ya, Na, K, ldx, ldya, ep, as_stream(stream));
}

int w8_linear_pair_invariant(const int8_t* Wa, const uint16_t* Sa, const int8_t* Wb, const uint16_t* Sb,
                             const uint16_t* x, int32_t t, int32_t T_pad, uint16_t* ya, uint16_t* yb, int64_t Na,
                             int64_t Nb, int64_t K, int64_t ldx, int64_t ldya, int64_t ldyb, void* stream) {
    return linear_pair(false, Wa, Sa, Wb, Sb, x, t, T_pad, ya, yb, Na, Nb, K, ldx, ldya, ldyb, stream);
}

int w8_linear_pair_invariant_packed(const int8_t* Wpa, const uint16_t* Spa, const int8_t* Wpb, const uint16_t* Spb,
                                    const uint16_t* x, int32_t t, int32_t T_pad, uint16_t* ya, uint16_t* yb,
                                    int64_t Na, int64_t Nb, int64_t K, int64_t ldx, int64_t ldya, int64_t ldyb,
                                    void* stream) {
    return linear_pair(true, Wpa, Spa, Wpb, Spb, x, t, T_pad, ya, yb, Na, Nb, K, ldx, ldya, ldyb, stream);
}

// the normalised activations of attn_input_proj: bf16 [t, round_up(H, 8)], 16-byte aligned rows
static int64_t attn_norm_ld(int64_t H) { return (H + 7) / 8 * 8; }

size_t w8_attn_input_proj_workspace_bytes(int32_t t, int64_t H) {
    if (t <= 0 || H < 1 || H > 65536) return 0;
    return (size_t)(((int64_t)t * attn_norm_ld(H) * 2 + 255) / 256 * 256);
}

static int attn_input_proj(bool packed, const uint16_t* h, const uint16_t* norm_weight, float eps,
                           const int8_t* W, const uint16_t* S, int32_t t, int32_t T_pad, uint16_t* y, int64_t N,
                           int64_t H, int64_t ldh, int64_t ldy, void* workspace, size_t workspace_bytes,
                           void* stream) {
    if (T_pad != 16 && T_pad != 32 && T_pad != 48 && T_pad != 64) return W8I_ET;
    if (t < 0 || t > T_pad) return W8I_ET;
    if (t == 0) return W8I_OK;
    if (!h) return W8I_ENULL;
    if (H < 1 || H > 65536 || ldh < H) return W8I_ESHAPE;
    if (!aligned(h, 2) || (norm_weight && !aligned(norm_weight, 2))) return W8I_EALIGN;
    if (!workspace || workspace_bytes < w8_attn_input_proj_workspace_bytes(t, H)) return W8I_EWORKSPACE;
    if (!aligned(workspace, 16)) return W8I_EALIGN;
    uint16_t* xn = static_cast<uint16_t*>(workspace);
    const int64_t ldn = attn_norm_ld(H);
    int st = check_projection(W, S, xn, t, T_pad, y, N, H, ldn, ldy, N);
    if (st != W8I_OK) return st;
    if (packed && packed_weight_bytes(N, H) >= ((int64_t)1 << 32)) return W8I_ESHAPE;
    if (packed && !aligned(S, 16)) return W8I_EALIGN;
    st = launch_rmsnorm(h, norm_weight, eps, xn, t, H, ldh, ldn, as_stream(stream));
    if (st != W8I_OK) return st;
    return packed ? launch_linear_packed(W, S, xn, t, T_pad, y, N, H, ldn, ldy, as_stream(stream))
                  : launch_linear(W, S, xn, t, T_pad, y, N, H, ldn, ldy, as_stream(stream));
}

int w8_attn_input_proj_invariant(const uint16_t* h, const uint16_t* norm_weight, float eps, const int8_t* W_q,
                                 const uint16_t* scales, int32_t t, int32_t T_pad, uint16_t* y, int64_t N, int64_t H,
                                 int64_t ldh, int64_t ldy, void* workspace, size_t workspace_bytes, void* stream) {
    return attn_input_proj(false, h, norm_weight, eps, W_q, scales, t, T_pad, y, N, H, ldh, ldy, workspace,
                           workspace_bytes, stream);
}

int w8_attn_input_proj_invariant_packed(const uint16_t* h, const uint16_t* norm_weight, float eps, const int8_t* Wp,
                                        const uint16_t* Sp, int32_t t, int32_t T_pad, uint16_t* y, int64_t N,
                                        int64_t H, int64_t ldh, int64_t ldy, void* workspace, size_t workspace_bytes,
                                        void* stream) {
    return attn_input_proj(true, h, norm_weight, eps, Wp, Sp, t, T_pad, y, N, H, ldh, ldy, workspace,
                           workspace_bytes, stream);
}

size_t vocab_block_logprob_workspace_bytes(int32_t t, int64_t V, int32_t block) {
    if (t <= 0 || V <= 0 || block < 256 || block > 32768 || (block & (block - 1)) != 0) return 0;
    return logprob_workspace_bytes(t, V, block);
}

// checks shared by the logprob entry points (all but the workspace)
static int check_logprob(const uint16_t* logits, const int64_t* targets, int32_t block, const float* out, int32_t t,
                         int64_t V, int64_t ldl) {
    if (block < 256 || block > 32768 || (block & (block - 1)) != 0) return W8I_EBLOCK;
    if (t < 0 || t > 65535) return W8I_ET;
    if (t == 0) return W8I_OK;
    if (!logits || !targets || !out) return W8I_ENULL;
    if (V < 1 || V > kMaxDim || ldl < V) return W8I_ESHAPE;
    if ((V + block - 1) / block > 0x7fffffffLL) return W8I_ESHAPE;
    if (!aligned(logits, 2) || !aligned(targets, 8) || !aligned(out, 4)) return W8I_EALIGN;
    return W8I_OK;
}

static int block_logprob(const uint16_t* logits, const int64_t* targets, int32_t block, float* out, int32_t t,
                         int64_t V, int64_t ldl, void* workspace, size_t workspace_bytes, bool direct, void* stream) {
    const int st = check_logprob(logits, targets, block, out, t, V, ldl);
    if (st != W8I_OK || t == 0) return st;
    if (!workspace || workspace_bytes < logprob_workspace_bytes(t, V, block)) return W8I_EWORKSPACE;
    if (!aligned(workspace, 16)) return W8I_EALIGN;
    return launch_logprob(logits, targets, block, out, t, V, ldl, workspace, direct, as_stream(stream));
}

int vocab_block_logprob(const uint16_t* logits, const int64_t* targets, int32_t block, float* out, int32_t t,
                        int64_t V, int64_t ldl, void* workspace, size_t workspace_bytes, void* stream) {
    return block_logprob(logits, targets, block, out, t, V, ldl, workspace, workspace_bytes, false, stream);
}

int vocab_block_logprob_direct(const uint16_t* logits, const int64_t* targets, int32_t block, float* out, int32_t t,
                               int64_t V, int64_t ldl, void* workspace, size_t workspace_bytes, void* stream) {
    return block_logprob(logits, targets, block, out, t, V, ldl, workspace, workspace_bytes, true, stream);
}

size_t w8_head_logprob_workspace_bytes(int32_t t, int64_t V, int32_t block) {
    if (t <= 0 || V <= 0 || V > kMaxDim || block < 256 || block > 32768 || (block & (block - 1)) != 0) return 0;
    return logprob_from_max_workspace_bytes(t, V, block, tiles_of(V));
}

static int head_logprob(bool packed, const int8_t* W, const uint16_t* S, const uint16_t* x, const int64_t* targets,
                        int32_t t, int32_t T_pad, int32_t block, uint16_t* logits, float* out, int64_t V, int64_t K,
                        int64_t ldx, int64_t ldl, void* workspace, size_t workspace_bytes, void* stream) {
    int st = check_projection(W, S, x, t, T_pad, logits, V, K, ldx, ldl, V);
    if (st != W8I_OK || t == 0) return st;
    if (T_pad > 32 && t > 32) return W8I_ET;
    if (packed && packed_weight_bytes(V, K) >= ((int64_t)1 << 32)) return W8I_ESHAPE;
    if (packed && !aligned(S, 16)) return W8I_EALIGN;
    st = check_logprob(logits, targets, block, out, t, V, ldl);
    if (st != W8I_OK) return st;
    if (!workspace || workspace_bytes < w8_head_logprob_workspace_bytes(t, V, block)) return W8I_EWORKSPACE;
    if (!aligned(workspace, 16)) return W8I_EALIGN;
    int nm = 0;  // column maxima per row the projection writes (one per workgroup), at most tiles_of(V)
    st = launch_linear_max(packed, W, S, x, t, T_pad, logits, V, K, ldx, ldl, static_cast<float*>(workspace), &nm,
                           as_stream(stream));
    if (st != W8I_OK) return st;
    return launch_logprob_from_max(logits, targets, block, out, t, V, ldl, workspace, nm, as_stream(stream));
}

int w8_head_logprob_invariant(const int8_t* W_q, const uint16_t* scales, const uint16_t* x, const int64_t* targets,
                              int32_t t, int32_t T_pad, int32_t block, uint16_t* logits, float* out, int64_t V,
                              int64_t K, int64_t ldx, int64_t ldl, void* workspace, size_t workspace_bytes,
                              void* stream) {
    return head_logprob(false, W_q, scales, x, targets, t, T_pad, block, logits, out, V, K, ldx, ldl, workspace,
                        workspace_bytes, stream);
}

int w8_head_logprob_invariant_packed(const int8_t* Wp, const uint16_t* Sp, const uint16_t* x, const int64_t* targets,
                                     int32_t t, int32_t T_pad, int32_t block, uint16_t* logits, float* out, int64_t V,
                                     int64_t K, int64_t ldx, int64_t ldl, void* workspace, size_t workspace_bytes,
                                     void* stream) {
    return head_logprob(true, Wp, Sp, x, targets, t, T_pad, block, logits, out, V, K, ldx, ldl, workspace,
                        workspace_bytes, stream);
}

int vocab_block_logprob_noalloc(const uint16_t* logits, const int64_t* targets, int32_t block, float* out, int32_t t,
                                int64_t V, int64_t ldl, void* stream) {
    const int st = check_logprob(logits, targets, block, out, t, V, ldl);
    if (st != W8I_OK || t == 0) return st;
    if (logprob_workspace_bytes(t, V, block) > W8I_NOALLOC_SCRATCH_BYTES) return W8I_ESCRATCH;
    void* ws = nullptr;
    const int sst = noalloc_scratch(&ws);
    if (sst != W8I_OK) return sst;
    return launch_logprob(logits, targets, block, out, t, V, ldl, ws, false, as_stream(stream));
}

size_t vocab_argmax_workspace_bytes(int32_t t, int64_t V) {
    if (t <= 0 || V <= 0 || V > ((int64_t)1 << 31)) return 0;
    return argmax_workspace_bytes(t, V);
}

int vocab_argmax(const uint16_t* logits, int64_t* out, int32_t t, int64_t V, int64_t ldl, void* workspace,
                 size_t workspace_bytes, void* stream) {
    if (t < 0 || t > 65535) return W8I_ET;
    if (t == 0) return W8I_OK;
    if (!logits || !out) return W8I_ENULL;
    if (V < 1 || V > ((int64_t)1 << 31) || ldl < V || ldl > kMaxDim) return W8I_ESHAPE;
    if (!aligned(logits, 2) || !aligned(out, 8)) return W8I_EALIGN;
    if (!workspace || workspace_bytes < argmax_workspace_bytes(t, V)) return W8I_EWORKSPACE;
    if (!aligned(workspace, 8)) return W8I_EALIGN;
    return launch_argmax(logits, out, t, V, ldl, workspace, as_stream(stream));
}

int w8i_rmsnorm(const uint16_t* x, const uint16_t* weight, float eps, uint16_t* y, int32_t t, int64_t H, int64_t ldx,
                int64_t ldy, void* stream) {
    if (t < 0 || t > 0x7fffffff) return W8I_ET;
    if (t == 0) return W8I_OK;
    if (!x || !y) return W8I_ENULL;
    if (H < 1 || H > 65536 || ldx < H || ldy < H) return W8I_ESHAPE;
    if (!aligned(x, 2) || !aligned(y, 2) || (weight && !aligned(weight, 2))) return W8I_EALIGN;
    return launch_rmsnorm(x, weight, eps, y, t, H, ldx, ldy, as_stream(stream));
}

int w8i_swiglu(const uint16_t* gate_up, uint16_t* y, int32_t t, int64_t F, int64_t ldg, int64_t ldy, void* stream) {
    if (t < 0 || t > 65535) return W8I_ET;
    if (t == 0) return W8I_OK;
    if (!gate_up || !y) return W8I_ENULL;
    if (F < 1 || F > kMaxDim || ldg < 2 * F || ldy < F) return W8I_ESHAPE;
    if (!aligned(gate_up, 2) || !aligned(y, 2)) return W8I_EALIGN;
    return launch_swiglu(gate_up, y, t, F, ldg, ldy, as_stream(stream));
}

int w8i_residual_add(const uint16_t* a, const uint16_t* b, uint16_t* y, int32_t t, int64_t H, int64_t lda,
                     int64_t ldb, int64_t ldy, void* stream) {
    if (t < 0 || t > 65535) return W8I_ET;
    if (t == 0) return W8I_OK;
    if (!a || !b || !y) return W8I_ENULL;
    if (H < 1 || H > kMaxDim || lda < H || ldb < H || ldy < H) return W8I_ESHAPE;
    if (!aligned(a, 2) || !aligned(b, 2) || !aligned(y, 2)) return W8I_EALIGN;
    return launch_residual_add(a, b, y, t, H, lda, ldb, ldy, as_stream(stream));
}

int w8i_exp32(const float* x, float* y, int64_t n, void* stream) {
    if (n < 0) return W8I_ESHAPE;
    if (n == 0) return W8I_OK;
    if (!x || !y) return W8I_ENULL;
    if (!aligned(x, 4) || !aligned(y, 4)) return W8I_EALIGN;
    if (n > ((int64_t)1 << 38)) return W8I_ESHAPE;
    return launch_exp32(x, y, n, as_stream(stream));
}

int w8i_log32(const float* x, float* y, int64_t n, void* stream) {
    if (n < 0) return W8I_ESHAPE;
    if (n == 0) return W8I_OK;
    if (!x || !y) return W8I_ENULL;
    if (!aligned(x, 4) || !aligned(y, 4)) return W8I_EALIGN;
    if (n > ((int64_t)1 << 38)) return W8I_ESHAPE;
    return launch_log32(x, y, n, as_stream(stream));
}

}  // extern "C"
