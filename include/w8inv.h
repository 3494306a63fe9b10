/*
 * w8inv.h -- C ABI of the batch-invariant W8A16 decode projection library
 * (libw8inv.so, hand-written HIP for gfx950 / MI355X).
 *
 * Conventions for every entry point below
 *  - All data pointers are DEVICE memory owned by the caller (for example
 *    the storage of torch tensors).  The library never allocates, frees or
 *    keeps a pointer after the call returns.
 *  - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL is the
 *    null stream), which must belong to the calling thread's current device,
 *    as the pointers must.  Nothing synchronises: the return value is the
 *    result of host-side argument validation and of the launch itself, not
 *    of the kernels' execution.
 *  - bf16 and fp16 values are passed as their 16-bit patterns (uint16_t).
 *  - A call with t == 0 (or n == 0) validates nothing else, launches nothing
 *    and returns W8I_OK.
 *  - Invalid arguments return a negative w8i_status and launch nothing.  No
 *    input is ever silently replaced by another computation.
 *  - The library has no runtime switches: for given arguments the
 *    arithmetic, and therefore every output bit, is fixed.  Its only state is
 *    the fixed device scratch array of the entry point that allocates nothing
 *    (vocab_block_logprob_noalloc, at the end of this header).
 */
#ifndef W8INV_H
#define W8INV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    W8I_OK = 0,
    W8I_ENULL = -1,      /* a required pointer is NULL                               */
    W8I_ESHAPE = -2,     /* a size or leading dimension is out of range              */
    W8I_EALIGN = -3,     /* a pointer or leading dimension breaks an alignment rule  */
    W8I_ET = -4,         /* t < 0, t > T_pad, or T_pad not supported                 */
    W8I_EBLOCK = -5,     /* vocabulary block width not a power of two in [256,32768] */
    W8I_EWORKSPACE = -6, /* workspace NULL or smaller than the size query returns    */
    W8I_EHIP = -7,       /* the HIP runtime reported an error when launching         */
    W8I_ESCRATCH = -8    /* the call needs more than the library's fixed scratch     */
} w8i_status;

/* Human-readable name of a status code (static storage). */
const char *w8i_status_string(int status);

/* Library version string (static storage). */
const char *w8i_version(void);

/* ---------------------------------------------------------------------------
 * W8A16 linear at a fixed decode width.
 *
 * Source: the ninfer issue on t-dependent kernel dispatch (GitHub issue 80),
 * table "Where t selects arithmetic" row "ops::linear W8G32" (int8 weights,
 * one scale per 32 consecutive K elements, 16-bit activations) and the
 * "Proposal: opt-in fixed decode width" section: one reduction schedule, set
 * by the padded width T_pad, serves every real t; padding columns are never
 * read from the caller nor stored, and no output column's arithmetic involves
 * another column, so column j's bits depend neither on t, on j's neighbours
 * nor on the order of the columns.
 *
 *   y[j, n] = bf16_rne( sum_k  q[n, k] * s[n, k / 32] * x[j, k] )   j < t, n < N
 *
 *   W_q    int8  [N, K] row-major, codes in [-127, 127] (-128 is accepted);
 *          16-byte aligned.
 *   scales fp16  [N, K/32] row-major (one scale per row and 32 consecutive k);
 *          2-byte aligned.  Subnormal and zero scales are used exactly.
 *   x      bf16  [t, ldx] row-major: token j's K features are contiguous;
 *          16-byte aligned, ldx >= K, ldx % 8 == 0.
 *   y      bf16  [t, ldy] row-major: token j's N outputs are contiguous;
 *          2-byte aligned, ldy >= N.  Only y[j, n] with j < t, n < N is written.
 *          y must not overlap W_q, scales or x: other workgroups still read
 *          them while y is written (not checked).
 *   t      real columns, 0 <= t <= T_pad.
 *   T_pad  fixed decode width: 16, 32, 48 or 64.  The kernel computes all
 *          T_pad columns (the first ones real, the rest zero) for every t.
 *   N      output rows, N >= 1 (any N: the last row strip is masked).
 *   K      reduction length, K >= 32 and K % 32 == 0; N * K < 2^32
 *          (4 GiB of codes per call) and ldx <= 2^24.
 *
 * Arithmetic, fixed for every (t, T_pad, N, device):
 *   - int8 codes become bf16 exactly; each 32-element group's products are
 *     summed by bf16 matrix-core instructions into fp32 starting from zero;
 *   - that group sum is multiplied by its fp16 scale and accumulated in fp64;
 *   - K is cut into 8 contiguous slices of whole pairs of groups, slices
 *     0..3 three times as long as slices 4..7: with G = K/32 groups, P =
 *     floor(G/2) pairs and c = (0, 3, 6, 9, 12, 13, 14, 15, 16), slice i covers
 *     groups [2*floor(P*c_i/16), 2*floor(P*c_{i+1}/16)) and, when G is odd, slice 7
 *     also takes the last group.  Each slice is summed in ascending group order
 *     (an empty slice is +0) and the 8 slice sums are combined by the left
 *     fold ((((((s0+s1)+s2)+s3)+s4)+s5)+s6)+s7.  The plan depends on K only;
 *   - the fp64 result is rounded once to bf16, nearest-even.
 *   No atomics, no autotuning, no arithmetic of a live column chosen from t.
 *   t only sets how much padding work is skipped: activation loads whose 8
 *   columns are all padding are not issued (their LDS regions hold zeros),
 *   and the products of such padding columns are not formed (a 32-column
 *   tile with no live column skips its matrix-core steps); at T_pad 48 or 64
 *   a call with t <= 32 runs the one-tile kernel of T_pad 32, the second tile
 *   being padding only.  Every live column's MFMAs, fp64 sums and rounding are
 *   the same for every t and every T_pad.
 *
 * workspace (optional, never required; caller-owned device memory, 8-byte
 * aligned, not overlapping the other buffers): the size query returns 0 where
 * the call cannot use one, and for small N (at most 2048 rows, run at T_pad 16
 * or 32) the bytes of 8 fp64 slice sums per output, 8 * min(T_pad, 32) * N *
 * 8.  Given a workspace of at least 8 * t * N * 8 bytes such a call runs the 8
 * K-slices of each 32-row strip on separate workgroups (gemm_w8g32_kslice),
 * parks each slice sum in the workspace and folds them in a second launch
 * (kslice_fold): the same slices, MFMAs, fp64 operations in the same order,
 * left fold and rounding, so the same bits as the one-launch kernel, which
 * runs when workspace is NULL or smaller.  The workspace's contents on return
 * are unspecified.  W8I_EALIGN if a non-NULL workspace is not 8-byte aligned.
 * ------------------------------------------------------------------------- */
size_t w8_linear_invariant_workspace_bytes(int64_t N, int64_t K, int32_t T_pad);

int w8_linear_invariant(const int8_t *W_q, const uint16_t *scales, const uint16_t *x,
                        int32_t t, int32_t T_pad, uint16_t *y,
                        int64_t N, int64_t K, int64_t ldx, int64_t ldy,
                        void *workspace, size_t workspace_bytes, void *stream);

/* Name of the kernel that w8_linear_invariant runs for these arguments (static
 * storage; "" for arguments it would reject), for matching profiler records.
 * The choice depends on N, K, T_pad and on whether `scales` is 16-byte
 * aligned, and every kernel runs the K plan above, so it changes no bit of the
 * result.  t enters only at T_pad 48 or 64: a call with t <= 32 runs the kernel
 * this query names for T_pad 32.  The name is that of the one-launch kernel; a
 * call given the optional workspace (below) runs gemm_w8g32_kslice and
 * kslice_fold instead.  Pure host function: no device access. */
const char *w8_linear_invariant_kernel(int64_t N, int64_t K, int32_t T_pad, const uint16_t *scales);

/* ---------------------------------------------------------------------------
 * Packed weight layout (optional).
 *
 * The same W8G32 projection over weights rearranged once, at load time, into
 * the order the projection kernel streams them: per 32-row strip and pair of
 * groups, one 2 KB block of codes already in the matrix-core operand order
 * (whole cache lines per load, no register shuffles) and one 128-byte line of
 * its 64 scales (no staging of scales before the main loop).  Only the layout
 * changes: w8_linear_invariant_packed(w8_pack(W_q, scales), ...) gives the bits
 * of w8_linear_invariant(W_q, scales, ...) for every argument, with the same K
 * plan.  (Source of the operation: as for w8_linear_invariant.)
 *
 * Layout, with G = K/32, P = ceil(G/2) and strips = ceil(N/32):
 *   Wp int8 [strips][P][2048]: byte 1024 gs + 512 c + 16 r + b of block (s, p)
 *      is W_q[32 s + r][64 p + 32 gs + 16 c + b]   (r < 32; gs, c < 2; b < 16)
 *   Sp fp16 [strips][P][64]:   element 2 r + gs of block (s, p) is
 *      scales[32 s + r][2 p + gs]
 *   Rows past N, and the group past an odd G, are zero.
 *
 * w8_pack_bytes: the sizes of Wp and Sp (W8I_ESHAPE when Wp would reach 4 GiB).
 * w8_pack: writes Wp and Sp (device buffers of those sizes, 16-byte aligned)
 *   from W_q (16-byte aligned) and scales (2-byte aligned) on `stream`; no
 *   overlap between the inputs and the outputs.
 * w8_linear_invariant_packed: as w8_linear_invariant (x, y, t, T_pad, N, K,
 *   ldx, ldy, workspace and their rules), with Wp / Sp from w8_pack(N, K)
 *   (16-byte aligned).  Any N: the persistent kernel where the plain layout
 *   runs it (T_pad <= 32, N >= 131072), the K-slice kernels for small N given
 *   the workspace, else the LDS-staged split kernel, all with per-stage scale
 *   loads.
 * w8_linear_invariant_packed_workspace_bytes: the workspace size query, equal
 *   to w8_linear_invariant_workspace_bytes for the same (N, K, T_pad).
 * ------------------------------------------------------------------------- */
int w8_pack_bytes(int64_t N, int64_t K, size_t *wp_bytes, size_t *sp_bytes);

int w8_pack(const int8_t *W_q, const uint16_t *scales, int64_t N, int64_t K, int8_t *Wp, uint16_t *Sp,
            void *stream);

size_t w8_linear_invariant_packed_workspace_bytes(int64_t N, int64_t K, int32_t T_pad);

int w8_linear_invariant_packed(const int8_t *Wp, const uint16_t *Sp, const uint16_t *x, int32_t t,
                               int32_t T_pad, uint16_t *y, int64_t N, int64_t K, int64_t ldx, int64_t ldy,
                               void *workspace, size_t workspace_bytes, void *stream);

/* Name of the kernel w8_linear_invariant_packed runs (static storage; "" for
 * arguments it would reject): a function of N and T_pad (at T_pad 48 or 64 a
 * call with t <= 32 runs the kernel named for T_pad 32; given the optional
 * workspace, small N runs the K-slice kernel and its fold instead).  Pure
 * host function. */
const char *w8_linear_invariant_packed_kernel(int64_t N, int64_t K, int32_t T_pad);

/* ---------------------------------------------------------------------------
 * Fused W8 projection epilogues.
 *
 * Source: the ninfer issue (GitHub issue 80), table "Where t selects
 * arithmetic", row "attn_input_proj, linear_swiglu, linear_pair, linear_add
 * (W8)": the fused decode ops run the W8 linear's main loop with an epilogue.
 * Here they run the same K plan as w8_linear_invariant, so every projection
 * output has that call's bits, and the epilogue is the glue call's arithmetic:
 *
 *   w8_linear_add_invariant:    y = w8i_residual_add(w8_linear_invariant(x), residual)
 *   w8_linear_swiglu_invariant: y = w8i_swiglu(w8_linear_invariant(x))
 *
 * bit for bit, with the 34816-wide (say) intermediate never written.  Both
 * always run the LDS-staged split kernel.  Operands, T_pad, t, K, ldx, the
 * alignment rules and the errors are those of w8_linear_invariant; no
 * workspace is needed.
 *
 * w8_linear_add_invariant: W_q [N, K], scales [N, K/32], residual bf16
 *   [t, ldr] (2-byte aligned, ldr >= N), y bf16 [t, ldy].  y may be the
 *   residual itself (same pointer and ldr == ldy: each element is read before
 *   it is written); any other overlap is W8I_ESHAPE.
 * w8_linear_swiglu_invariant: W_q [2F, K], scales [2F, K/32]: rows [0, F) are
 *   the gate projection, rows [F, 2F) the up projection (the layout whose
 *   output w8i_swiglu takes).  y bf16 [t, ldy], ldy >= F:
 *   y[j, h] = silu(gate[j, h]) * up[j, h] as w8i_swiglu computes it from the
 *   two bf16-rounded projection outputs.  2F * K < 2^32.
 * ------------------------------------------------------------------------- */
int w8_linear_add_invariant(const int8_t *W_q, const uint16_t *scales, const uint16_t *x,
                            const uint16_t *residual, int32_t t, int32_t T_pad, uint16_t *y,
                            int64_t N, int64_t K, int64_t ldx, int64_t ldr, int64_t ldy, void *stream);

int w8_linear_swiglu_invariant(const int8_t *W_q, const uint16_t *scales, const uint16_t *x,
                               int32_t t, int32_t T_pad, uint16_t *y, int64_t F, int64_t K,
                               int64_t ldx, int64_t ldy, void *stream);

/* The same two over weights in the packed layout (w8_pack of the [N, K], resp.
 * [2F, K], projection; Wp and Sp 16-byte aligned): the bits of the plain-layout
 * call, as for w8_linear_invariant_packed.  Declared with the packed layout
 * below. */
int w8_linear_add_invariant_packed(const int8_t *Wp, const uint16_t *Sp, const uint16_t *x,
                                   const uint16_t *residual, int32_t t, int32_t T_pad, uint16_t *y,
                                   int64_t N, int64_t K, int64_t ldx, int64_t ldr, int64_t ldy,
                                   void *stream);

int w8_linear_swiglu_invariant_packed(const int8_t *Wp, const uint16_t *Sp, const uint16_t *x,
                                      int32_t t, int32_t T_pad, uint16_t *y, int64_t F, int64_t K,
                                      int64_t ldx, int64_t ldy, void *stream);

/* ---------------------------------------------------------------------------
 * Two projections of one activation batch, and the attention input projection.
 *
 * Source: the ninfer issue (GitHub issue 80), table "Where t selects
 * arithmetic", row "attn_input_proj, linear_swiglu, linear_pair, linear_add
 * (W8)".  The page names these fused decode ops without defining them; the
 * readings here:
 *
 * w8_linear_pair_invariant: two projections of the same activations in one
 *   launch, ya = w8_linear_invariant(Wa, Sa, x) and yb = w8_linear_invariant(Wb,
 *   Sb, x), bit for bit (the launch's workgroups cover the row strips of both;
 *   each output is the single call's computation).  Wa [Na, K], Wb [Nb, K] with
 *   their scales; ya bf16 [t, ldya], yb bf16 [t, ldyb].  The rules and errors of
 *   w8_linear_invariant apply to each projection; ya and yb must not overlap
 *   each other or the inputs (not checked).  Always the LDS-staged split kernel.
 * w8_attn_input_proj_invariant: the attention block's input projection, RMSNorm
 *   of the hidden state followed by its (fused QKV) projection:
 *     y = w8_linear_invariant(W_q, scales, w8i_rmsnorm(h, norm_weight, eps))
 *   bit for bit.  h bf16 [t, ldh] (H features, 1 <= H <= 65536, 2-byte
 *   aligned), norm_weight bf16 [H] or NULL (weight 1), W_q [N, H], y bf16
 *   [t, ldy].  The normalised activations (bf16 [t, H] rows padded to a multiple
 *   of 8) go to `workspace` (16-byte aligned, at least
 *   w8_attn_input_proj_workspace_bytes(t, H) bytes; contents are scratch): one
 *   call, two launches -- the norm's correctly rounded per-element division
 *   runs once per element instead of once per projection workgroup.
 * The _packed forms take weights from w8_pack (16-byte aligned) and give the
 * same bits.
 * ------------------------------------------------------------------------- */
int w8_linear_pair_invariant(const int8_t *Wa, const uint16_t *Sa, const int8_t *Wb, const uint16_t *Sb,
                             const uint16_t *x, int32_t t, int32_t T_pad, uint16_t *ya, uint16_t *yb,
                             int64_t Na, int64_t Nb, int64_t K, int64_t ldx, int64_t ldya, int64_t ldyb,
                             void *stream);

int w8_linear_pair_invariant_packed(const int8_t *Wpa, const uint16_t *Spa, const int8_t *Wpb,
                                    const uint16_t *Spb, const uint16_t *x, int32_t t, int32_t T_pad,
                                    uint16_t *ya, uint16_t *yb, int64_t Na, int64_t Nb, int64_t K,
                                    int64_t ldx, int64_t ldya, int64_t ldyb, void *stream);

size_t w8_attn_input_proj_workspace_bytes(int32_t t, int64_t H);

int w8_attn_input_proj_invariant(const uint16_t *h, const uint16_t *norm_weight, float eps,
                                 const int8_t *W_q, const uint16_t *scales, int32_t t, int32_t T_pad,
                                 uint16_t *y, int64_t N, int64_t H, int64_t ldh, int64_t ldy,
                                 void *workspace, size_t workspace_bytes, void *stream);

int w8_attn_input_proj_invariant_packed(const uint16_t *h, const uint16_t *norm_weight, float eps,
                                        const int8_t *Wp, const uint16_t *Sp, int32_t t, int32_t T_pad,
                                        uint16_t *y, int64_t N, int64_t H, int64_t ldh, int64_t ldy,
                                        void *workspace, size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * Target-token logprob by fixed-width vocabulary blocks (LM-head epilogue).
 *
 * Source: the tokenspeed "Numerics envelopes" page, alignment.trainer table
 * row "--logprob-order blockwise" (row max, shift, target gather, sum_exp over
 * fixed-width vocabulary blocks with each block's own fixed tree, an fp32 left
 * fold across blocks, negative cross-entropy), its "Logprobs" section (bf16
 * logits are widened exactly to fp32 inside the kernel; the negated form
 * gives -0.0 for a certain token) and the block_sumexp leaf contract
 * paragraph (partials in vocabulary order, folded left to right).
 *
 * For each column j < t, with l_v = fp32(logits[j, v]):
 *   m    = max_{v < V} l_v
 *   e_v  = EXP32(l_v - m) for v < V (the subtraction is one fp32 operation),
 *          +0 for the virtual padding V <= v < nb*block, nb = ceil(V/block)
 *   P_b  = balanced pairwise fp32 tree over e_{b*block .. b*block+block-1}
 *          in index order: T(i,1) = e_i, T(i,2w) = T(i,w) + T(i+w,w)
 *   S    = ((P_0 + P_1) + P_2) + ... + P_{nb-1}        (fp32)
 *   out  = -(LOG32(S) - (l_target - m))                (fp32)
 * EXP32 / LOG32 are the correctly rounded fp32 values of e^x and ln x.
 * A NaN logit in the row, or a target outside [0, V), gives out = NaN; a +inf
 * logit gives NaN through the arithmetic (inf - inf).
 *
 *   logits  bf16 [t, ldl] row-major (column j's V logits contiguous);
 *           2-byte aligned, ldl >= V.  (16-byte alignment with ldl % 8 == 0
 *           selects 128-bit loads; the results are identical either way.)
 *   targets int64 [t] token ids.
 *   block   power of two in [256, 32768].
 *   out     fp32 [t].
 *   workspace device buffer of at least vocab_block_logprob_workspace_bytes()
 *           bytes, 16-byte aligned; contents are scratch.
 * ------------------------------------------------------------------------- */
size_t vocab_block_logprob_workspace_bytes(int32_t t, int64_t V, int32_t block);

int vocab_block_logprob(const uint16_t *logits, const int64_t *targets, int32_t block,
                        float *out, int32_t t, int64_t V, int64_t ldl,
                        void *workspace, size_t workspace_bytes, void *stream);

/* The blockwise-direct form (tokenspeed numerics, "Logprobs": target -
 * log(sum_exp) for trainers that need +0.0): the same reduction, the last step
 * out = s_t - LOG32(S) in fp32, so out is +0.0 for a certain token and equals
 * vocab_block_logprob's value wherever that is not zero.  Arguments, workspace
 * and errors as for vocab_block_logprob. */
int vocab_block_logprob_direct(const uint16_t *logits, const int64_t *targets, int32_t block,
                               float *out, int32_t t, int64_t V, int64_t ldl,
                               void *workspace, size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * The LM head fused with the blockwise logprob's row maximum.
 *
 * Source: tokenspeed numerics, "Logprobs" section and the block_sumexp leaf
 * contract paragraph (the row max is taken first, every block partial is then
 * formed from logits shifted by it); the projection as for
 * w8_linear_invariant.  The fixed arithmetic needs the row's global maximum
 * before any block partial, so only that first pass can join the head
 * projection: each of its workgroups writes, with the logits, the column
 * maxima over all the rows it stores (exact in any order), and the logprob's
 * block-partial and fold kernels take the row maximum from those
 * per-workgroup maxima instead of a pass over the logits.
 *
 *   logits = w8_linear_invariant(W_q, scales, x, t, T_pad)        bit for bit
 *   out    = vocab_block_logprob(logits, targets, block)          bit for bit
 *
 * Operands as for the two calls: W_q int8 [V, K] (V output rows = the
 * vocabulary), scales fp16 [V, K/32], x bf16 [t, ldx], logits bf16 [t, ldl]
 * (ldl >= V; written), targets int64 [t], block a power of two in
 * [256, 32768], out fp32 [t].  The projection always runs the persistent
 * kernel (the one w8_linear_invariant runs for N >= 131072 at T_pad <= 32):
 * T_pad 16 or 32, or 48 / 64 with t <= 32 (W8I_ET otherwise).  workspace:
 * 16-byte aligned, at least w8_head_logprob_workspace_bytes(t, V, block)
 * bytes (room for per-workgroup maxima [t, ceil(V/256)] -- one workgroup per
 * CU, at most one per 256-row tile -- and block partials [t, ceil(V/block)]
 * in fp32); contents are scratch.  The _packed form takes w8_pack's layout.
 * ------------------------------------------------------------------------- */
size_t w8_head_logprob_workspace_bytes(int32_t t, int64_t V, int32_t block);

int w8_head_logprob_invariant(const int8_t *W_q, const uint16_t *scales, const uint16_t *x,
                              const int64_t *targets, int32_t t, int32_t T_pad, int32_t block,
                              uint16_t *logits, float *out, int64_t V, int64_t K, int64_t ldx, int64_t ldl,
                              void *workspace, size_t workspace_bytes, void *stream);

int w8_head_logprob_invariant_packed(const int8_t *Wp, const uint16_t *Sp, const uint16_t *x,
                                     const int64_t *targets, int32_t t, int32_t T_pad, int32_t block,
                                     uint16_t *logits, float *out, int64_t V, int64_t K, int64_t ldx,
                                     int64_t ldl, void *workspace, size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * Canonical greedy argmax of each column (LM-head epilogue).
 *
 * Source: tokenspeed numerics, "Logprobs" section: the vocabulary-parallel
 * argmax reduces (maximum, global index) keys with MAX so that ties select the
 * lowest index, with one key for both signed zeros; the ninfer issue's
 * sampling row asks for the canonical lowest-index argmax because exact logit
 * ties happen.  A NaN counts as larger than every number, and the lowest-index
 * NaN wins (the pages are silent; this is what torch and numpy do).
 *
 *   out[j] = the lowest v < V with l_v = max_u l_u (or the lowest NaN index)
 *
 *   logits bf16 [t, ldl] row-major, 2-byte aligned, ldl >= V, 1 <= V <= 2^31
 *          (16-byte rows select 128-bit loads; the result is the same).
 *   out    int64 [t], 8-byte aligned.
 *   workspace device buffer of at least vocab_argmax_workspace_bytes(t, V)
 *          bytes, 8-byte aligned; contents are scratch.
 * Integer keys only: the result is exact and independent of t, of the other
 * columns and of the order of any reduction.
 * ------------------------------------------------------------------------- */
size_t vocab_argmax_workspace_bytes(int32_t t, int64_t V);

int vocab_argmax(const uint16_t *logits, int64_t *out, int32_t t, int64_t V, int64_t ldl,
                 void *workspace, size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * Column-local glue between the projections of one decode layer.  The ninfer
 * issue's "Where t selects arithmetic" notes that norms and other per-lane
 * ops are invariant; these kernels keep every column's arithmetic independent
 * of the other columns.  bf16 in and out, fp32 arithmetic (SwiGLU: fp64), bf16 rounding
 * nearest-even.  Pointers 2-byte aligned.
 *
 * w8i_rmsnorm: y[j,:] = x[j,:] * w / sqrt(mean(x[j,:]^2) + eps), w = weight
 *   (bf16 [H]) or 1 when weight is NULL.  The sum of squares is a balanced
 *   pairwise fp32 tree over the H features zero-padded to a power of two;
 *   then mean = sum / H, d = sqrt(mean + eps), y = (x / d) * w, each one
 *   correctly rounded fp32 operation.  1 <= H <= 65536.
 * w8i_swiglu: y[j,h] = silu(g) * u with g = gate_up[j,h], u = gate_up[j,F+h]:
 *   silu(g) = g / (1 + e^-g), evaluated in fp64 (e^x by the device library's
 *   fp64 exp) and rounded once to bf16; fp32 would overflow e^-g for g < -88.7
 *   where g e^g u can still be a normal bf16.
 * w8i_residual_add: y[j,h] = a[j,h] + b[j,h] in fp32, rounded to bf16
 *   (y may alias a or b).
 * ------------------------------------------------------------------------- */
int w8i_rmsnorm(const uint16_t *x, const uint16_t *weight, float eps, uint16_t *y,
                int32_t t, int64_t H, int64_t ldx, int64_t ldy, void *stream);

int w8i_swiglu(const uint16_t *gate_up, uint16_t *y, int32_t t, int64_t F,
               int64_t ldg, int64_t ldy, void *stream);

int w8i_residual_add(const uint16_t *a, const uint16_t *b, uint16_t *y, int32_t t,
                     int64_t H, int64_t lda, int64_t ldb, int64_t ldy, void *stream);

/* ---------------------------------------------------------------------------
 * Verification hooks: the device EXP32 / LOG32 used above, applied
 * elementwise (y[i] = EXP32(x[i]) or LOG32(x[i]), fp32, 4-byte aligned), so
 * that tests can compare them with the correctly rounded values.
 * ------------------------------------------------------------------------- */
int w8i_exp32(const float *x, float *y, int64_t n, void *stream);
int w8i_log32(const float *x, float *y, int64_t n, void *stream);

/* ---------------------------------------------------------------------------
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the
 * blockwise target logprob with no workspace argument.
 *
 * vocab_block_logprob_noalloc computes exactly what vocab_block_logprob
 * computes (same kernels, same bits) for the same logits, targets, block,
 * out, t, V and ldl, with the same argument rules and errors, but its block
 * maxima and block partials go to a scratch array that the library holds in
 * device memory: a file-scope device array of W8I_NOALLOC_SCRATCH_BYTES
 * bytes, one per GPU the library runs on, kept until the process ends (its
 * address is looked up on the first call on each device; nothing is
 * allocated or freed, by this call or any later one).
 *
 *   - Calls with vocab_block_logprob_workspace_bytes(t, V, block) larger than
 *     W8I_NOALLOC_SCRATCH_BYTES return W8I_ESCRATCH and launch nothing
 *     (1 MiB holds, for example, t = 64 columns of a 248320-entry vocabulary
 *     in blocks of 256, or t = 32 columns of 2^22 entries in blocks of 4096).
 *   - Every call on one GPU uses that GPU's one array, and its contents are
 *     whatever the last call left (every element a call reads is written by
 *     the same call first).  Calls that can overlap in time on one GPU --
 *     issued on different streams without ordering between them, or from
 *     several host threads -- race on the array and give undefined results;
 *     calls ordered on one stream (or by events) are safe.
 * ------------------------------------------------------------------------- */
#define W8I_NOALLOC_SCRATCH_BYTES ((size_t)1 << 20)

int vocab_block_logprob_noalloc(const uint16_t *logits, const int64_t *targets, int32_t block,
                                float *out, int32_t t, int64_t V, int64_t ldl, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* W8INV_H */
