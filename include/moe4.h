/*
 * moe4.h -- C interface of libmoe4: the routed mixture-of-experts expert layer
 * computed directly on 4-bit expert stacks, with hand-written HIP kernels for
 * AMD Instinct MI355X (gfx950).
 *
 * Sources, cited by page title and section:
 *  - "How do I train and serve MoE models released in MXFP4 (gpt-oss,
 *    DeepSeek-V4)?" -- "Why it happens" (MXFP4 = two e2m1 nibbles per byte, 32
 *    values per e8m0 power-of-two scale; gpt-oss per-expert biases, interleaved
 *    gate/up rows, clamped GLU), "Two fidelity paths" (bit-exact MXFP4 decode;
 *    NF4 re-quantisation of the decoded stack), "Supported scope" (64-bit
 *    expert offsets in the MXFP4 grouped kernels).
 *  - "MoE Training & Inference Guides -- Cerin Amroth", "Solutions -- one page
 *    per problem": grouped-nf4-gemm entries (routed expert GEMM on NF4 packed
 *    weights in one launch, nibbles decoded in registers, fp32 accumulation, no
 *    bf16 expert tensor; the same on released e2m1 blocks and e8m0 scales) and
 *    the experts4bit-qlora QLoRA entry (per-expert low-rank delta before each
 *    routed expert's activation, over a frozen NF4 stack).
 *  - project page "experts4bit-qlora" -- "What it does" (fused [E, 2I, H] and
 *    [E, H, I] expert stacks), "Use this when" (input gradient through the
 *    frozen 4-bit weights), "Do not use this when" and "Limitations --
 *    qlora-fused-moe-experts" (never fall back silently; refuse a base whose
 *    epilogue differs from the kernel's instead of computing the wrong thing;
 *    one fp32 absmax per 64 NF4 weights).
 *
 * Conventions for every entry point:
 *  - Pointers marked "device" are device (HBM) pointers owned by the caller.
 *    The library allocates nothing; scratch memory is the caller's workspace
 *    (see moe4_workspace_size), except for moe4_expert_forward_noalloc, whose
 *    scratch is a fixed buffer in the library's device code (one per GPU).
 *  - bf16 values are passed as uint16_t bit patterns.
 *  - `stream` is a hipStream_t (NULL = the null stream). Every call only
 *    enqueues work on it and returns; argument validation is synchronous and
 *    happens before anything is enqueued. Device faults surface at the
 *    caller's next synchronisation.
 *  - Every call returns MOE4_OK or a negative status and then sets a message
 *    for moe4_last_error() naming the first offending argument. No call falls
 *    back to another computation; a combination the kernels do not implement
 *    exactly is refused with MOE4_EUNSUPPORTED.
 *  - Tensors read or written with vector loads must be 16-byte aligned (noted
 *    per argument); float and int32 arrays 4-byte aligned.
 *  - Weight offsets are computed in 64-bit arithmetic.
 *  - Calls that share a workspace, or write the same outputs, must be ordered
 *    on one stream; the library has no internal locking.
 */
#ifndef MOE4_H
#define MOE4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
enum {
  MOE4_OK = 0,
  MOE4_EINVAL = -1,       /* a required pointer is NULL, or an enum is unset/unknown */
  MOE4_EUNSUPPORTED = -2, /* a combination the kernels do not compute exactly */
  MOE4_ESHAPE = -3,       /* a size outside the stated bounds or divisibility */
  MOE4_EALIGN = -4,       /* a pointer without the stated alignment */
  MOE4_EWORKSPACE = -5,   /* workspace missing or smaller than moe4_workspace_size */
  MOE4_EDEVICE = -6       /* the HIP runtime refused a launch */
};

/* storage format of an expert stack */
enum { MOE4_FMT_NF4 = 1, MOE4_FMT_MXFP4 = 2, MOE4_FMT_NF4_DQ = 3 };
/* where gate and up rows sit in the fused [2I, H] stack (no default) */
enum { MOE4_GU_HALVES = 1, MOE4_GU_INTERLEAVED = 2 };
/* expert activation (no default) */
enum { MOE4_ACT_SWIGLU = 1, MOE4_ACT_SWIGLU_CLAMPED = 2 };
/* element type of moe4_combine's output (no default) */
enum { MOE4_DTYPE_BF16 = 1, MOE4_DTYPE_F32 = 2 };
/* kernel choice for the expert GEMMs: AUTO picks by rows per expert */
enum { MOE4_VARIANT_AUTO = 0, MOE4_VARIANT_SKINNY = 1, MOE4_VARIANT_TILED = 2 };

/*
 * One layer's experts. Row n of a stack is output feature n; the reduction
 * dimension is last (y = x W^T).
 *
 * NF4 (blockwise absmax, block 64 along the reduction dimension; two codes per
 * byte, even element in the low nibble; w = NF4[code] * absmax):
 *   gu_q u8 [E, 2I, H/2]   gu_s f32 [E, 2I, H/64]
 *   dn_q u8 [E, H, I/2]    dn_s f32 [E, H, I/64]
 * NF4_DQ (NF4 whose absmax is double-quantised, see moe4_compress_absmax):
 *   gu_q, dn_q as NF4; gu_s u8 [E, 2I, H/64] and dn_s u8 [E, H, I/64] absmax
 *   codes; gu_s2 / dn_s2 f32 [ceil(n/256)] absmax2 and gu_soff / dn_soff f32
 *   [1] offset of each stack (n = its number of absmax); dq_book f32 [256].
 *   absmax = fp32(fp32(dq_book[code] * absmax2[i / 256]) + offset), i the
 *   flat absmax index in the stack. The kernels decode both levels in
 *   place; only a forward whose weight rows hold more than 256 absmax (H or
 *   I above 16384) expands the absmax into the workspace first (its
 *   workspace then grows by the two fp32 absmax arrays).
 * MXFP4 (OCP MX: e2m1 nibbles, 32 per block, one e8m0 scale per block; even
 * element in the low nibble; w = e2m1(n) * 2^(scale - 127)):
 *   gu_q u8 [E, 2I, H/32, 16]   gu_s u8 [E, 2I, H/32]
 *   dn_q u8 [E, H, I/32, 16]    dn_s u8 [E, H, I/32]
 * gu_layout: HALVES = gate rows 0..I-1, up rows I..2I-1;
 *            INTERLEAVED = gate rows 2j, up rows 2j+1 (gpt-oss).
 * act: SWIGLU:  h = silu(g) * u
 *      SWIGLU_CLAMPED: g' = min(g, act_limit), u' = clamp(u, -act_limit,
 *      act_limit), h = (u' + 1) * g' * sigmoid(act_alpha * g') (gpt-oss uses
 *      alpha 1.702, limit 7). Biases are added before the activation.
 * gu_bias bf16 [E, 2I] / dn_bias bf16 [E, H]: optional (NULL = none).
 * lora_A bf16 [E, r, H] and lora_B bf16 [E, 2I, r]: optional, both or neither;
 *   gu += lora_scale * (x A_e^T) B_e^T before the activation; 1 <= r <= 64.
 * variant: MOE4_VARIANT_*; AUTO unless a test needs one kernel family.
 * All stack pointers are device pointers; gu_q/dn_q 16-byte aligned.
 * Bounds (else MOE4_ESHAPE): 1 <= E <= 1024; H and I positive multiples of
 * the block (64 NF4, 32 MXFP4); E*2I*H <= 2^40; I*H < 2^31 - 2^24 (one
 * expert's packed matrix is addressed with 32-bit byte offsets);
 * 1280 * max(H, 2I) < 2^31 - 2^24 (a 320-row tile of fp32 values likewise).
 */
typedef struct moe4_experts {
  int32_t format;
  int32_t E, H, I;
  int32_t gu_layout;
  int32_t act;
  float act_alpha, act_limit;
  const void* gu_q;
  const void* gu_s;
  const void* dn_q;
  const void* dn_s;
  const uint16_t* gu_bias;
  const uint16_t* dn_bias;
  const uint16_t* lora_A;
  const uint16_t* lora_B;
  int32_t lora_r;
  float lora_scale;
  int32_t variant;
  /* MOE4_FMT_NF4_DQ only (NULL otherwise) */
  const float* gu_s2;
  const float* dn_s2;
  const float* gu_soff;
  const float* dn_soff;
  const float* dq_book;
} moe4_experts;

/*
 * NF4 quantisation of a flat fp32 array (device), block 64 (the only size).
 * Per block: absmax = max|w|; x = w / absmax (IEEE fp32 division); code = the
 * number of the 15 fp32 midpoints between adjacent NF4 levels that are
 * strictly below x (nearest level; a value on a midpoint takes the lower
 * code); an all-zero block has absmax 0 and codes 7. Inputs must be finite.
 * [experts4bit-qlora page, "Limitations -- qlora-fused-moe-experts": one fp32
 * absmax per 64 weights; MXFP4 page, "Two fidelity paths": the NF4 stack is the
 * quantiser's output.]
 *   w      f32 [n], 16-byte aligned;  n % 64 == 0 (else MOE4_ESHAPE), n >= 0
 *   packed u8  [n/2] out, two codes per byte, even element in the low nibble
 *   absmax f32 [n/64] out
 */
int moe4_quantize_nf4(const float* w, int64_t n, int32_t blocksize,
                      uint8_t* packed, float* absmax, void* stream);

/*
 * Double quantisation of an NF4 stack's absmax [experts4bit-qlora page,
 * "Limitations -- qlora-fused-moe-experts", the double-quantised absmax item:
 * one offset, an 8-bit code per absmax and one fp32 per 256 absmax, about a
 * quarter of the bytes, lossy against the fp32 absmax]. The pages name the
 * 8-bit code book but print none: it is an argument, 256 strictly increasing
 * fp32 values (else the codes are unspecified).
 *   offset[0] = fp32 rounding of the float64 mean of absmax[0..n)
 *   per group g of 256 (the last may be shorter): d = fp32(absmax - offset),
 *   absmax2[g] = max |d|, code = the book entry nearest to fp32(d / absmax2[g])
 *   (0 when absmax2[g] = 0), decided by the fp32 midpoints of adjacent
 *   entries formed in float64; a value on a midpoint takes the lower code.
 *   absmax f32 [n] (finite), book f32 [256]; code u8 [n] out (4-byte aligned),
 *   absmax2 f32 [ceil(n/256)] out, offset f32 [1] out (device memory)
 *   ws: at least MOE4_DQ_WS_BYTES bytes of device scratch (8-byte aligned)
 */
enum { MOE4_DQ_WS_BYTES = 8192 };
int moe4_compress_absmax(const float* absmax, int64_t n, const float* book, uint8_t* code,
                         float* absmax2, float* offset, void* ws, size_t ws_bytes,
                         void* stream);

/*
 * The decoded absmax of a double-quantised stack [same page and item]:
 * out[i] = fp32(fp32(book[code[i]] * absmax2[i / 256]) + offset[0]), one fp32
 * product and one fp32 sum (no fused multiply-add).
 *   code u8 [n], absmax2 f32 [ceil(n/256)], offset f32 [1], book f32 [256]
 *   (device memory); out f32 [n] out
 */
int moe4_expand_absmax(const uint8_t* code, const float* absmax2, const float* offset,
                       const float* book, int64_t n, float* out, void* stream);

/*
 * Bit-exact MXFP4 -> bf16 decode [MXFP4 page, "Why it happens" and "Two
 * fidelity paths"]. out[r, k] = bf16(e2m1(nibble) * 2^(scale - 127)), element
 * k of row r taken from blocks[r, k/32, (k%32)/2] (even k = low nibble). Every
 * value is exact in bf16 (normal or subnormal) or overflows to +-inf; the sign
 * of zero is kept; scale byte 0xFF (e8m0 NaN) gives 0x7FC0.
 *   blocks u8 [R, K/32, 16] (16-byte aligned), scales u8 [R, K/32]
 *   out    bf16 [R, K] (16-byte aligned); K % 32 == 0
 */
int moe4_decode_mxfp4(const uint8_t* blocks, const uint8_t* scales, int64_t R, int64_t K,
                      uint16_t* out, void* stream);

/*
 * MXFP4 -> NF4 re-quantisation of a stack in one pass [MXFP4 page, "Two
 * fidelity paths": the convenient QLoRA path decodes the released blocks
 * exactly and quantises the decoded stack to NF4]. Computes exactly
 * moe4_quantize_nf4 applied to the moe4_decode_mxfp4 output read as fp32, row
 * by row, so NF4 block q of a row covers MXFP4 blocks 2q and 2q + 1. Scale
 * bytes up to 252 always decode to finite values; for a block that decodes to
 * inf or NaN (bytes 253..255) the output is unspecified.
 *   blocks u8 [R, K/32, 16] (16-byte aligned), scales u8 [R, K/32]
 *   packed u8 [R, K/2] out (16-byte aligned), absmax f32 [R, K/64] out
 *   K % 64 == 0 (else MOE4_ESHAPE)
 */
int moe4_convert_mxfp4_nf4(const uint8_t* blocks, const uint8_t* scales, int64_t R, int64_t K,
                           uint8_t* packed, float* absmax, void* stream);

/*
 * Top-k routing on given fp32 router logits [Offload page, "Why it happens":
 * top-k routing sends each token to a small subset of the experts; project
 * page "experts4bit-qlora", "Current measured position": the top-k choice
 * itself flips under rounding of the logits, so the logits are taken as given
 * fp32 inputs and the choice is exact on them]. Per token: the k largest
 * logits, output in that order; weights = softmax over all E restricted to
 * the k and, if renormalize != 0, divided by their sum (softmax, then top-k,
 * then renormalise). Readings where the pages are silent: the choice is made
 * on the logits (not on the rounded probabilities); equal logits -> lower
 * expert index; +0 == -0. NaN logits give unspecified output.
 *   logits f32 [T, E]; 1 <= k <= E <= 1024; T >= 0
 *   topk_idx i32 [T, k] out; topk_w f32 [T, k] out
 */
int moe4_route(const float* logits, int32_t T, int32_t E, int32_t k, int32_t renormalize,
               int32_t* topk_idx, float* topk_w, void* stream);

/*
 * Router logits, the step in front of moe4_route [experts4bit-qlora page,
 * "Current measured position": rounding flips router top-k choices between
 * arithmetically equivalent forwards, so routing is compared against a
 * measured floor]: logits[t, e] = sum_h x[t, h] * wr[e, h] (+ bias[e]),
 * products of bf16 values summed in fp32 (MFMA, order unspecified; each
 * logit is within the fp32 dot-product bound gamma_H * sum |x w| of the exact
 * sum).
 *   x bf16 [T, H], wr bf16 [E, H] (both 16-byte aligned); bias f32 [E] or NULL
 *   logits f32 [T, E] out; 1 <= E <= 1024; H a positive multiple of 8 below 2^25
 */
int moe4_router_logits(const uint16_t* x, const uint16_t* wr, const float* bias, int32_t T,
                       int32_t H, int32_t E, float* logits, void* stream);

/*
 * Backward of the routing weights [same page and section]. With
 * out[t] = sum_j w[t, j] * y_perm[row_of_slot[t*k + j]], given the upstream
 * gradient dOut:
 *   dw[t, j] = <dOut[t], y_perm[row_of_slot[t*k + j]]>   (fp32 sums)
 *   dlogits[t, e]: renormalize != 0 (weights = softmax of the k chosen
 *   logits): w[t, j] * (dw[t, j] - sum_i w[t, i] dw[t, i]) for e = topk_idx[t, j],
 *   0 for experts not chosen; renormalize == 0 (weights = the full softmax p of
 *   `logits`): p[t, e] * (g[t, e] - sum_i w[t, i] dw[t, i]), g = dw at the
 *   chosen experts, 0 elsewhere. The top-k choice itself has no gradient.
 *   topk_idx i32 [T, k] (distinct experts in [0, E) per token, as moe4_route
 *   writes them; otherwise the output is unspecified), topk_w f32 [T, k]
 *   logits f32 [T, E] (read only when renormalize == 0, then required)
 *   dout bf16 [T, H], y_perm f32 [T*k, H] (16-byte aligned), row_of_slot i32 [T*k]
 *   dw f32 [T, k] out, dlogits f32 [T, E] out; H % 8 == 0
 */
int moe4_route_backward(const int32_t* topk_idx, const float* topk_w, const float* logits,
                        int32_t renormalize, const uint16_t* dout, const float* y_perm,
                        const int32_t* row_of_slot, int32_t T, int32_t k, int32_t E, int32_t H,
                        float* dw, float* dlogits, void* stream);

/*
 * Stable permutation of the T*k routed slots (s = t*k + j) by expert, plus the
 * row gather [Solutions index, grouped-nf4-gemm entry: the routed expert GEMM
 * runs over every expert in one launch, so its input rows are grouped by
 * expert; project page "experts4bit-qlora", "What it does": the experts of a
 * layer are one fused [E, ...] stack indexed by expert]. Rows of expert e are
 * offsets[e] .. offsets[e+1]-1. Reading where the pages are silent: inside an
 * expert, rows keep ascending slot order (a stable counting sort), which
 * makes every index deterministic; any order gives the same layer output. x_perm[r] = x[slot_of_row[r] / k], or with row_scale,
 * bf16(fp32(row_scale[s] * x[s / k])) (IEEE product, one rounding), which
 * scales an upstream gradient by its routing weight for the backward.
 *   topk_idx i32 [T, k] with values in [0, E) (else unspecified output)
 *   offsets i32 [E+1] out; slot_of_row i32 [T*k] out; row_of_slot i32 [T*k] out
 *   x bf16 [T, H] or NULL (then no gather); row_scale f32 [T*k] or NULL
 *   x_perm bf16 [T*k, H] out (required when x is given); x, x_perm 16-byte
 *   aligned, H % 8 == 0
 *   ws: workspace of at least moe4_workspace_size bytes (256-byte aligned)
 */
int moe4_permute(const int32_t* topk_idx, int32_t T, int32_t k, int32_t E,
                 int32_t* offsets, int32_t* slot_of_row, int32_t* row_of_slot,
                 const uint16_t* x, const float* row_scale, int32_t H, uint16_t* x_perm,
                 void* ws, size_t ws_bytes, void* stream);

/*
 * The row gather of moe4_permute on a permutation already computed [the same
 * passages]: x_perm[r] = x[slot_of_row[r] / k], or with row_scale,
 * bf16(fp32(row_scale[s] * x[s / k])) for s = slot_of_row[r], as moe4_permute
 * writes them. For the backward of a layer whose forward permuted its tokens:
 * the upstream gradient gathered with the routing weights, without ranking the
 * slots again.
 *   x bf16 [T, H], 16-byte aligned, H % 8 == 0
 *   slot_of_row i32 [T*k] (a permutation of the slots, as moe4_permute writes
 *   it; a row whose entry lies outside [0, T*k) is written as zeros)
 *   row_scale f32 [T*k] or NULL
 *   x_perm bf16 [T*k, H] out, 16-byte aligned (caller-owned)
 * Asynchronous on stream; argument errors are returned before anything is
 * launched.
 */
int moe4_gather_rows(const uint16_t* x, int32_t T, int32_t k, int32_t H,
                     const int32_t* slot_of_row, const float* row_scale, uint16_t* x_perm,
                     void* stream);

/*
 * moe4_route followed by moe4_permute (without row_scale), in one launch when
 * the batch is small (a decode step of at most 4 tokens),
 * otherwise as the two calls [the passages of both]. Every output is bit for
 * bit the two calls' output (same selection order, weights and stable
 * permutation). Arguments as moe4_route and moe4_permute; ws as moe4_permute.
 */
int moe4_route_permute(const float* logits, int32_t T, int32_t E, int32_t k,
                       int32_t renormalize, int32_t* topk_idx, float* topk_w, int32_t* offsets,
                       int32_t* slot_of_row, int32_t* row_of_slot, const uint16_t* x, int32_t H,
                       uint16_t* x_perm, void* ws, size_t ws_bytes, void* stream);

/*
 * Grouped expert forward over permuted rows [Solutions index, grouped-nf4-gemm
 * entries; QLoRA entry for the adapter]:
 *   gu = x_perm W_gu[e]^T + b_gu[e] + lora_scale * (x_perm A_e^T) B_e^T
 *   h  = act(gate, up);   y_perm = h W_d[e]^T + b_d[e]
 * Weights are dequantised in registers to bf16 and multiplied on bf16 MFMA
 * with fp32 accumulation; h (the down GEMM's operand) is rounded to bf16,
 * y_perm stays fp32 so that the combine rounds only once.
 *   x_perm bf16 [rows, H] (16-byte aligned); offsets i32 [E+1] from
 *   moe4_permute with offsets[E] == rows; rows = T*k >= 0
 *   y_perm f32 [rows, H] out (16-byte aligned)
 *   save_gu f32 [rows, 2I] out or NULL: pre-activation gu (for the backward;
 *   fp32 so that the clamp masks of the backward see unrounded values)
 *   save_xa f32 [rows, r] out or NULL: x_perm A_e^T (for the backward; LoRA only)
 */
int moe4_expert_forward(const moe4_experts* ex, const uint16_t* x_perm, const int32_t* offsets,
                        int32_t rows, float* y_perm, float* save_gu, float* save_xa,
                        void* ws, size_t ws_bytes, void* stream);

/*
 * moe4_expert_forward with the row gather fused into the gate_up GEMM's loads
 * [same passages; the gather of moe4_permute's definition]: row r of the
 * grouped GEMM reads row slot_of_row[r] / k of x itself, so x_perm is never
 * written. The results are bit for bit those of moe4_permute (with x) followed by
 * moe4_expert_forward: the same operand values reach the same MFMAs. For a
 * forward without adapters (the adapter path and its backward take x_perm).
 *   x bf16 [T, H] (16-byte aligned), T * H * 2 < 2^29 bytes; k >= 1
 *   slot_of_row i32 [T*k] and offsets i32 [E+1] from moe4_permute (or
 *   moe4_route_permute) called without x; rows == T*k
 *   y_perm, save_gu, ws as moe4_expert_forward; MOE4_EUNSUPPORTED with adapters
 */
int moe4_expert_forward_gather(const moe4_experts* ex, const uint16_t* x, int32_t T, int32_t k,
                               const int32_t* slot_of_row, const int32_t* offsets, int32_t rows,
                               float* y_perm, float* save_gu, void* ws, size_t ws_bytes,
                               void* stream);

/*
 * moe4_expert_forward without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid allocation): the same computation and kernels, with the scratch
 * memory (the bf16 activations h, the adapter projection xa, and for weight
 * rows of more than 256 absmax the expanded absmax of a double-quantised
 * stack) in a buffer of
 * MOE4_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends. Allocates nothing.
 *   A call that needs more scratch than that (moe4_workspace_size's forward
 *   part: rows * I * 2 bytes, + rows * r * 4 with LoRA, + the two fp32 absmax
 *   arrays of an NF4_DQ stack on the prefill-sized path) returns
 *   MOE4_EWORKSPACE. `stream` must belong to the current device (else
 *   MOE4_EINVAL). Nothing in the scratch is assumed to start at any value.
 *   All calls on one GPU share its buffer: calls that overlap on a GPU (two
 *   streams, two threads) race; order them on one stream.
 */
enum { MOE4_NOALLOC_SCRATCH_BYTES = 16 << 20 };
int moe4_expert_forward_noalloc(const moe4_experts* ex, const uint16_t* x_perm,
                                const int32_t* offsets, int32_t rows, float* y_perm,
                                float* save_gu, float* save_xa, void* stream);

/*
 * Weighted un-permute: out[t] = sum_{j=0..k-1} w[t,j] * y_perm[row_of_slot[t*k+j]],
 * summed in fp32 in ascending j; topk_w == NULL gives the plain sum (used to
 * sum dx_perm into dX after the backward). The pages do not spell the combine
 * out: this is the reading of the standard routed-MoE output, the routing
 * weights of a token's k experts applied to their outputs [project page
 * "experts4bit-qlora", "What it does": fused MoE layers served and trained as
 * the model defines them; Offload page, "Why it happens": each token uses its
 * top-k experts]. Reading: the down bias is inside y_perm, so it is weighted
 * too; the fixed ascending-j order makes the sum deterministic. out_dtype MOE4_DTYPE_BF16 stores
 * the fp32 sum rounded once to bf16 (the model dtype); MOE4_DTYPE_F32 stores
 * the fp32 sum itself (the same bits before rounding).
 *   y_perm f32 [T*k, H] (16-byte aligned); out [T, H] of out_dtype (16-byte
 *   aligned); H % 8 == 0
 */
int moe4_combine(const float* y_perm, const int32_t* row_of_slot, const float* topk_w,
                 int32_t T, int32_t k, int32_t H, void* out, int32_t out_dtype, void* stream);

/*
 * Backward of the expert path with respect to its input and the LoRA adapters
 * (the frozen 4-bit base and the biases get no gradient) [experts4bit-qlora
 * page, "Use this when": training with the input gradient through the frozen
 * 4-bit weights]. Given dy_perm = moe4_permute(dOut, row_scale = topk_w):
 *   dH = dy_perm W_d[e];  dGU = act'(gu) * dH;  t = dGU B_e
 *   dx_perm = dGU W_gu[e] + lora_scale * t A_e
 *   dA[e] = lora_scale * t^T x_perm;  dB[e] = lora_scale * dGU^T xa
 * dA and dB are written for every expert (zero for experts with no rows).
 *   save_gu f32 [rows, 2I] and save_xa f32 [rows, r] from moe4_expert_forward
 *   dy_perm bf16 [rows, H]; dx_perm f32 [rows, H] out (16-byte aligned)
 *   dA f32 [E, r, H] out, dB f32 [E, 2I, r] out (required with LoRA, else NULL)
 */
int moe4_expert_backward(const moe4_experts* ex, const uint16_t* x_perm, const int32_t* offsets,
                         int32_t rows, const float* save_gu, const float* save_xa,
                         const uint16_t* dy_perm, float* dx_perm, float* dA, float* dB,
                         void* ws, size_t ws_bytes, void* stream);

/*
 * Optional launch timing, for measurement. After this call the calling
 * thread's moe4_expert_forward records events[0] / events[1] (hipEvent_t
 * handles created by the caller) on `stream` immediately before / after its
 * gate_up GEMM launch and events[2] / events[3] around its down GEMM launch;
 * moe4_expert_backward records its down-projection dgrad and gate_up dgrad
 * launches the same way. The array is read at each call, not copied, and must
 * stay valid until timing is switched off with (NULL, 0). n_events must be 0
 * or at least 4 (else MOE4_EINVAL).
 */
int moe4_set_timing_events(void* const* events, int32_t n_events);

/* Workspace bytes needed by moe4_permute, moe4_expert_forward and
 * moe4_expert_backward for this stack and T tokens at top-k (the maximum of
 * the three). Returns 0 if the descriptor or sizes are invalid. */
size_t moe4_workspace_size(const moe4_experts* ex, int32_t T, int32_t k);

/* Message of the calling thread's last failure ("" after success). */
const char* moe4_last_error(void);

/* Kernel family of the calling thread's last moe4_expert_forward or
 * moe4_expert_backward: MOE4_VARIANT_SKINNY or MOE4_VARIANT_TILED (0 if none
 * ran), so callers can assert which kernel engaged. */
int moe4_last_variant(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE4_H */
