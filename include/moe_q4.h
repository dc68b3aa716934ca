/*
 * moe_q4.h -- C ABI of the MI355X (gfx950) Q4_0 W4A8 mixture-of-experts
 * expert-matmul library (libmoe_q4.so).
 *
 * Source pages: "A 35B Hybrid-Attention Mixture-of-Experts Model on a 6GB 2011
 * GPU: Hand-Written 4-bit CUDA Inference for Fermi" (gist.science 2606.24031),
 * cited by page language and section:
 *   [nl Methodologie 1]  Dutch technical summary, Methodologie item 1: prefill
 *                        runs a grouped 4-bit GEMM for the MoE routing; decode
 *                        runs a W4A8 integer kernel (4-bit weights, 8-bit
 *                        activations, integer multiply-adds) over weights that
 *                        are read where they reside.
 *   [nl Methodologie 2]  same page, item 2: group-wise symmetric 4-bit weights
 *                        of the Q4_0 family, 8-bit activations.
 *   [nl Methodologie 4]  same page, item 4: single-pass prefill (the whole
 *                        prompt in one pass, maximal GEMM batch).
 *
 * Formats (the pages name the Q4_0 family without fixing its numbers; these
 * are the readings the library implements):
 *   Q4_0 weights, structure of arrays.  A matrix with R rows and K columns
 *     (K % 32 == 0) is a nibble array qs[R][K/2] (uint8) and a scale array
 *     d[R][K/32] (IEEE binary16 bit patterns).  Block b of row r covers
 *     columns 32b..32b+31; byte i of the block (qs[r][16b+i]) carries column
 *     32b+i in its low nibble and 32b+16+i in its high nibble; the weight is
 *     (q - 8) * d[r][b].
 *   Q8_0 activations.  x[rows][cols] (fp32) becomes xq[rows][cols] (int8) and
 *     xd[rows][cols/32] (fp32): per 32-wide block d = amax / 127 (correctly
 *     rounded), q = round-half-even(x / d) (correctly rounded divide),
 *     clamped to [-127, 127]; amax = 0 gives d = 0 and q = 0.
 *
 * Conventions shared by every call:
 *   - Every tensor pointer is DEVICE memory owned by the caller.  The library
 *     never allocates, frees or synchronises; all work is enqueued on
 *     `stream` (a hipStream_t; NULL is the null stream) and is asynchronous.
 *   - The return value is a status code (MOE_Q4_OK or a negative error).
 *     Arguments are validated before anything is enqueued; on a validation
 *     error nothing is written.  A failed kernel launch returns
 *     MOE_Q4_ERR_HIP; faults inside a kernel surface at the caller's next
 *     synchronisation, as usual for HIP.
 *   - Inputs must be finite; outputs must not alias inputs (one documented
 *     exception: moe_q4_decode_fused's y may be its x).
 *   - Calls keep no state between them and are reentrant; calls that share
 *     an output or workspace buffer must be ordered by the caller.
 */
#ifndef MOE_Q4_H
#define MOE_Q4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
enum {
    MOE_Q4_OK = 0,
    MOE_Q4_ERR_INVALID_ARG = -1, /* null pointer, bad size, misaligned pointer */
    MOE_Q4_ERR_WORKSPACE = -2,   /* workspace missing or smaller than required */
    MOE_Q4_ERR_UNSUPPORTED = -3, /* valid but outside the shapes this build supports */
    MOE_Q4_ERR_HIP = -4          /* the HIP runtime reported a launch error */
};

/* flags */
enum {
    MOE_Q4_QUANT_RMSNORM = 1u, /* quantize_act: first scale each row by 1/sqrt(mean(x^2) + 1e-6) */
    MOE_Q4_ACCUMULATE = 2u     /* decode/prefill: y += result instead of y = result */
};

/* Shape limits of this build. */
#define MOE_Q4_MAX_EXPERTS 1024
#define MOE_Q4_MAX_TOPK 16
#define MOE_Q4_MAX_DECODE_TOKENS 64
#define MOE_Q4_MAX_FUSED_TOKENS 8
#define MOE_Q4_MAX_FUSED_HQ_BYTES 65536 /* T * k * I bound of moe_q4_decode_fused */
#define MOE_Q4_MAX_STACK_LAYERS 48       /* layers of one moe_q4_decode_stack call */
#define MOE_Q4_WS_ERROR_OFFSET 2112      /* sticky error word of the fused and stack decodes' sync area */
#define MOE_Q4_STATIC_SCRATCH_BYTES (8u << 20) /* device scratch of moe_q4_decode_static, per GPU */

/*
 * The experts of one MoE layer, all resident in device memory (nothing is
 * streamed).  A host struct of device pointers, read during the call only.
 *   gate_qs, up_qs [E][I][H/2]   gate_d, up_d [E][I][H/32]
 *   down_qs        [E][H][I/2]   down_d       [E][H][I/32]
 * Supported: 1 <= E <= 1024; H in {256, 512, 1024, 2048}; I in {256, 512, 1024}.
 * Every pointer 16-byte aligned.
 */
typedef struct moe_q4_experts {
    int32_t num_experts; /* E */
    int32_t hidden;      /* H */
    int32_t inter;       /* I */
    const uint8_t* gate_qs;
    const uint8_t* up_qs;
    const uint8_t* down_qs;
    const uint16_t* gate_d;
    const uint16_t* up_d;
    const uint16_t* down_d;
} moe_q4_experts;

/*
 * Q8_0 activation quantisation [nl Methodologie 2] (8-bit activations).
 *   x  [rows][cols] fp32, 16-byte aligned, cols % 32 == 0, 32 <= cols <= 16384
 *   xq [rows][cols] int8 (4-byte aligned), xd [rows][cols/32] fp32 (out)
 *   flags: 0 or MOE_Q4_QUANT_RMSNORM (the row factor is computed in fp64 and
 *          each scaled element is rounded to fp32 before quantisation).
 * rows == 0 is a valid no-op.
 */
int moe_q4_quantize_act(const float* x, int64_t rows, int64_t cols, uint32_t flags, int8_t* xq, float* xd,
                        void* stream);

/*
 * Router [nl Methodologie 1] (the MoE routing that feeds the grouped GEMM):
 * softmax over the E logits of each token, keep the k largest, renormalise
 * over the kept k, then group the T*k (token, slot) pairs by expert.
 *   logits [T][E] fp32 (in)
 *   topk_ids [T][k] int32 (out): chosen experts, larger logit first, equal
 *            logits broken by the lower expert id
 *   topk_w [T][k] fp32 (out): renormalised weights (computed in fp64)
 *   expert_offsets [E+1] int32 (out): exclusive prefix sum of per-expert pair
 *            counts; expert_offsets[E] == T*k
 *   sorted_pairs [T*k] int32 (out): pair ids p = t*k + j grouped by expert,
 *            ascending p within each expert (a stable counting sort)
 * 1 <= E <= 1024, 1 <= k <= min(E, 16), 0 <= T, T*k < 2^31.  Results are
 * deterministic (no order-dependent atomics).
 */
int moe_q4_route(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* topk_ids, float* topk_w,
                 int32_t* expert_offsets, int32_t* sorted_pairs, void* stream);

/*
 * Bytes of workspace that moe_q4_decode / moe_q4_decode_fused / moe_q4_prefill
 * need for a call with these sizes (a multiple of 256).  Layout, with P = T*k
 * and A(v) = v rounded up to a multiple of 256:
 *   [0, 20480)                      sync area of moe_q4_decode_fused (the
 *                                   other calls never touch it): arrival and
 *                                   departure counters, at byte 2112 a uint32
 *                                   error word, a call counter, and from byte
 *                                   4096 an exchange area for h tagged with
 *                                   the call counter.  It must be zero before
 *                                   the first fused call on a workspace
 *                                   (zero-fill it once when allocating it);
 *                                   every fused call leaves the counters at
 *                                   zero.  The error word is sticky: nonzero
 *                                   means a bounded wait gave up (that call's
 *                                   results are invalid; zero the area again).
 *   [20480, 20480 + P*I)            hq: int8 [P][I], the re-quantised SwiGLU
 *                                   output; row s = the pair at sorted position s
 *   [20480 + A(P*I), + P*(I/32)*4)  hd: fp32 [P][I/32], its block scales
 *   [20480 + A(P*I) + A(P*I/8), + P*H*4)
 *                                   o: fp32 [P][H], per-pair down output
 *                                   (row p = pair id) of moe_q4_decode's
 *                                   expert-major path and of moe_q4_prefill
 * hq/hd hold the call's values when it completes.
 */
size_t moe_q4_workspace_size(int32_t T, int32_t E, int32_t k, int32_t H, int32_t I);

/*
 * One MoE layer, decode [nl Methodologie 1] (W4A8 integer GEMV over resident
 * 4-bit weights): for every token t,
 *   y[t] (+)= sum_j topk_w[t][j] * W_down[e] Q8_0( silu(W_gate[e] x_t) * (W_up[e] x_t) ),
 *   e = topk_ids[t][j], x_t = the Q8_0 row (xq[t], xd[t]).
 * Each block dot is an exact int32 sum of (q_w - 8) * q_a, scaled in fp32 by
 * d_w * d_a.  Every touched expert's weights are read once per call, however
 * many of the T tokens chose it.  The combine is a fixed-order sum (j = 0..k-1):
 * results are deterministic.
 *   w: experts; xq [T][H] int8 (16-byte aligned), xd [T][H/32] fp32
 *   topk_ids, topk_w, expert_offsets, sorted_pairs: moe_q4_route's outputs
 *   flags: 0 or MOE_Q4_ACCUMULATE; y [T][H] fp32 (out, or in/out), 16-byte aligned
 *   ws / ws_bytes: workspace of at least moe_q4_workspace_size(T, E, k, H, I)
 * 0 <= T <= 64 (MOE_Q4_ERR_UNSUPPORTED above).
 */
int moe_q4_decode(const moe_q4_experts* w, const int8_t* xq, const float* xd, int32_t T, int32_t k,
                  const int32_t* topk_ids, const float* topk_w, const int32_t* expert_offsets,
                  const int32_t* sorted_pairs, uint32_t flags, float* y, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_q4_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The same kernels and results as
 * moe_q4_decode (bit for bit); the workspace is a static device array of the
 * library, MOE_Q4_STATIC_SCRATCH_BYTES (8 MiB) on each GPU it runs on, held
 * until the process ends.  The call allocates and frees nothing.
 *   Arguments as moe_q4_decode, minus ws / ws_bytes.
 *   Returns MOE_Q4_ERR_WORKSPACE when moe_q4_workspace_size(T, E, k, H, I)
 *   exceeds MOE_Q4_STATIC_SCRATCH_BYTES (e.g. T = 64, k = 8, H = 2048,
 *   I = 512 needs 4.5 MB and fits), MOE_Q4_ERR_HIP when the array's device
 *   address cannot be obtained.
 * Every call on one GPU shares that GPU's array and leaves its h codes there
 * (nothing in it must start at zero): calls that overlap on one GPU (on
 * different streams, or from several host threads without ordering) race
 * and give wrong results.  Order them on one stream.
 */
int moe_q4_decode_static(const moe_q4_experts* w, const int8_t* xq, const float* xd, int32_t T, int32_t k,
                         const int32_t* topk_ids, const float* topk_w, const int32_t* expert_offsets,
                         const int32_t* sorted_pairs, uint32_t flags, float* y, void* stream);

/*
 * One MoE layer, decode, in a single launch [nl Methodologie 1, 2]: Q8_0
 * quantisation of x (optionally after the RMS pre-norm), routing of `logits`
 * and the layer of moe_q4_decode, with results bit-identical to
 *   moe_q4_quantize_act(x, T, H, flags & MOE_Q4_QUANT_RMSNORM) ;
 *   moe_q4_route(logits, T, E, k) ; moe_q4_decode(..., flags & MOE_Q4_ACCUMULATE)
 * (with the pre-norm, the fp64 row factor is summed in another order and may
 * differ in its last bit).  For small batches, where launches rather than
 * bytes bound the layer.
 *   w: experts; x [T][H] fp32 (16-byte aligned); logits [T][E] fp32
 *   flags: MOE_Q4_QUANT_RMSNORM and/or MOE_Q4_ACCUMULATE
 *   topk_ids, topk_w, expert_offsets, sorted_pairs: the router outputs, as
 *     moe_q4_route writes them (out)
 *   y [T][H] fp32 (out, or in/out), 16-byte aligned.  y may be the same
 *     buffer as x (a residual stream updated in place): every read of x
 *     precedes every write of y.  No other output may alias an input.
 *   ws / ws_bytes: workspace of at least moe_q4_workspace_size(T, E, k, H, I),
 *     whose sync words are zero (see moe_q4_workspace_size); calls sharing a
 *     workspace must be ordered (one stream).
 * 1 <= T <= MOE_Q4_MAX_FUSED_TOKENS and T*k*I <= MOE_Q4_MAX_FUSED_HQ_BYTES
 * (MOE_Q4_ERR_UNSUPPORTED otherwise); T == 0 is a valid no-op.
 */
int moe_q4_decode_fused(const moe_q4_experts* w, const float* x, const float* logits, int32_t T, int32_t k,
                        uint32_t flags, int32_t* topk_ids, float* topk_w, int32_t* expert_offsets,
                        int32_t* sorted_pairs, float* y, void* ws, size_t ws_bytes, void* stream);

/*
 * L consecutive MoE layers of one token in one launch: the W4A8 decode over
 * resident 4-bit experts [nl Methodologie 1, nl Methodologie 2], applied
 * layer after layer to a residual stream h:
 *   h <- [h +] MoE_l(Q8_0([RMSNorm] h)),  l = 0 .. L-1,
 * each layer exactly as moe_q4_decode_fused with T = 1 and x = y = h (the
 * hidden states are bit-identical to that chain of calls).  Every layer's
 * router logits are inputs, so the launch selects layer l+1's experts and
 * streams their weights while layer l finishes.
 *   layers   host array of L expert sets (read during the call only), all
 *            with the same num_experts E, hidden H and inter I
 *   L        1 .. MOE_Q4_MAX_STACK_LAYERS
 *   logits   [L][E] fp32: the router logits of each layer
 *   k        1 .. 8, k <= E
 *   flags    MOE_Q4_QUANT_RMSNORM and/or MOE_Q4_ACCUMULATE, applied at every
 *            layer (both: a pre-norm residual stack)
 *   h        [H] fp32 (in/out, 16-byte aligned): h_0 in, h_L out
 *   h_all    [L][H] fp32 or NULL: h_{l+1} after each layer l (out)
 *   hq_all, hd_all  [L][k][I] int8 and [L][k][I/32] fp32, both or neither
 *            (NULL): each layer's re-quantised h, rows in sorted-pair order
 *            (ascending expert id) (out)
 *   ws / ws_bytes  at least moe_q4_stack_workspace_size(H) bytes, 256-byte
 *            aligned, zero-filled before its first use and afterwards
 *            touched only by this library (it may be shared with
 *            moe_q4_decode_fused calls ordered on one stream).  The call
 *            first routes every layer (moe_q4_route's kernels over the
 *            [L][E] logits as L one-token rows, into the workspace), then
 *            runs the layers in one persistent launch whose grid the device
 *            holds at once (nothing else may occupy the device meanwhile).
 *            The sticky error word at byte MOE_Q4_WS_ERROR_OFFSET becomes
 *            nonzero if a bounded wait of the launch gave up (the outputs
 *            are then invalid).
 * Shapes: H in {256, 512, 1024, 2048}, I in {512, 1024}, E <= MOE_Q4_MAX_EXPERTS
 * (MOE_Q4_ERR_UNSUPPORTED otherwise, also when the launch's k*I/32 + H/16
 * workgroups cannot all be resident on the device at once).
 */
int moe_q4_decode_stack(const moe_q4_experts* layers, int32_t L, const float* logits, int32_t k, uint32_t flags,
                        float* h, float* h_all, int8_t* hq_all, float* hd_all, void* ws, size_t ws_bytes,
                        void* stream);
size_t moe_q4_stack_workspace_size(int32_t H);

/*
 * L consecutive MoE layers of a batch of T tokens (1 <= T <= 16) in one
 * persistent launch: the W4A8 decode over resident 4-bit experts
 * [nl Methodologie 1, nl Methodologie 2] applied layer after layer to a
 * residual stream h [T][H]:
 *   h <- [h +] MoE_l(Q8_0([RMSNorm] h)),  l = 0 .. L-1,
 * every layer with moe_q4_decode's arithmetic (the same block dots, SwiGLU,
 * Q8_0 re-quantisation and slot-order combine) and moe_q4_route's routing
 * (the same ids, weights and pair order).  One difference: with the pre-norm,
 * the fp64 row factor of layers after the first is summed in another order
 * than moe_q4_quantize_act's, so it may differ in its last bit.  At these
 * batch sizes every touched expert is a bandwidth-bound matvec [nl
 * Resultaten: thin-M GEMM]; the launch streams the next task's weights while
 * the current one computes, across layer boundaries too.
 *   layers   host array of L expert sets (same E, H, I), read during the call
 *   L        1 .. MOE_Q4_MAX_STACK_LAYERS
 *   T        1 .. 16 tokens
 *   logits   [L][T][E] fp32: the router logits of every layer
 *   k        1 .. 8, k <= E
 *   flags    MOE_Q4_QUANT_RMSNORM and/or MOE_Q4_ACCUMULATE, at every layer
 *   h        [T][H] fp32 (in/out, 16-byte aligned): h_0 in, h_L out
 *   h_all    [L][T][H] fp32 or NULL: h_{l+1} after each layer l (out)
 *   hq_all, hd_all  [L][T*k][I] int8 and [L][T*k][I/32] fp32, both or
 *            neither: each layer's re-quantised h, rows in that layer's
 *            sorted-pair order (moe_q4_route's sorted_pairs) (out)
 *   ws / ws_bytes  at least moe_q4_stack_batch_workspace_size(L, T, E, k,
 *            H, I) bytes, 256-byte aligned, zero-filled before its first
 *            use and afterwards touched only by this call (sticky error word
 *            at byte MOE_Q4_WS_ERROR_OFFSET: nonzero if a bounded wait gave
 *            up; the outputs are then invalid).  Calls sharing a workspace
 *            must be ordered on one stream.
 * Two launches: the routing of every layer (one workgroup per layer) and the
 * persistent decode, whose grid is as large as the device holds at once (the
 * occupancy query); nothing else may occupy the device meanwhile, or its
 * waits give up and set the error word.
 * Shapes: H in {1024, 2048}, I in {256, 512, 1024}, E <= 1024
 * (MOE_Q4_ERR_UNSUPPORTED otherwise).
 */
int moe_q4_decode_stack_batch(const moe_q4_experts* layers, int32_t L, int32_t T, const float* logits, int32_t k,
                              uint32_t flags, float* h, float* h_all, int8_t* hq_all, float* hd_all, void* ws,
                              size_t ws_bytes, void* stream);
size_t moe_q4_stack_batch_workspace_size(int32_t L, int32_t T, int32_t E, int32_t k, int32_t H, int32_t I);

/*
 * One MoE layer, prefill [nl Methodologie 1] (grouped 4-bit GEMM over the
 * routed experts) in a single pass over all T tokens [nl Methodologie 4]:
 * the same function as moe_q4_decode, scheduled as an int8-MFMA grouped GEMM
 * (gate/up, fused SwiGLU and Q8_0 re-quantisation) followed by a grouped down
 * GEMM that stores each pair's output row o into the workspace, and a combine
 * that forms y_t (+)= sum_j topk_w[t][j] o[t*k+j] in slot order: no atomics,
 * the same y on every run.  Arguments as moe_q4_decode; any T >= 0.
 */
int moe_q4_prefill(const moe_q4_experts* w, const int8_t* xq, const float* xd, int32_t T, int32_t k,
                   const int32_t* topk_ids, const float* topk_w, const int32_t* expert_offsets,
                   const int32_t* sorted_pairs, uint32_t flags, float* y, void* ws, size_t ws_bytes,
                   void* stream);

/*
 * One MoE layer, prefill, W4A16 [nl Methodologie 1, nl Methodologie 2]: the
 * same packed experts with 16-bit activations (the pages tie 8-bit
 * activations to decode; here the activations are not quantised).  The layer
 * input and h are rounded to fp16 (nearest, ties to even); the weights are
 * dequantised to fp16 as fl16((q - 8) * d) and the products accumulate in
 * fp32 on the matrix cores; the combine is moe_q4_prefill's (per-pair rows of
 * o in the workspace, then an ordered sum: the same y on every run).
 *   x      [T][H] fp32 (device, 16-byte aligned): the layer input (no
 *          quantize_act step);
 *   routing arrays as moe_q4_decode (from moe_q4_route);
 *   flags  0 or MOE_Q4_ACCUMULATE;
 *   ws     at least moe_q4_prefill_a16_workspace_size(T, k, H, I) bytes,
 *          256-byte aligned: [0, A(T*H*2)) the input in fp16, then h in fp16
 *          [P][I] in sorted-pair order (both with every group of 8 elements
 *          stored in the order 0,2,1,3,4,6,5,7, the matrix cores' operand
 *          order), then o fp32 [P][H] (row p = pair id); A(v) = v rounded up
 *          to a multiple of 256.
 * Shapes as moe_q4_prefill (H, I multiples of 256); any T >= 0.
 */
int moe_q4_prefill_a16(const moe_q4_experts* w, const float* x, int32_t T, int32_t k, const int32_t* topk_ids,
                       const float* topk_w, const int32_t* expert_offsets, const int32_t* sorted_pairs, uint32_t flags,
                       float* y, void* ws, size_t ws_bytes, void* stream);
size_t moe_q4_prefill_a16_workspace_size(int32_t T, int32_t k, int32_t H, int32_t I);

/*
 * Single-matrix W4A8 matvec [nl Methodologie 1] (the decode kernel's inner
 * loop on one Q4_0 matrix): y[t][n] = sum_b d[n][b] * xd[t][b] * isum[t][n][b].
 *   qs [N][K/2], d [N][K/32] (16-byte aligned); xq [T][K], xd [T][K/32]
 *   y [T][N] fp32 (out).  K in {256, 512, 1024, 2048}, N >= 0, 0 <= T <= 64.
 */
int moe_q4_gemv(const uint8_t* qs, const uint16_t* d, int32_t N, int32_t K, const int8_t* xq, const float* xd,
                int32_t T, float* y, void* stream);

/*
 * Inspection hooks for parity tests: the exact int32 block dot products
 * isum = sum_{i<32} (q_w - 8) * q_a [nl Methodologie 1] as the production
 * device code computes them.
 *
 * moe_q4_debug_block_dots: the decode (v_dot4) device routine on one matrix.
 *   qs [N][K/2], xq [T][K] -> out [T][N][K/32] int32.  K in {256, ..., 2048}
 *   (the gate/up row walk) or K in {256, 512, 1024} with `down_walk` = 1
 *   (the down-projection row walk); 0 <= T <= 64.
 *
 * moe_q4_debug_prefill_dots: the prefill gate/up (which = 0) or down
 *   (which = 1) grouped MFMA kernel with a dump epilogue.  For gate/up, xq/xd
 *   are the token activations [T][H]; for down, the activations are hq/hd in
 *   `ws` from a preceding moe_q4_prefill call with the same routing.
 *   out: int32 [P][2][I][H/32] (gate, up) or [P][H][I/32] (down), rows in
 *   sorted-pair order.  Intended for small shapes.
 */
int moe_q4_debug_block_dots(const uint8_t* qs, int32_t N, int32_t K, const int8_t* xq, int32_t T,
                            int32_t down_walk, int32_t* out, void* stream);
int moe_q4_debug_prefill_dots(const moe_q4_experts* w, const int8_t* xq, const float* xd, int32_t T, int32_t k,
                              const int32_t* expert_offsets, const int32_t* sorted_pairs, int32_t which,
                              int32_t* out, void* ws, size_t ws_bytes, void* stream);

/*
 * Router projection, the step in front of moe_q4_route [nl Methodologie 1]
 * (the pages name the MoE routing but give no router arithmetic; the plain
 * reading is a dense fp32 projection of the layer input):
 *   logits[t][e] = sum_h x_n[t][h] * wr[e][h]
 *   x      [T][H] fp32 (device, 16-byte aligned), the layer input;
 *   wr     [E][H] fp32 (device, 16-byte aligned), the router weights;
 *   flags  0 or MOE_Q4_QUANT_RMSNORM: x_n = x / sqrt(mean(x^2) + 1e-6) per row,
 *          the row factor in fp64 (applied to each finished dot product);
 *   logits [T][E] fp32 (device, out), the input of moe_q4_route.
 * 32 <= H <= 16384 with H % 32 == 0 (INVALID_ARG / UNSUPPORTED otherwise),
 * 1 <= E <= 1024, T >= 0 (T == 0 is a no-op).  fp32 sums in a fixed order:
 * deterministic, within fp32 rounding of the exact projection.
 */
int moe_q4_router_logits(const float* x, int32_t T, int32_t H, const float* wr, int32_t E, uint32_t flags,
                         float* logits, void* stream);

/*
 * Measurement probes: the achievable ceilings that the decode (HBM-bound)
 * and prefill (int8 matrix-core-bound) kernels are measured against, beside
 * the published peaks.  They compute nothing of the method.
 *
 * moe_q4_probe_read: reads `bytes` bytes at `buf` (device memory, 16-byte
 *   aligned, bytes a positive multiple of 16) once, with coalesced 16-byte
 *   non-temporal loads over two workgroups per CU.  `sink` (device, one uint32) is
 *   written only in the (practically impossible) case that the XOR of all
 *   words read equals a fixed constant: it exists so the loads cannot be
 *   dropped.  Bytes read per call: `bytes`.
 *
 * moe_q4_probe_mfma_i8: `workgroups` workgroups of 4 waves; each wave runs
 *   4 * iters v_mfma_i32_32x32x32_i8 (2 * 32 * 32 * 32 = 65536 int ops each)
 *   on register operands, in four independent accumulation chains.  Total
 *   int ops per call: 262144 * iters * 4 * workgroups.  `sink` as above.
 *
 * moe_q4_probe_w4a8_step: `workgroups` workgroups of 4 waves (launched two
 *   per CU, as the prefill kernels run); each wave runs `iters` steps of the
 *   W4A8 prefill's inner product on registers: two v_mfma_i32_32x32x32_i8
 *   and, for each of their 2 x 16 outputs per lane, two fp32 FMAs that apply
 *   a weight and an activation block scale.  This is the highest int8 rate
 *   the per-block-scaled formulation can reach with no memory traffic.  Total
 *   int ops per call: 131072 * iters * 4 * workgroups.  `sink` (device, one
 *   float) as above.
 *
 * All: async on `stream`; INVALID_ARG for null or misaligned pointers and
 * non-positive sizes, HIP on a launch failure.
 */
int moe_q4_probe_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);
int moe_q4_probe_mfma_i8(int32_t iters, int32_t workgroups, int32_t* sink, void* stream);
int moe_q4_probe_w4a8_step(int32_t iters, int32_t workgroups, float* sink, void* stream);

/* Human-readable name of a status code (a static string). */
const char* moe_q4_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_Q4_H */
