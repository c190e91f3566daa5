/*
 * moe.h - C ABI of the routed top-k mixture-of-experts layer for AMD Instinct
 * MI355X (gfx950).
 *
 * The layer is the one the first page (the FlyDSL-in-JAX talk summary) describes
 * under "Optimierung gerouteter MoE-GEMMs" (5:56) and "End-to-End-Integration in
 * MaxText" (8:14): tokens are routed to their top-2 experts, the selected tokens
 * are gathered, a grouped GEMM computes each expert's gate and up
 * projections with a SwiGLU, a second grouped GEMM computes the down
 * projection, and the results are scattered back and combined with the routing
 * weights; expert weights are rearranged once, when they are loaded (8:14).
 * The same talk summary describes the call boundary it
 * used ("fly_call", 4:07; the C trampoline that unpacks buffers, scalars and
 * streams, 5:05): this header is the same kind of boundary, a set of C calls
 * taking device pointers, sizes and a stream.
 *
 * Shapes: x[T,H] tokens, W_r[E,H] router, W1/W3[E,I,H] gate/up, W2[E,H,I] down,
 * top-k with k <= E. Element types: bf16; OCP e4m3fn ("FP8", the precision the
 * talk summary's Mixtral 8x7B kernel runs in, 5:56/7:31) with fp32 scales; or
 * MXFP8 (the second page's scaled-GEMM format, section "Grenzen und Folgen
 * für Anwender": e4m3fn values with one E8M0 scale per 32 values along the
 * reduction; scale code b means 2^(b-127)). MXFP8 block scales are chosen as in the OCP Microscaling
 * specification: x = floor(log2 max|v|) - 8 (0 for an all-zero block), clamped
 * to [-127, 127], code x + 127; values e4m3fn(clamp(v / 2^x, -448, 448)).
 * MXFP4 (the same section's "packed FP4-E2M1 operands"): expert weights are
 * OCP E2M1 codes (1 sign, 2 exponent bits with bias 1, 1 mantissa bit:
 * magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6), two per byte with value 2i in the
 * low nibble of byte i, and one E8M0 scale per 32 values along the reduction;
 * tokens and the intermediate are MXFP8 as above. The weight codes come
 * quantised from the caller.
 *
 * Conventions for every call:
 *   - All array arguments are DEVICE pointers owned by the caller, allocated
 *     with at least the documented size, 16-byte aligned unless noted. The
 *     library never allocates or frees memory and keeps no state between calls,
 *     except moe_stage2_noalloc's scratch array (and its address per device).
 *   - Calls are asynchronous and ordered on `stream` (hipStream_t, may be 0).
 *     Nothing is copied back to the host; device-side counts (total_padded)
 *     stay on the device and later kernels read them there.
 *   - Arguments are checked on the host before any HIP call; a failed check
 *     returns an error code and launches nothing. moe_last_error() then holds
 *     a message naming the argument.
 *   - T == 0 returns MOE_OK and launches nothing (no output is written).
 *   - Layout is row-major; bf16 is passed as its 16-bit pattern, e4m3fn as
 *     its 8-bit code.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1, /* null or misaligned pointer, negative size, k > E ... */
    MOE_ERR_UNSUPPORTED = 2, /* shape outside the supported set (see each call)     */
    MOE_ERR_WORKSPACE = 3,   /* workspace smaller than the size query returned      */
    MOE_ERR_HIP = 4          /* a HIP launch reported an error                      */
} moe_status;

typedef enum { MOE_BF16 = 0, MOE_FP8_E4M3FN = 1, MOE_MXFP8 = 2, MOE_MXFP4 = 3 } moe_dtype;

/* Static string for a status code. */
const char* moe_status_string(int status);
/* Message of the last failed call on this host thread ("" if none). */
const char* moe_last_error(void);
/* Library version string. */
const char* moe_version(void);

/*
 * moe_route - router logits, top-k selection, renormalised routing weights,
 * and (optionally) the per-token FP8 quantisation of x.
 *
 * Top-2 routing is the talk summary's Mixtral setting (8:14); small-K TopK is
 * one of the operators the second page (the PyTorch FlyDSL news item, "Das
 * Wichtigste in Kürze") lists. Definition:
 *   l[t,e] = sum_h x[t,h] * W_r[e,h] (+ bias[e]), in fp32, in this fixed order
 *     so that ids are reproducible bit for bit: the H products go to 64
 *     partial sums, element h to partial (h/8) mod 64; each partial adds its
 *     products in ascending h; the partials are then folded pairwise,
 *     p[l] += p[l+off] for off = 32,16,8,4,2,1; l = p[0]; then one fp32 add
 *     of bias[e].
 *   ids[t, 0..k-1]: experts in order of decreasing logit, ties to the lower
 *     expert index (IEEE compare, -0 == +0).
 *   w[t,j] = exp(l_j - l_0) / sum_{i<k} exp(l_i - l_0)  (softmax over the k
 *     selected logits = full softmax renormalised over the selection), fp32.
 *   FP8 (when x_q != NULL): s_t = max_h |x[t,h]| / 448 (1 if that is 0), fp32;
 *     x_q[t,h] = e4m3fn(clamp(x[t,h] / s_t, -448, 448)), fp32 divide,
 *     round to nearest even.
 *
 * x        bf16 [T,H]          w_router bf16 [E,H]       bias fp32 [E] or NULL
 * topk_ids int32 [T,k] (out)   topk_w   fp32 [T,k] (out)
 * logits   fp32 [T,E] (out) or NULL
 * x_q      uint8 [T,H] (out) or NULL; x_scale fp32 [T] (out), required iff x_q
 * Supported: H % 128 == 0, H <= 8192, 1 <= E <= 64, 1 <= k <= min(E, 8).
 */
moe_status moe_route(const void* x, const void* w_router, const float* bias, int T, int H,
                     int E, int k, int32_t* topk_ids, float* topk_w, float* logits, void* x_q,
                     float* x_scale, hipStream_t stream);

/*
 * moe_route_mx - moe_route with the MXFP8 quantisation of x instead of the
 * per-token one (the block format of the second page, section "Grenzen und
 * Folgen für Anwender").
 * Routing (ids, weights, logits) is exactly moe_route's. Then, for every token
 * t and block b of 32 consecutive hidden values: x = floor(log2 max|x[t, 32b..
 * 32b+31]|) - 8 (0 if that block is all zero), clamped to [-127, 127];
 * x_scale_e8m0[t, b] = x + 127; x_q[t, h] = e4m3fn(clamp(x[t,h] / 2^x, -448,
 * 448)), round to nearest even (the division by a power of two is exact).
 *
 * x_q uint8 [T,H] (out, 8-byte aligned); x_scale_e8m0 uint8 [T, H/32] (out;
 * 8-byte aligned when it feeds moe_stage1). Both required. Other arguments and
 * the supported shapes as moe_route.
 */
moe_status moe_route_mx(const void* x, const void* w_router, const float* bias, int T, int H,
                        int E, int k, int32_t* topk_ids, float* topk_w, float* logits, void* x_q,
                        void* x_scale_e8m0, hipStream_t stream);

/*
 * moe_align - groups the T*k token-slots by expert and pads each group to the
 * M-tile (the per-expert group sizes that change with every batch, talk
 * summary 5:56).
 *
 * Slot s = t*k + j is token t's j-th choice. For e = 0..E-1 in turn, the
 * group of e lists every slot with topk_ids[s] == e in ascending s, followed
 * by the sentinel T*k up to a multiple of block_m.
 *   expert_count[e]   slots of expert e
 *   expert_offset[e]  first row of e's group (expert_offset[E] = total)
 *   total_padded[0]   sum_e ceil(count_e / block_m) * block_m
 *   sorted_slot[p]    slot in padded row p, for p < total_padded
 *   tile_expert[i]    expert of rows [i*block_m, (i+1)*block_m), i < total/block_m
 * Entries past total_padded are not written.
 *
 * topk_ids int32 [T*k]; sorted_slot int32 [moe_align_capacity()];
 * tile_expert int32 [capacity/block_m]; expert_count int32 [E];
 * expert_offset int32 [E+1]; total_padded int32 [1]. All device memory.
 * An id outside [0,E) makes total_padded 0: the stages then compute nothing
 * and moe_stage2 writes an all-zero output.
 * Supported: block_m in {32, 64, 128, 256}, 1 <= E <= 64.
 */
int64_t moe_align_capacity(int T, int k, int E, int block_m); /* ceil((T*k+E*(bm-1))/bm)*bm */
moe_status moe_align(const int32_t* topk_ids, int T, int k, int E, int block_m,
                     int32_t* sorted_slot, int32_t* tile_expert, int32_t* expert_count,
                     int32_t* expert_offset, int32_t* total_padded, hipStream_t stream);

/*
 * moe_route_align - moe_route (mx = 0) or moe_route_mx (mx = 1) followed by
 * moe_align of the ids it writes, for a decode step: the outputs are bit for
 * bit those of the two calls (x_scale is then moe_route's float x_scale or
 * moe_route_mx's uint8 x_scale_e8m0). A single token (T = 1) with
 * H <= 4096 takes one launch (one workgroup routes the token, then groups its
 * slots, ordered by its own barrier); larger batches take the two calls'
 * launches. For callers that run the layer at decode batch sizes, where a
 * launch costs several microseconds of a call of about a hundred.
 * Arguments, layouts, ownership and errors: those of both calls; block_m and
 * the grouping outputs as moe_align's (topk_ids is its input).
 */
moe_status moe_route_align(const void* x, const void* w_router, const float* bias, int T, int H,
                           int E, int k, int mx, int32_t* topk_ids, float* topk_w, float* logits,
                           void* x_q, void* x_scale, int block_m, int32_t* sorted_slot,
                           int32_t* tile_expert, int32_t* expert_count, int32_t* expert_offset,
                           int32_t* total_padded, hipStream_t stream);

/*
 * moe_preshuffle - one-time, load-time relayout of the expert weights into the
 * order the matrix-core kernels read them in (talk summary 8:14). A pure byte
 * permutation: each expert's matrix (rows = output features, a row = the
 * reduction) is cut into fragments of 32 rows x 64 bytes (64 e4m3fn or 32 bf16
 * values, one 32x32 matrix-core step), stored row-block major then reduction
 * block. A fragment is two 1 KB pieces; in piece pc the 16 bytes at l*16
 * (lane l = 0..63) are row l mod 32, bytes (l/32)*32 + pc*16 .. +15 of the
 * fragment's 64 (MXFP8: bytes pc*32 + (l/32)*16 .. +15, so that each piece
 * pair is one 32-value scale block in the matrix-core instruction's grouping).
 * MXFP4 fragments are 32 rows x 32 bytes (64 E2M1 values) in one 1 KB piece:
 * the 16 bytes at l*16 are row l mod 32, bytes (l/32)*16 .. +15 of the
 * fragment's 32 (the instruction's order for 4-bit operands).
 * Gate and up rows are interleaved in blocks of 32 (W1 block, W3 block, ...),
 * so one wave holds the gate and up value of the same intermediate column.
 *
 * w1, w3   [E,I,H] row-major; w2 [E,H,I] row-major (bf16 or e4m3fn codes;
 *          MXFP4: packed E2M1, [E,I,H/2] and [E,H,I/2] bytes)
 * s1, s3   FP8: fp32 [E,I]; s2 FP8: fp32 [E,H] per-output-channel scales.
 *          MXFP8, MXFP4: E8M0 codes, s1, s3 uint8 [E,I,H/32]; s2 uint8 [E,H,I/32]
 *          (one per row and 32 reduction values). BF16: NULL.
 * w13_out  [moe_preshuffle_bytes(dt,E,H,I,0)] bytes; w2_out [.., 1] bytes
 * s13_out  [.., 2] bytes; s2_out [.., 3] bytes (FP8, MXFP8, MXFP4, else unused).
 *          FP8: fp32 [E,2,I] (gate scales then up scales) and fp32 [E,H].
 *          MXFP8, MXFP4 (4-byte aligned): the codes in the order the kernels read
 *          them: per expert, groups of four 32-row blocks (composite rows as
 *          above), then reduction fragment kb (64 values), then lane l = 0..63,
 *          then the four blocks: the code of row l mod 32 of the block, value
 *          block 2*kb + l/32.
 * Supported: H % 128 == 0 and I % 128 == 0 (bf16), H % 256 and I % 256 (FP8,
 * MXFP8, MXFP4).
 */
int64_t moe_preshuffle_bytes(moe_dtype dt, int E, int H, int I,
                             int which /*0: W1+W3, 1: W2, 2: their scales s13, 3: s2*/);
moe_status moe_preshuffle(moe_dtype dt, int E, int H, int I, const void* w1, const void* w3,
                          const void* w2, const void* s1, const void* s3, const void* s2,
                          void* w13_out, void* w2_out, void* s13_out, void* s2_out,
                          hipStream_t stream);

/*
 * moe_stage1 - gather + grouped gate/up GEMM + SwiGLU (talk summary 5:56; the
 * SwiGLU of its glossary). For each padded row p < total_padded with slot
 * s = sorted_slot[p], token t = s / k, expert e = tile_expert[p / block_m]:
 *   g = W1[e] x_t, u = W3[e] x_t (fp32 accumulation; FP8: x_t = x_q[t]*x_scale[t],
 *   W = code * scale; MXFP8: every value times 2^(code - 127) of its 32-value
 *   block, tokens and weights alike; MXFP4: the same with E2M1 weight values),
 *   act[p, i] = bf16(silu(g_i) * u_i),
 *   silu(z) = z/(1+e^-z).
 * Pad rows (s == T*k) get act = 0.
 * FP8 also writes act_amax: per row p, partial maxima of |silu(g_i) * u_i| (the
 * fp32 values, before their bf16 rounding) over column blocks,
 * [capacity][moe_stage1_amax_floats()/capacity] floats (row-major); stage 2
 * reduces them to the row's requantisation scale and quantises with a
 * correctly rounded fp32 quotient.
 *
 * x_or_xq  bf16 [T,H] (BF16) or e4m3fn [T,H] (FP8 from moe_route, MXFP8 and
 *          MXFP4 from moe_route_mx)
 * x_scale  fp32 [T] (FP8), E8M0 uint8 [T,H/32] (MXFP8, MXFP4; 8-byte aligned) or NULL;
 * w13, s13 from moe_preshuffle
 * sorted_slot, tile_expert, total_padded from moe_align with the same block_m
 * act      bf16 [capacity, I] (out); act_amax as above (FP8) or NULL (else unused)
 * Supported: block_m in {32, 64, 128, 256}; H, I multiples of 128 (bf16) or 256
 * (FP8, MXFP8, MXFP4); MXFP8 and MXFP4 also H <= 8192 and I <= 16384;
 * activations below 2 GiB.
 */
int64_t moe_stage1_amax_floats(moe_dtype dt, int T, int k, int E, int H, int I, int block_m);
moe_status moe_stage1(moe_dtype dt, const void* x_or_xq, const void* x_scale, const void* w13,
                      const void* s13, const int32_t* sorted_slot, const int32_t* tile_expert,
                      const int32_t* total_padded, int T, int k, int E, int H, int I,
                      int block_m, void* act, float* act_amax, hipStream_t stream);

/*
 * moe_stage1_save_preact - moe_stage1 for the bf16 layer in a training step
 * (the custom VJP of the talk summary's "Ausblick und Roadmap", 10:07): the
 * same act, and also the pre-activations the backward needs, so that
 * moe_backward need not recompute them: gu bf16 [capacity, 2I], g = W1[e] x_t in
 * columns 0..I-1 and u = W3[e] x_t in I..2I-1 of row p, for the real rows only
 * (pad rows are left as they are). The values are bit-identical to those
 * moe_backward recomputes. gu 16-byte aligned, caller-owned; other arguments
 * and errors as moe_stage1 with dt = MOE_BF16.
 */
moe_status moe_stage1_save_preact(const void* x, const void* w13, const int32_t* sorted_slot,
                                  const int32_t* tile_expert, const int32_t* total_padded, int T,
                                  int k, int E, int H, int I, int block_m, void* act, void* gu,
                                  hipStream_t stream);

/*
 * moe_stage2 - grouped down GEMM + weighted scatter-combine (talk summary 5:56,
 * "Scatter"). For each real row p (slot s, token t = s / k, expert e):
 *   y = W2[e] act_p   (FP8: act_p requantised per row, scale = max|act_p|/448,
 *                      code = e4m3fn(act_p / scale); MXFP8, MXFP4: act_p
 *                      quantised per block of 32 values as moe_route_mx does x;
 *                      fp32 accumulation)
 *   out[t, :] = bf16( sum_{j=0..k-1} w[t,j] * y_{t,j} ), summed in ascending j
 *   in fp32: a fixed order, no floating-point atomics, so results are
 *   reproducible bit for bit. (At prefill sizes the tiles of a partial last
 *   round of workgroups are cut into pieces along the reduction whose
 *   partials are summed in piece order; the cut follows from the shapes and
 *   the device-side padded total only, with a fixed round of 256 workgroups,
 *   never from a property queried from the device.)
 *
 * act, act_amax from moe_stage1 (act_amax unused, may be NULL, unless FP8);
 * w2, s2 from moe_preshuffle; topk_w fp32 [T,k]
 * out bf16 [T,H] (out); workspace [moe_stage2_workspace_bytes()] bytes (device,
 * 256-byte aligned): per-slot weighted partials, for FP8, MXFP8 and MXFP4 the
 * requantised intermediate, and at prefill sizes the partials of those
 * reduction pieces.
 * Calls that use one workspace must be ordered (same stream or synchronised).
 */
int64_t moe_stage2_workspace_bytes(moe_dtype dt, int T, int k, int E, int H, int I, int block_m);
moe_status moe_stage2(moe_dtype dt, const void* act, const float* act_amax, const void* w2,
                      const void* s2, const int32_t* sorted_slot, const int32_t* tile_expert,
                      const int32_t* total_padded, const float* topk_w, int T, int k, int E,
                      int H, int I, int block_m, void* out, void* workspace,
                      size_t workspace_bytes, hipStream_t stream);

/*
 * moe_stage2_noalloc - moe_stage2 for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. The same launches and results as moe_stage2, bit for bit;
 * the caller passes the inputs and the output and no workspace: the partials
 * and the requantised intermediate live in one scratch array of 128 MiB inside
 * the library (a file-scope device array; every GPU the library runs on holds
 * its own copy until the process ends). The call allocates and frees nothing.
 *
 * Limit: shapes whose moe_stage2_workspace_bytes() exceeds 128 MiB are
 * rejected with MOE_ERR_WORKSPACE and a message (for the Mixtral shape: every
 * FP8 decode batch up to T = 256 fits; the T = 8192 prefill does not and takes
 * moe_stage2 with a workspace). Every call on one GPU shares that GPU's array: calls that
 * overlap on one GPU (different streams, or host threads without ordering)
 * race and must not be issued. Arguments and errors otherwise as moe_stage2.
 */
moe_status moe_stage2_noalloc(moe_dtype dt, const void* act, const float* act_amax,
                              const void* w2, const void* s2, const int32_t* sorted_slot,
                              const int32_t* tile_expert, const int32_t* total_padded,
                              const float* topk_w, int T, int k, int E, int H, int I,
                              int block_m, void* out, hipStream_t stream);

/*
 * Backward pass of the bf16 layer: the custom VJP the talk summary names as
 * its next step ("Ausblick und Roadmap", 10:07; the glance summary's
 * "What's Next?" also lists wider backward support). For an output gradient dout, the
 * gradients of sum_t <dout_t, out_t> with respect to x, W1, W3, W2, W_r and the
 * router bias, the forward's top-k selection held fixed (it is piecewise
 * constant). Per slot s = t*k + j of expert e with routing weight w_j:
 *   g = W1[e] x_t, u = W3[e] x_t, a = silu(g) u   (a is the forward's act row)
 *   z = W2[e]^T dout_t,  dw_j = <z, a>,  da = w_j z
 *   dg = da u s (1 + g (1 - s)), du = da g s, s = sigmoid(g)
 *   dW2[e] += (w_j dout_t) a^T,  dW1[e] += dg x_t^T,  dW3[e] += du x_t^T
 *   dl_j = w_j (dw_j - sum_i w_i dw_i)       (softmax over the selected logits)
 *   dx_t = sum_j (W1[e_j]^T dg_j + W3[e_j]^T du_j) + sum_j dl_j W_r[e_j]
 *   dW_r[e] = sum of dl_j x_t over the slots of e,  dbias[e] = sum of dl_j
 * Arithmetic: bf16 operands on the matrix cores with fp32 accumulation; g, u,
 * dg, du and w_j dout are held in bf16 between the launches; every sum runs in
 * a fixed order, so the results are reproducible bit for bit.
 *
 * moe_backward_preshuffle - one-time relayout of the transposed weights the
 * backward GEMMs read (W2^T [E][I][H] and [W1^T | W3^T] [E][H][2I], in the
 * bf16 fragment order of moe_preshuffle). w1, w3 bf16 [E,I,H], w2 bf16 [E,H,I];
 * w2t_out [moe_backward_preshuffle_bytes(E,H,I,0)] bytes, w13t_out [.., 1].
 * Supported: H, I multiples of 128.
 *
 * moe_backward - the gradients. Inputs from the forward call on the same
 * tokens: x bf16 [T,H], w_router bf16 [E,H], topk_ids / topk_w (moe_route),
 * sorted_slot, tile_expert, expert_offset, total_padded (moe_align with
 * block_m), act bf16 [capacity, I] (moe_stage1), gu_saved: the pre-activations
 * from moe_stage1_save_preact on the same call (bf16 [capacity, 2I]), or NULL to
 * recompute them (one more stage-1 GEMM; the results are the same bits either
 * way), w13 (moe_preshuffle, bf16), w2t, w13t (moe_backward_preshuffle); dout
 * bf16 [T,H].
 * Outputs (fp32, overwritten): dx [T,H]; dw1, dw3 [E,I,H]; dw2 [E,H,I];
 * dw_router [E,H]; dbias [E] or NULL. Experts without a slot get zero
 * gradients. workspace [moe_backward_workspace_bytes()] bytes, 256-byte
 * aligned. Supported: the bf16 shapes of moe_stage1 (H, I multiples of 128),
 * 4 * capacity * I below 2 GiB.
 */
int64_t moe_backward_preshuffle_bytes(int E, int H, int I, int which /*0: W2^T, 1: W13^T*/);
moe_status moe_backward_preshuffle(int E, int H, int I, const void* w1, const void* w3,
                                   const void* w2, void* w2t_out, void* w13t_out,
                                   hipStream_t stream);
int64_t moe_backward_workspace_bytes(int T, int k, int E, int H, int I, int block_m);
moe_status moe_backward(const void* x, const void* w_router, const int32_t* topk_ids,
                        const float* topk_w, const int32_t* sorted_slot,
                        const int32_t* tile_expert, const int32_t* expert_offset,
                        const int32_t* total_padded, const void* act, const void* gu_saved,
                        const void* w13, const void* w2t, const void* w13t, const void* dout,
                        int T, int k,
                        int E, int H, int I, int block_m, float* dx, float* dw1, float* dw3,
                        float* dw2, float* dw_router, float* dbias, void* workspace,
                        size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
