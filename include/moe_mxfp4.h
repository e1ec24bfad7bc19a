/*
 * moe_mxfp4.h -- C ABI of the routed MXFP4 mixture-of-experts layer on
 * MI355X (gfx950).
 *
 * The layer (DeepSeek-V4.1-Flash's MoE block as the pages describe it):
 *   384 routed experts with 6 chosen per token plus 1 shared expert
 *     (ai.rs article on DeepSeek-V4.1-Flash, table in "What V4.1 Flash is,
 *     in bytes"; FreeToken issue #444, "Architecture delta vs deepseek_v4");
 *   each expert three 5120 x 2304 FP4 matrices (FreeToken issue #444,
 *     "Architecture delta vs deepseek_v4") stored as packed E2M1 codes with
 *     one E8M0 scale per 32 weights (same issue, janit's comment, section 2);
 *   the shared expert gets the same input and arithmetic as the routed ones
 *     (ai.rs article, "What remains is the reference rounding itself");
 *   the gate is a discrete top-k choice whose accumulation order must be
 *     fixed for runs to be reproducible (same section).
 * Softmax scoring, renormalised top-k weights and the SwiGLU expert form are
 * the readings taken where the pages are silent.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - All array pointers are DEVICE pointers (HIP), except `bank` structs,
 *    which live in host memory and hold device pointers.
 *  - The caller owns every buffer. The library allocates nothing, frees
 *    nothing and keeps no pointer after a call returns; scratch memory comes
 *    only from the caller's workspace `ws` (`ws_bytes` long, 16-byte aligned).
 *    moe_workspace_bytes(T, H, I, E, k) bytes suffice for every call below
 *    (for moe_expert_ffn_mxfp4 with R rows, take k = ceil(R / T)).
 *  - Work is enqueued on `stream` and the call returns without waiting; the
 *    host never synchronises. Results are valid after the stream reaches
 *    them. Calls on distinct streams with distinct buffers may overlap.
 *  - bf16 arrays are passed as `const void*` holding bf16 bit patterns.
 *  - Arguments are validated before anything is enqueued: on a negative
 *    return nothing was launched. A device fault surfaces at the caller's
 *    next stream synchronisation. No C++ exception crosses this boundary.
 *  - T == 0 is valid and does nothing (data pointers may then be NULL; the
 *    sizes and banks are still validated).
 *  - Results are bitwise reproducible: no floating-point atomics, and every
 *    sum is taken in a fixed order.
 *
 * Limits: 1 <= E <= 1024, 1 <= k <= min(E, 64), H and I multiples of 32,
 * 32 <= H <= 8192, 32 <= I <= 4096, T*k < 2^31. Violations return
 * MOE_ERR_INVALID_ARG (malformed) or MOE_ERR_UNSUPPORTED (outside limits).
 */
#ifndef MOE_MXFP4_H
#define MOE_MXFP4_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* null required pointer, misalignment, bad size */
  MOE_ERR_UNSUPPORTED = -2, /* well-formed but outside the compiled limits  */
  MOE_ERR_WORKSPACE = -3,   /* ws_bytes smaller than the call needs          */
  MOE_ERR_HIP = -4,         /* a kernel launch failed                        */
  MOE_ERR_TIMEOUT = -5      /* a bounded in-kernel wait gave up (reported by
                               moe_workspace_status, never by a launch call) */
};

/*
 * An MXFP4 expert bank (FreeToken issue #444, janit's comment, section 2:
 * packed E2M1 codes plus one E8M0 scale per 32 weights, not transposed).
 *
 *   gate_up_codes  [E][2][I][H/2]   matrix 0 = gate, 1 = up; K = H
 *   gate_up_scales [E][2][I][H/32]
 *   down_codes     [E][H][I/2]      K = I
 *   down_scales    [E][H][I/32]
 *
 * Rows run along the reduction dimension K. Byte b of a row holds element
 * 2b in its low nibble and 2b+1 in its high nibble. E2M1 codes 0..7 are
 * +{0, 0.5, 1, 1.5, 2, 3, 4, 6} and 8..15 their negatives; scale byte s
 * multiplies its 32 elements by 2^(s-127), and s == 255 is NaN (OCP MX).
 * Code arrays must be 16-byte aligned. The shared expert is a bank with E=1.
 */
typedef struct moe_mxfp4_bank {
  const uint8_t* gate_up_codes;
  const uint8_t* gate_up_scales;
  const uint8_t* down_codes;
  const uint8_t* down_scales;
  int32_t E, H, I;
} moe_mxfp4_bank;

/*
 * An FP8 expert bank: the reference checkpoint's dense format, fp8 weights
 * in 32 x 32 blocks with ue8m0 scales (FreeToken issue #444, "Is the
 * quantization already supported"). 128 x 128 blocks here would mis-scale
 * every weight without any error (ai.rs article on DeepSeek-V4.1-Flash, "The
 * defect that never raised an error"; FreeToken issue #444, angelbaba01L's
 * comment). Used for the shared expert, so E must be 1.
 *
 *   gate_up_w      [E][2][I][H]       E4M3 bytes, matrix 0 = gate, 1 = up
 *   gate_up_scales [E][2][I/32][H/32] E8M0: block (i, j) covers rows
 *                                     32i..32i+31, columns 32j..32j+31
 *   down_w         [E][H][I]          E4M3 bytes
 *   down_scales    [E][H/32][I/32]
 *
 * E4M3 is the OCP fp8 format (1 sign, 4 exponent bits with bias 7, 3
 * mantissa bits; S.1111.111 is NaN); scale byte s multiplies its block by
 * 2^(s - 127), s == 255 is NaN. Rows run along the reduction dimension, as
 * in the MXFP4 banks. Weight arrays must be 16-byte aligned.
 */
typedef struct moe_fp8_bank {
  const uint8_t* gate_up_w;
  const uint8_t* gate_up_scales;
  const uint8_t* down_w;
  const uint8_t* down_scales;
  int32_t E, H, I;
} moe_fp8_bank;

/*
 * An NVFP4 expert bank, the expert format other engines load V4.1 in
 * (FreeToken issue #444, the comment on the other pull request: "NVFP4
 * experts"; the same issue, "Is the quantization already supported"): E2M1
 * codes with one E4M3 scale per 16 (the layout the same issue gives for the
 * model's fp4 KV cache, "Architecture delta vs deepseek_v4", its list of
 * what is new), plus one fp32 scale per expert and matrix.
 *
 *   gate_up_codes  [E][2][I][H/2]   packed as in moe_mxfp4_bank
 *   gate_up_scales [E][2][I][H/16]  E4M3 (OCP fp8) bytes, one per 16 codes
 *   down_codes     [E][H][I/2]
 *   down_scales    [E][H][I/16]
 *   global_scales  [E][3] fp32 (gate, up, down) multiplying the whole
 *                  matrix, or NULL for 1
 *
 * Code arrays 16-byte aligned, scale arrays 4-byte aligned.
 */
typedef struct moe_nvfp4_bank {
  const uint8_t* gate_up_codes;
  const uint8_t* gate_up_scales;
  const uint8_t* down_codes;
  const uint8_t* down_scales;
  const float* global_scales;
  int32_t E, H, I;
} moe_nvfp4_bank;

/* Workspace bytes that suffice for any call below at these sizes. */
size_t moe_workspace_bytes(int T, int H, int I, int E, int k);

/* Human-readable name of a return code (static string). */
const char* moe_status_str(int status);

/*
 * Kernel timing hook (measurement only; no step of the layer depends on it).
 * While set, the i-th kernel launch (i < n) of every call below made from
 * the same host thread carries events[2i] and events[2i+1] as its start and
 * stop events, which the runtime stamps when that kernel's dispatch begins
 * and ends, so hipEventElapsedTime(events[2i], events[2i+1]) is the kernel's
 * own duration. The array holds 2n caller-created events (hipEventCreate)
 * that must outlive their use. moe_set_kernel_events(NULL, 0) turns the hook
 * off. Returns MOE_OK, or MOE_ERR_INVALID_ARG for n < 0 or a NULL array with
 * n > 0.
 */
int moe_set_kernel_events(hipEvent_t* events, int n);

/*
 * Status of the bounded waits of the last few-token call made with the
 * workspace `ws`: the layer entry points at T <= 16 tokens run persistent
 * kernels whose workgroups hand data to one another inside a launch and wait
 * for it with a bounded number of polls. If one of those waits gives up
 * (which a correct run never does), the call still finishes with every
 * access in bounds, and the failure shows in the outputs themselves:
 *   - one token (a single launch): every output column group whose inputs
 *     passed through that wait is NaN (all of `out` if the routing's wait
 *     gave up), and if the routing's wait gave up, `topk_ids_out` is -1 and
 *     `topk_w_out` NaN;
 *   - 2..16 tokens: if a wait of an earlier launch gave up, the call's last
 *     launch writes NaN to every element of `out`, -1 to `topk_ids_out` and
 *     NaN to `topk_w_out`; a wait of the last launch itself (2..8 tokens:
 *     its combine's wait for the routed rows) writes NaN to the outputs it
 *     feeds.
 * This call reads the result recorded in the
 * first 16 bytes of `ws` with a blocking device-to-host copy: synchronise
 * the call's stream first, and pass the same workspace before reusing it.
 * Returns MOE_OK (every wait completed, or the last call made with `ws` had
 * no bounded waits), MOE_ERR_TIMEOUT, MOE_ERR_INVALID_ARG (ws NULL) or
 * MOE_ERR_HIP (the copy failed).
 */
int moe_workspace_status(const void* ws);

/*
 * Test hook for the reporting above (never needed in use). While `on` is
 * nonzero, the first bounded wait of the routing in every few-token layer
 * call made from this host thread expects a tag no word carries and gives up
 * after 256 polls; every other wait and kernel runs as usual, so each
 * launch still ends normally. moe_set_wait_test(0) restores normal waits.
 * Returns MOE_OK.
 */
int moe_set_wait_test(int on);

/* Number of kernels the last call from this host thread launched. */
int moe_last_call_launches(void);

/* Name of launch i of that call (static string), or NULL if out of range. */
const char* moe_launch_name(int i);

/*
 * Router: logits, softmax, top-k with renormalised weights.
 * The gate picks k experts per token (ai.rs article, "How 502 GB runs on a
 * 32 GB card": 6 of 384 per layer) and is a discrete switch (same article,
 * "What remains is the reference rounding itself").
 *
 *   x_bf16        [T][H] bf16, 16-byte aligned
 *   w_router_bf16 [E][H] bf16, 16-byte aligned
 *   logit_bias    [E] fp32 added to every token's logits, or NULL
 *   topk_ids      [T][k] int32 out: chosen experts by descending logit;
 *                 exact ties go to the lower expert id
 *   topk_w        [T][k] fp32 out: exp(l_j - l_1) / sum_j' exp(l_j' - l_1),
 *                 i.e. the softmax over all E renormalised over the chosen k
 *   logits_out    [T][E] fp32 out (x W_r^T + bias, fp32 accumulation), or
 *                 NULL to keep them in the workspace
 * Logits accumulate bf16 products exactly in fp32.
 */
int moe_router_topk(const void* x_bf16, const void* w_router_bf16,
                    const float* logit_bias, int T, int H, int E, int k,
                    int32_t* topk_ids, float* topk_w, float* logits_out,
                    void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Bucketing: a stable counting sort of the T*k (token, slot) pairs by
 * expert id, computed with prefix sums and no atomics. Pairs are taken in
 * (token, slot) order, so each expert's rows list its tokens ascending. The
 * pages trace run-to-run differences to slot assignment that depends on
 * timing (ai.rs article, "What remains is the reference rounding itself");
 * this order is a pure function of topk_ids.
 *
 *   topk_ids       [T][k] int32 in
 *   expert_offsets [E+1] int32 out: rows of expert e are
 *                  [expert_offsets[e], expert_offsets[e+1])
 *   row_token      [T*k] int32 out: token of each row
 *   inv_row        [T][k] int32 out: row of pair (t, j)
 * Ids outside [0, E) are dropped: their inv_row entry is -1, they own no
 * row, and expert_offsets[E] counts only valid pairs.
 */
int moe_permute(const int32_t* topk_ids, int T, int k, int E,
                int32_t* expert_offsets, int32_t* row_token, int32_t* inv_row,
                void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Expert FFN over bucketed rows with MXFP4 weights (FreeToken issue #444,
 * "Architecture delta vs deepseek_v4" for the 3 x 5120 x 2304 shape; the
 * SwiGLU form is the reading taken where the pages are silent):
 *   y_rows[r] = W_down[e] (silu(W_gate[e] x_t) * (W_up[e] x_t)),
 *   e = the bucket holding r, t = row_token[r], silu(z) = z / (1 + e^-z).
 * Weights are dequantised exactly; products accumulate in fp32.
 *
 *   x_bf16         [T][H] bf16 activations
 *   bank           routed bank (E experts) or a one-expert bank
 *   expert_offsets [E+1] int32 from moe_permute; NULL only when bank->E == 1,
 *                  meaning rows [0, R)
 *   row_token      [R] int32 in [0, T); NULL means row r reads token r (R <= T).
 *                  Out-of-range entries and offsets are clamped, never read
 *                  or written out of bounds (the affected rows are garbage)
 *   R              number of rows (== expert_offsets[E])
 *   y_rows         [R][H] fp32 out
 * Precision: up to 128 rows, h = silu(g) * u stays in fp32. Above that the
 * rows run on the bf16 / fp16 matrix cores (grouped GEMM), which round h
 * once to fp16 for the down product (about 2e-4 relative error): an |h| of
 * 65520 or more becomes +-inf there, and every output of that row comes out
 * NaN or inf, never finite and wrong. Such magnitudes are far outside the
 * layer's activations (|h| stays below about 10^3 for bf16 N(0,1) tokens and
 * the configs' scales).
 */
int moe_expert_ffn_mxfp4(const void* x_bf16, const moe_mxfp4_bank* bank,
                         const int32_t* expert_offsets, const int32_t* row_token,
                         int T, int R, float* y_rows,
                         void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Weighted combine in a fixed order (the pages tie irreproducible outputs to
 * a varying accumulation order: ai.rs article, "What remains is the
 * reference rounding itself"):
 *   out[t] = y_shared[t] + sum_{j = 0..k-1} topk_w[t][j] * y_rows[inv_row[t][j]]
 * summed in fp32 in the order shown. Pairs with inv_row == -1 add nothing.
 *
 *   y_rows [R][H] fp32; inv_row [T][k]; topk_w [T][k];
 *   y_shared [T][H] fp32 or NULL; out [T][H] fp32 (may not alias inputs).
 *   R is needed to bounds-check inv_row (entries >= R are an error the
 *   kernel turns into a NaN row rather than an out-of-bounds read).
 */
int moe_combine(const float* y_rows, const int32_t* inv_row, const float* topk_w,
                const float* y_shared, int T, int k, int H, int R, float* out,
                hipStream_t stream);

/*
 * The whole layer: router -> top-k -> bucketing -> routed experts and the
 * shared expert -> combine, all enqueued on `stream` with no host sync.
 *
 *   routed         bank of E routed experts (E, H, I taken from it)
 *   shared         one-expert bank added with weight 1, or NULL
 *   out            [T][H] fp32
 *   topk_ids_out   [T][k] int32 or NULL; topk_w_out [T][k] fp32 or NULL
 * Up to 16 tokens every step keeps fp32 (the persistent few-token kernels);
 * more tokens run the grouped GEMM, with h in fp16 as described for
 * moe_expert_ffn_mxfp4 (an out-of-range h gives non-finite rows).
 */
int moe_layer_forward(const void* x_bf16, const void* w_router_bf16,
                      const float* logit_bias, const moe_mxfp4_bank* routed,
                      const moe_mxfp4_bank* shared, int T, int k, float* out,
                      int32_t* topk_ids_out, float* topk_w_out,
                      void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * moe_layer_forward for callers that cannot allocate: code under HIP graph
 * capture, tight serving loops and harnesses that forbid hipMalloc. Same
 * arguments, results, bit patterns and errors as moe_layer_forward, except
 * that there is no workspace argument: the scratch is a 16 MiB array of
 * device memory that the library holds on each GPU it runs on, from its
 * load until the process ends. This call never allocates or frees memory.
 *
 *  - A call whose workspace need (as for moe_layer_forward) exceeds 16 MiB
 *    returns MOE_ERR_WORKSPACE and enqueues nothing. At the real layer shape
 *    (H 5120, I 2304, 384 experts, top-6, a shared expert) every call of up
 *    to 16 tokens fits: decode and verification blocks.
 *  - Every call on one GPU uses that GPU's one array, which keeps the last
 *    call's contents; nothing in it needs clearing between calls. Calls that
 *    overlap on one GPU (other streams, other host threads) race on it and
 *    must be serialised by the caller.
 *  - A bounded in-kernel wait that gives up shows in the outputs as with
 *    moe_layer_forward (NaN out, ids -1); moe_workspace_status cannot read
 *    this array.
 *  - The first call on a device looks up the array's address on that device
 *    (MOE_ERR_HIP if the lookup fails).
 */
int moe_layer_forward_noalloc(const void* x_bf16, const void* w_router_bf16,
                              const float* logit_bias, const moe_mxfp4_bank* routed,
                              const moe_mxfp4_bank* shared, int T, int k, float* out,
                              int32_t* topk_ids_out, float* topk_w_out, hipStream_t stream);

/*
 * One FP8 expert over T rows (the shared expert or a dense SwiGLU FFN in the
 * checkpoint's fp8 format): y[t] = W_down (silu(W_gate x_t) * (W_up x_t)),
 * weights dequantised exactly (E4M3 times a power of two), products summed
 * in fp32. x_bf16 [T][H] bf16, y [T][H] fp32, both 16-byte aligned; bank->E
 * must be 1. moe_workspace_bytes(T, H, I, 1, 1) suffices.
 */
int moe_expert_ffn_fp8(const void* x_bf16, const moe_fp8_bank* bank, int T, float* y,
                       void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * moe_layer_forward with the shared expert in the FP8 format above (the
 * reference checkpoint's layout: FP4 routed experts, FP8 dense weights;
 * FreeToken issue #444, "Is the quantization already supported"). Routing, routed experts,
 * ordering and determinism are those of moe_layer_forward; the shared row
 * is added first in the combine, with weight 1. `shared` is required.
 * moe_workspace_bytes covers its workspace.
 */
int moe_layer_forward_fp8_shared(const void* x_bf16, const void* w_router_bf16,
                                 const float* logit_bias, const moe_mxfp4_bank* routed,
                                 const moe_fp8_bank* shared, int T, int k, float* out,
                                 int32_t* topk_ids_out, float* topk_w_out,
                                 void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * moe_expert_ffn_mxfp4 for an NVFP4 bank: same arguments, buckets, limits and
 * errors. Weights are dequantised exactly (E2M1 x E4M3 is exact in bf16 and
 * fp16); the matrix scale multiplies the fp32 sums.
 */
int moe_expert_ffn_nvfp4(const void* x_bf16, const moe_nvfp4_bank* bank,
                         const int32_t* expert_offsets, const int32_t* row_token,
                         int T, int R, float* y_rows,
                         void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * moe_layer_forward with NVFP4 routed experts and, optionally, an NVFP4
 * shared expert (E = 1). Routing, bucketing, ordering and determinism are
 * those of moe_layer_forward. Every T runs the separate router, top-k,
 * bucketing, expert and combine launches (the fused few-token launches take
 * MXFP4 banks only). moe_workspace_bytes covers its workspace.
 */
int moe_layer_forward_nvfp4(const void* x_bf16, const void* w_router_bf16,
                            const float* logit_bias, const moe_nvfp4_bank* routed,
                            const moe_nvfp4_bank* shared, int T, int k, float* out,
                            int32_t* topk_ids_out, float* topk_w_out,
                            void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Opt-in mode with MXFP8 activations on the scaled matrix cores.
 *
 * The reference model runs its linear layers in fp8 with block scales and
 * activations rounded on the fly (FreeToken issue #444, "Is the quantization
 * already supported": a dynamic activation scheme with ue8m0 scales); the pages
 * also tabulate what that rounding costs against full precision, about
 * 1.45 % relative error for one fp8 linear layer (ai.rs article on
 * DeepSeek-V4.1-Flash, "What remains is the reference rounding itself").
 * This mode takes the same kind of rounding for the expert FFNs so that the
 * gfx950 scaled MFMA can multiply E4M3 activations by the bank's E2M1 codes
 * as stored (no weight conversion). It is an approximation of the layer,
 * not the layer: its results differ from moe_layer_forward by the
 * activation rounding, a few percent relative, and it is selected only by
 * calling the entry points below.
 *
 * The rounding (OCP Microscaling v1.0 conversion, the reading taken where
 * the pages are silent): per block of 32 consecutive values, scale byte
 * s = clamp(floor(log2(max |v|)) - 8, -127, 127) + 127 (an all-zero block
 * takes s = 0); each value v becomes the E4M3 code nearest to
 * v / 2^(s - 127), ties to even, magnitudes above 448 clamped to 448, the
 * sign kept (a negative value that rounds to zero gives 0x80).
 */

/*
 * MXFP8 rounding of bf16 rows: codes[t][h] (E4M3 byte) and
 * scales[t][h / 32] (E8M0 byte) of x_bf16 [T][H]. H a multiple of 32;
 * x_bf16 and codes 16-byte aligned. Bitwise a pure function of x.
 */
int moe_quantize_mxfp8(const void* x_bf16, int T, int H, uint8_t* codes, uint8_t* scales,
                       hipStream_t stream);

/*
 * moe_layer_forward in the MXFP8-activation mode. Arguments, ownership,
 * ordering, determinism and the routing (router, top-k, weights and
 * bucketing on the exact bf16 x) are those of moe_layer_forward. The expert
 * FFNs of the routed and the shared expert take x rounded to MXFP8 per row
 * (blocks of 32 along H) and round h = silu(g) * u to MXFP8 per row (blocks
 * of 32 along I) before the down product; every product sums in fp32. Every
 * T runs the grouped GEMM (the mode is meant for prefill).
 * Needs H and I multiples of 256 and 128, H, I <= 8192, T*H < 2^31 and
 * (T*k + T)*I < 2^31, else MOE_ERR_UNSUPPORTED. moe_workspace_bytes covers
 * its workspace.
 */
int moe_layer_forward_mxfp8_act(const void* x_bf16, const void* w_router_bf16,
                                const float* logit_bias, const moe_mxfp4_bank* routed,
                                const moe_mxfp4_bank* shared, int T, int k, float* out,
                                int32_t* topk_ids_out, float* topk_w_out,
                                void* ws, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MXFP4_H */
