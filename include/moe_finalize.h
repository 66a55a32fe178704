/*
 * moe_finalize.h -- C ABI of the MI355X (gfx950) MoE finalize library, libmoe_finalize.so.
 *
 * Sources (cited by key):
 *   [FI6631]  flashinfer PR #6631, "perf(comm): gather MoE-finalize routes together and accumulate
 *             in FP32": Description, test changes, benchmark script, review walkthrough.
 *   [TR16778] TensorRT-LLM PR #16778, "MoE: fp32 accumulation in deferred MoEAllReduce finalize":
 *             Description / Fix.
 *   [FI6546]  flashinfer PR #6546, small-batch trtllm-gen MoE finalize: Description.
 *   [FI3385]  flashinfer PR #3385, "feat: MNNVL Allreduce quant fusion and performance
 *             optimization": walkthrough and review comments.
 *
 * What is computed, for token t < T and hidden element h < H ([FI6631] Description and the FP64
 * reference of its benchmark script; [TR16778] Fix):
 *   route k of token t is present iff 0 <= p = expanded_idx_to_permuted_idx[t*K + k] < N_rows;
 *   acc  = sum over present k of w[t,k] * X[p, h]        (float32 accumulation)
 *   s    = RNE_T(RSF * acc + shared[t, h])               (the one rounding to the activation dtype)
 *   r    = RNE_T(s + residual[t, h])                     (residual_out)
 *   norm = RNE_T(r * gamma[h] / sqrt(mean_h(r^2) + eps))  (norm_out; RMSNorm of the rounded r)
 * optionally followed by NVFP4 or FP8-E4M3 quantization of norm ([FI3385] walkthrough).
 *
 * Conventions shared by every entry point:
 *   - Memory. Every array argument is caller-owned DEVICE memory on the current HIP device,
 *     row-major and dense (leading dimension = the row length given). The library allocates
 *     nothing per call and keeps no pointer after it returns.
 *   - Streams. `stream` is a hipStream_t (NULL = the default stream). Calls only enqueue work and
 *     return; they never synchronize, so they can be captured into a HIP graph.
 *   - dtypes. act_dtype is MOE_DTYPE_BF16 or MOE_DTYPE_FP16 and types X, shared, residual,
 *     gamma and every activation output. scales_dtype is MOE_DTYPE_FP32 or MOE_DTYPE_BF16.
 *   - Optional inputs. expert_scales == NULL means weight 1.0; shared_expert_output == NULL means
 *     no shared term; routed_scaling_factor 1.0 means "off" ([FI6631] review summary and commit
 *     notes: missing scales handled, the factor is 1.0 when off).
 *   - Absent routes. Any index outside [0, num_permuted_rows) (-1 marks "no route",
 *     [FI6631] test changes) contributes nothing; neither its row nor its scale is read. An index
 *     is never an error and never faults.
 *   - Alignment. X, shared, residual, gamma and every output must be 16-byte aligned
 *     (128-bit loads, [FI6546] Description; the vector-width guard of [FI3385] review), idx and
 *     fp32 scales 4-byte, bf16 scales 2-byte. hidden must be a multiple of 8 (16 for NVFP4).
 *   - Limits. 1 <= top_k <= 64 ([FI6546] Description: the small-batch rule admits topK <= 64);
 *     num_tokens >= 0 (0 is a successful no-op); num_permuted_rows >= 0.
 *   - Aliasing. Outputs may not overlap inputs or each other, except residual_out == residual
 *     (exactly the same pointer) for an in-place residual update.
 *   - Errors. 0 on success, a negative MOE_FIN_ERR_* code otherwise. Nothing is enqueued when a
 *     check fails. No exception or abort crosses the ABI. moe_finalize_error_string() names a code.
 *   - Determinism. Results are bitwise reproducible run to run and under graph capture/replay.
 *   - Workspace (RMSNorm entry points). With workspace == NULL each token's row is handled by one
 *     workgroup. With a workspace, a row may be spread over several workgroups that exchange
 *     their partial sums of squares through it (summed in a fixed slice order, so results do
 *     not depend on timing; the sum of squares is associated differently from the whole-row
 *     kernel, so norm_out may differ from the NULL-workspace result in the last bit). It is
 *     caller-owned device memory of at least moe_finalize_workspace_size(...) bytes, 256-byte
 *     aligned, ZERO-FILLED ONCE before its first use; every call leaves it ready for the next
 *     (no per-call clearing, so graph replays need no memset node). Calls that may run at the
 *     same time (different streams) must use different workspaces. Its first 32-bit word is a
 *     sticky flag that a kernel sets to nonzero if a workgroup gave up waiting for the other
 *     slices of its row; it stays 0 in normal use. A workgroup that gives up counts the missing
 *     partial sums as NaN, so its part of that token's norm_out is NaN (FP8 codes 0x7F; NVFP4
 *     block scales 0x7F with zero codes) instead of a wrong finite value; residual_out is not
 *     affected. No reset is needed afterwards (a workgroup that starts late still finds its row's
 *     partials, and the next call works normally); the flag stays set until the caller clears it.
 *     Progress: a token's slices are consecutive workgroups and rows are split only while the
 *     grid stays near one workgroup per compute unit of the current device (its count is
 *     queried once per device), so workgroups dispatched before a waiting one never wait on it
 *     (the scale-padding workgroups of an NVFP4 call come last and wait on nothing) and the
 *     slices of a row run together. The wait is bounded (about a second, see
 *     moe_finalize_set_wait_limit) even if other work were to hold every CU; the flag and the
 *     NaN outputs then report it.
 */
#ifndef MOE_FINALIZE_H_
#define MOE_FINALIZE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define MOE_FIN_OK 0
#define MOE_FIN_ERR_NULL_POINTER (-1)   /* a required pointer is NULL                      */
#define MOE_FIN_ERR_BAD_SHAPE (-2)      /* negative count, or a size that overflows         */
#define MOE_FIN_ERR_BAD_TOPK (-3)       /* top_k outside [1, 64]                            */
#define MOE_FIN_ERR_HIDDEN (-4)         /* hidden <= 0, not a multiple of 8 (16 for NVFP4)  */
#define MOE_FIN_ERR_ALIGNMENT (-5)      /* a pointer is not aligned as required             */
#define MOE_FIN_ERR_DTYPE (-6)          /* unknown act_dtype / scales_dtype                 */
#define MOE_FIN_ERR_QUANT_TYPE (-7)     /* unknown quant_type                               */
#define MOE_FIN_ERR_SF_LAYOUT (-8)      /* scale layout not LINEAR or SWIZZLED_128x4        */
#define MOE_FIN_ERR_ALIAS (-9)          /* forbidden overlap between buffers                */
#define MOE_FIN_ERR_HIP (-10)           /* the HIP runtime refused the launch               */
#define MOE_FIN_ERR_WORKSPACE (-11)     /* workspace smaller than moe_finalize_workspace_size */
#define MOE_FIN_ERR_POLICY (-12)        /* unknown cache policy                             */
#define MOE_FIN_ERR_SCRATCH (-13)       /* num_tokens above the static scratch's 1024       */

/* Element types. */
#define MOE_DTYPE_BF16 0
#define MOE_DTYPE_FP16 1
#define MOE_DTYPE_FP32 2

/* Quantized output of moe_finalize_quant_run ([FI3385] walkthrough: FP8 and NVFP4 outputs). */
#define MOE_QUANT_NVFP4 1
#define MOE_QUANT_FP8_E4M3 2

/* NVFP4 block-scale layouts ([FI3385] review: only LINEAR and SWIZZLED_128x4 are accepted). */
#define MOE_SF_LINEAR 0
#define MOE_SF_SWIZZLED_128x4 1

/*
 * moe_finalize_run -- the finalize alone (gather, float32 weighted sum, routed scaling, shared
 * add, one rounding): out[t, h] = s as defined above. This is the op of [FI6546] Description
 * (the trtllm-gen finalize) with the float32 accumulation of [FI6631] / [TR16778].
 *
 *   permuted_rows         [num_permuted_rows, hidden] act_dtype: expert GEMM2 output rows.
 *   expanded_idx_to_permuted_idx [num_tokens, top_k] int32: entry (t, k) is the permuted row of
 *                          expanded index t*top_k + k; out of range (e.g. -1) = no route.
 *   expert_scales         [num_tokens, top_k] scales_dtype, or NULL (weight 1.0).
 *   shared_expert_output  [num_tokens, hidden] act_dtype, or NULL.
 *   out                   [num_tokens, hidden] act_dtype.
 */
int moe_finalize_run(const void* permuted_rows, int64_t num_permuted_rows,
                     const int32_t* expanded_idx_to_permuted_idx,
                     const void* expert_scales, int scales_dtype,
                     const void* shared_expert_output, float routed_scaling_factor,
                     void* out,
                     int64_t num_tokens, int64_t hidden, int top_k, int act_dtype,
                     void* stream);

/*
 * moe_finalize_rmsnorm_run -- finalize, then residual add and RMSNorm on the rounded sum
 * ([FI6631] Description: the residual add and RMSNorm work on the rounded sum; its benchmark
 * script: mean of squares over hidden, eps inside the square root, then times gamma).
 *
 *   residual      [num_tokens, hidden] act_dtype.
 *   gamma         [hidden] act_dtype (RMSNorm weight).
 *   eps           added to the mean of squares inside the square root.
 *   residual_out  [num_tokens, hidden] act_dtype, or NULL (not written); may equal `residual`.
 *   norm_out      [num_tokens, hidden] act_dtype.
 *   workspace, workspace_bytes  see "Workspace" above (NULL, 0 allowed).
 * Other arguments as in moe_finalize_run.
 */
int moe_finalize_rmsnorm_run(const void* permuted_rows, int64_t num_permuted_rows,
                             const int32_t* expanded_idx_to_permuted_idx,
                             const void* expert_scales, int scales_dtype,
                             const void* shared_expert_output, float routed_scaling_factor,
                             const void* residual, const void* gamma, float eps,
                             void* residual_out, void* norm_out,
                             void* workspace, size_t workspace_bytes,
                             int64_t num_tokens, int64_t hidden, int top_k, int act_dtype,
                             void* stream);

/*
 * moe_finalize_rmsnorm_noalloc_run -- moe_finalize_rmsnorm_run for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation, kernels and results, with no workspace argument. It calls
 * no allocating routine; the split-row exchange uses a static scratch array inside the library,
 * 131,328 bytes per device (256 + 128 per token for up to 1024 tokens), which each GPU the
 * library runs on holds until the process ends. The first call on a device also enqueues, ahead
 * of its own work on `stream`, one small kernel that zeroes that device's scratch.
 *   num_tokens  0..1024; more gives MOE_FIN_ERR_SCRATCH (nothing is enqueued).
 * All calls on one device share its scratch, which keeps the last call's exchange words: calls
 * that may overlap on one device (different streams, or threads) race and must not be made;
 * calls in order on one stream need no reset, and a timed-out call needs none either (see
 * "Workspace"). The timeout flag lives in the scratch and is not readable by the caller; a
 * timed-out call still shows as NaN norm_out. Other arguments, errors and results exactly as
 * moe_finalize_rmsnorm_run with a workspace (bit-identical outputs).
 */
int moe_finalize_rmsnorm_noalloc_run(const void* permuted_rows, int64_t num_permuted_rows,
                                     const int32_t* expanded_idx_to_permuted_idx,
                                     const void* expert_scales, int scales_dtype,
                                     const void* shared_expert_output,
                                     float routed_scaling_factor, const void* residual,
                                     const void* gamma, float eps, void* residual_out,
                                     void* norm_out, int64_t num_tokens, int64_t hidden,
                                     int top_k, int act_dtype, void* stream);

/*
 * moe_finalize_workspace_flag -- host query of a workspace's timeout flag (see "Workspace"):
 * *flag = its first 32-bit word, nonzero if a split-row wait of an earlier call gave up. With
 * workspace == NULL, the flag of the current device's static scratch of
 * moe_finalize_rmsnorm_noalloc_run (0 if that entry point has not run on the device). clear != 0
 * also resets a set flag to zero (a 16-byte fill kernel on `stream`; the split-row slots need
 * no reset). Enqueues a 4-byte copy on `stream` and waits for that stream, so the calls before
 * it on the stream are counted; a diagnostic for the host, not for a captured graph. Errors:
 * MOE_FIN_ERR_NULL_POINTER (flag), MOE_FIN_ERR_ALIGNMENT (workspace not 256-byte aligned),
 * MOE_FIN_ERR_HIP.
 */
int moe_finalize_workspace_flag(const void* workspace, int clear, int* flag, void* stream);

/*
 * moe_finalize_quant_run -- moe_finalize_rmsnorm_run followed by quantization of norm
 * ([FI3385] walkthrough: FP8 / NVFP4 quantized outputs with an output scale and a layout code;
 * [FI6631] test changes: the NVFP4 scale buffer is sized for SWIZZLED_128x4).
 *
 *   quant_type   MOE_QUANT_NVFP4 or MOE_QUANT_FP8_E4M3.
 *   quant_scale  device pointer to ONE float32: the per-tensor global scale gs (NVFP4) or the
 *                FP8 scale s8, positive and finite (as the pages' per-tensor scales 448*6/amax
 *                and 448/amax are; it is read on the device, so it is not checked: for a zero,
 *                negative or non-finite scale the codes are not specified, and the call still
 *                completes without touching memory outside its outputs). NVFP4: for every 16-element block of a row, sf = E4M3(gs*amax/6)
 *                and codes q = E2M1(x*gs/sf) (signed zeros when sf == 0). FP8: q = E4M3(x*s8).
 *                All conversions round to nearest even and saturate (E4M3 at 448, E2M1 at 6;
 *                infinities saturate too); every code equals the rounding of the exact real
 *                product or quotient, not of a float32 approximation of it, ties included.
 *                Non-finite values: an FP8 NaN is 0x7F whatever its
 *                sign; an NVFP4 block holding a NaN gets scale code 0x7F and all codes 0.
 *   quant_out    NVFP4: [num_tokens, hidden/2] bytes, element 2j in the low nibble of byte j.
 *                FP8:   [num_tokens, hidden] bytes.
 *   scale_out    NVFP4 only (else ignored, may be NULL): moe_finalize_sf_size(...) bytes of E4M3
 *                block scales in `sf_layout`; every padding byte is written as 0.
 *   sf_layout    MOE_SF_SWIZZLED_128x4 or MOE_SF_LINEAR (NVFP4 only).
 *   residual_out as in moe_finalize_rmsnorm_run (nullable).
 *   norm_out     [num_tokens, hidden] act_dtype, or NULL (then the unquantized norm is not stored).
 *   workspace, workspace_bytes  see "Workspace" above (NULL, 0 allowed).
 * Other arguments as in moe_finalize_rmsnorm_run.
 */
int moe_finalize_quant_run(const void* permuted_rows, int64_t num_permuted_rows,
                           const int32_t* expanded_idx_to_permuted_idx,
                           const void* expert_scales, int scales_dtype,
                           const void* shared_expert_output, float routed_scaling_factor,
                           const void* residual, const void* gamma, float eps,
                           int quant_type, const float* quant_scale,
                           void* quant_out, void* scale_out, int sf_layout,
                           void* residual_out, void* norm_out,
                           void* workspace, size_t workspace_bytes,
                           int64_t num_tokens, int64_t hidden, int top_k, int act_dtype,
                           void* stream);

/*
 * moe_finalize_workspace_size -- bytes of workspace the RMSNorm entry points may use for a call
 * with this shape (256 + 128 per token). Host-only. Returns 0 for num_tokens < 0.
 */
size_t moe_finalize_workspace_size(int64_t num_tokens, int64_t hidden, int top_k);

/*
 * moe_quantize_run -- NVFP4 or FP8-E4M3 quantization of a given [num_tokens, hidden] activation
 * tensor x (act_dtype), with exactly the encoder of moe_finalize_quant_run (same definitions,
 * layouts, rounding and saturation; see there). Applied to a precomputed norm_out it is the
 * quantize step of [FI3385] walkthrough on its own (the standalone RMSNorm + quant pattern);
 * it also lets a caller quantize values produced elsewhere.
 *   x           [num_tokens, hidden] act_dtype, 16-byte aligned.
 *   quant_scale device pointer to one float32 (gs for NVFP4, s8 for FP8).
 *   quant_out   NVFP4 [num_tokens, hidden/2] bytes | FP8 [num_tokens, hidden] bytes.
 *   scale_out   NVFP4: moe_finalize_sf_size(num_tokens, hidden, sf_layout) bytes (padding written
 *               as 0); ignored for FP8.
 * Errors as for moe_finalize_quant_run; hidden must be a multiple of 16 (NVFP4) or 8 (FP8).
 */
int moe_quantize_run(const void* x, int64_t num_tokens, int64_t hidden, int act_dtype,
                     int quant_type, const float* quant_scale, void* quant_out, void* scale_out,
                     int sf_layout, void* stream);

/*
 * moe_residual_rmsnorm_run -- the residual add and RMSNorm of moe_finalize_rmsnorm_run on a given
 * activation x instead of a finalize result: r = RNE_T(x + residual), norm = RNE_T(r * gamma /
 * sqrt(mean_h(r^2) + eps)). This is the separate residual + RMSNorm kernel that the fused
 * finalize is measured against ([FI6631] Related Issues: fused finalize versus finalize
 * followed by a residual + RMSNorm kernel) and the residual + RMSNorm stage of an all-reduce
 * fusion ([FI3385] Description). Runs on the finalize kernel with one route per token (row t of
 * x, weight 1), routed scaling 1 and no shared term, which reproduces x exactly.
 *
 *   x             [num_tokens, hidden] act_dtype, 16-byte aligned.
 *   residual, gamma, eps, residual_out, norm_out, workspace, workspace_bytes
 *                 as in moe_finalize_rmsnorm_run (residual_out may equal residual; it may not
 *                 overlap x).
 * Errors as for moe_finalize_rmsnorm_run (top_k checks do not apply).
 */
int moe_residual_rmsnorm_run(const void* x, const void* residual, const void* gamma, float eps,
                             void* residual_out, void* norm_out,
                             void* workspace, size_t workspace_bytes,
                             int64_t num_tokens, int64_t hidden, int act_dtype, void* stream);

/*
 * moe_rank_sum_rmsnorm_run -- one GPU's share of the cross-rank reduction that the pages fuse
 * between the finalize and the residual + RMSNorm ([FI6631] Description: the per-rank finalized
 * partials are summed in float32 and rounded once before the residual add and RMSNorm;
 * [FI3385] commit notes: every rank accumulates the ranks in the same fixed order). Given the
 * world_size partial rows that the ranks' finalize calls produced for the same tokens (already
 * gathered into this GPU's memory by the transport, which is not part of this library):
 *   s    = RNE_T(sum over r of partial[r, t, h])        (float32 sum, one rounding)
 *   r, norm as in moe_finalize_rmsnorm_run.
 * It is moe_finalize_rmsnorm_run with one route per rank (row r*T + t, weight 1), routed scaling
 * 1 and no shared term, so the sum follows the same fixed, timing-independent order on every
 * rank and call, and every result lies in the same float32 window as the finalize's.
 *
 *   rank_partials  [world_size, num_tokens, hidden] act_dtype, 16-byte aligned: rank r's rows.
 *   world_size     1..64 (MOE_FIN_ERR_BAD_TOPK otherwise); world_size * num_tokens <= 2^31 - 1.
 *   residual, gamma, eps, residual_out, norm_out, workspace, workspace_bytes
 *                  as in moe_finalize_rmsnorm_run (outputs may not overlap rank_partials).
 */
int moe_rank_sum_rmsnorm_run(const void* rank_partials, int world_size, const void* residual,
                             const void* gamma, float eps, void* residual_out, void* norm_out,
                             void* workspace, size_t workspace_bytes, int64_t num_tokens,
                             int64_t hidden, int act_dtype, void* stream);

/*
 * moe_rank_sum_quant_run -- moe_rank_sum_rmsnorm_run followed by the NVFP4 / FP8 quantization of
 * moe_finalize_quant_run (same arguments and conventions as there; norm_out nullable).
 */
int moe_rank_sum_quant_run(const void* rank_partials, int world_size, const void* residual,
                           const void* gamma, float eps, int quant_type, const float* quant_scale,
                           void* quant_out, void* scale_out, int sf_layout, void* residual_out,
                           void* norm_out, void* workspace, size_t workspace_bytes,
                           int64_t num_tokens, int64_t hidden, int act_dtype, void* stream);

/*
 * moe_finalize_sf_size -- bytes of the NVFP4 block-scale buffer for a [num_tokens, hidden]
 * output: SWIZZLED_128x4 pads rows to a multiple of 128 and blocks per row to a multiple of 4,
 * roundup(T,128) * roundup(H/16,4) ([FI6631] test changes: T*H/16 bytes is too small and was
 * overrun); LINEAR is T * H/16. Returns 0 for an unknown layout or a negative size.
 * Host-only, never touches the GPU.
 */
size_t moe_finalize_sf_size(int64_t num_tokens, int64_t hidden, int sf_layout);

/*
 * moe_finalize_launch_floor_run -- measurement aid: enqueue an EMPTY kernel with exactly the grid,
 * block and LDS size that entry point `entry` (0 = moe_finalize_run, 1 = moe_finalize_rmsnorm_run,
 * 2 = moe_finalize_quant_run, the RMSNorm ones with a workspace) would use for this shape. Its
 * time per launch is the launch-latency
 * floor the small-batch (T <= 16) timings are reported against. Reads and writes no memory.
 * Returns the validation codes of the entry point for bad shapes (an unknown `entry` gives
 * MOE_FIN_ERR_QUANT_TYPE).
 */
int moe_finalize_launch_floor_run(int entry, int64_t num_tokens, int64_t hidden, int top_k,
                                  void* stream);

/*
 * moe_finalize_launch_config -- the launch configuration entry point `entry` (0 =
 * moe_finalize_run, 1 = moe_finalize_rmsnorm_run, 2 = moe_finalize_quant_run) chooses for a shape,
 * with (with_workspace != 0) or without a workspace, on a device of `num_cus` compute units
 * (num_cus <= 0: the current device's count, which only this case queries; with a workspace the
 * slice rule depends on it). Host-only; launches nothing. Writes MOE_FIN_LAUNCH_CONFIG_FIELDS
 * int64 values to `out` (n_out is the caller's array length):
 *   out[0] workgroups in the grid (0 when num_tokens == 0): num_tokens * out[2], or for split
 *          rows with cacheable accesses (out[7] == 0) ceil(num_tokens / 8) * 8 * out[2] (the
 *          slices of a token share one of the 8 XCDs, and the workgroups of the padding tokens
 *          exit at once); a swizzled NVFP4 call whose
 *          num_tokens is not a multiple of 128 adds a few workgroups after these that only
 *          zero the scale bytes of the padding rows
 *   out[1] lanes per workgroup (route groups x lanes per group, a multiple of 64, <= 1024)
 *   out[2] workgroups per token for the RMSNorm entries (slices of a split row; 1 = whole rows)
 *   out[3] route groups G (wavefront groups that split top_k; partials combined in LDS)
 *   out[4] 8-element slots per lane P
 *   out[5] slots covered by one workgroup
 *   out[6] dynamic LDS bytes
 *   out[7] 1 when the streamed accesses are nontemporal (see moe_finalize_set_cache_policy)
 *   out[8] 1 when the library holds a kernel for this configuration
 * Returns the entry point's shape-validation code (an unknown `entry` gives
 * MOE_FIN_ERR_QUANT_TYPE), MOE_FIN_ERR_NULL_POINTER for out == NULL, MOE_FIN_ERR_BAD_SHAPE when
 * n_out < MOE_FIN_LAUNCH_CONFIG_FIELDS, MOE_FIN_ERR_HIP when num_cus <= 0 and the device count
 * cannot be queried.
 */
#define MOE_FIN_LAUNCH_CONFIG_FIELDS 9

/*
 * moe_finalize_set_cache_policy -- how later calls of every entry point, from any thread, treat
 * the tensors they stream (permuted rows, shared output and residual loads; residual_out and
 * norm_out stores; gamma and the route metadata always stay cacheable):
 *   MOE_FIN_CACHE_AUTO    (default) nontemporal from 4 MiB of permuted rows per call
 *                         (num_tokens * top_k * hidden * 2 bytes), cacheable below;
 *   MOE_FIN_CACHE_KEEP    always cacheable: for inputs that are already in the caches, or a
 *                         pipeline whose next kernel reads residual_out / norm_out at once;
 *   MOE_FIN_CACHE_STREAM  always nontemporal: for inputs that come from HBM.
 * moe_finalize_run never stores its output nontemporally. Results are bit-identical under every
 * policy. The policy is read when a call is enqueued, so a captured graph keeps the choice made
 * at capture. Returns the previous policy, or MOE_FIN_ERR_POLICY for an unknown value (the
 * policy is then unchanged). Besides the wait limit below, this is the library's only
 * process-wide setting.
 */
#define MOE_FIN_CACHE_AUTO 0
#define MOE_FIN_CACHE_KEEP 1
#define MOE_FIN_CACHE_STREAM 2
int moe_finalize_set_cache_policy(int policy);
int moe_finalize_launch_config(int entry, int64_t num_tokens, int64_t hidden, int top_k,
                               int with_workspace, int num_cus, int64_t* out, int n_out);

/*
 * moe_finalize_set_wait_limit -- how many times a workgroup of a split row polls for the other
 * slices' partial sums before it gives up (sets the workspace flag and writes NaN, see
 * "Workspace"). polls < 0 restores the default (4194304 polls, about 0.1-0.5 s); values above
 * 2^32 - 1 are clamped. 0 makes every split-row wait give up at once, which lets a caller check
 * its handling of a timed-out call without any GPU fault or hang. Process-wide, read when a
 * call is enqueued (a captured graph keeps the limit of its capture). Host-only. Returns the
 * previous limit.
 */
int64_t moe_finalize_set_wait_limit(int64_t polls);

/*
 * moe_finalize_stream_floor_run -- measurement aid: read `read_bytes` from `src` and write
 * `write_bytes` to `dst` in ONE kernel launch that does nothing else, the way an ideal finalize
 * would move its bytes (every 128-bit load of a lane issued before any is used, nontemporal loads
 * and stores). Its time per launch is the streaming ceiling for that many bytes in one launch on
 * this device, which the finalize timings are compared against beside the HBM peak.
 *   src  device memory, 16-byte aligned, read_bytes bytes (may be NULL if read_bytes == 0).
 *   dst  device memory, 16-byte aligned, write_bytes bytes, overlapping no part of src. Content
 *        written: with L = 1024 * 512 lanes, 16-byte chunk j of dst is the XOR of the chunks c of
 *        src with c % L == j % L (chunks past the end read as 0).
 * It is moe_finalize_stream_probe_run with 1 load per round, 1024 workgroups of 512 lanes and
 * nontemporal accesses: the fastest shape of a launch-shape sweep on MI355X at 9.2 and 18.4 MB.
 * read_bytes and write_bytes must be multiples of 16 and at most 2^31. Errors:
 * MOE_FIN_ERR_BAD_SHAPE, MOE_FIN_ERR_NULL_POINTER, MOE_FIN_ERR_ALIGNMENT, MOE_FIN_ERR_ALIAS,
 * MOE_FIN_ERR_HIP. Both sizes 0 is a successful no-op.
 */
int moe_finalize_stream_floor_run(const void* src, size_t read_bytes, void* dst,
                                  size_t write_bytes, void* stream);

/*
 * moe_finalize_stream_probe_run -- measurement aid: the stream kernel of
 * moe_finalize_stream_floor_run with its launch shape chosen by the caller, to find the fastest
 * single launch that moves a given number of bytes. `workgroups` workgroups of `workgroup_lanes`
 * lanes (64, 128, 256, 512 or 1024; L = workgroups * workgroup_lanes lanes in all) read src in
 * rounds of `loads_per_round` 128-bit loads per lane in flight (1, 2, 4, 8 or 16): lane l reads
 * every chunk c with c % L == l. 16-byte chunk j of dst is the XOR of the chunks c of src with
 * c % L == j % L. nontemporal != 0 marks every access nontemporal. Other arguments, limits and
 * errors as moe_finalize_stream_floor_run (1 <= workgroups <= 65536, else MOE_FIN_ERR_BAD_SHAPE).
 */
int moe_finalize_stream_probe_run(const void* src, size_t read_bytes, void* dst,
                                  size_t write_bytes, int loads_per_round, int workgroup_lanes,
                                  int64_t workgroups, int nontemporal, void* stream);

/* Static, NUL-terminated description of a return code. Host-only. */
const char* moe_finalize_error_string(int code);

/* Library version (major*10000 + minor*100 + patch). Host-only. */
int moe_finalize_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_FINALIZE_H_ */
