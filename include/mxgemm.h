/*
 * mxgemm.h - C ABI of libmxgemm, the MI355X (gfx950) block-scaled linear layer.
 *
 * The layer is the attention output projection of "Kimi-K3 DSpark O-Proj-only
 * MXFP4" (section "Exact quantization coverage"): weight stored (out, in) =
 * (7168, 8192) as MXFP4 - E2M1 elements, one E8M0 scale per 32 consecutive
 * input-channel values, scales (7168, 256) - run with dynamic MXFP4
 * activations through an A4W4 GEMM.  Its sibling is the PTPC FP8 scheme of
 * "Kimi-K3-DSpark-FP8-PTPC" (section "Phase 1 FP8 PTPC Quantization"): E4M3
 * weights with an FP32 per-output-channel scale (out_features, 1) and dynamic
 * per-token FP8 activations computed online.
 *
 * Conventions for every entry point
 *   - Pointers are DEVICE pointers to caller-owned, contiguous, row-major
 *     buffers.  The library never allocates device memory, keeps no state
 *     between calls and never synchronizes the host: every call only enqueues
 *     kernels on `stream` (a hipStream_t; NULL is the default stream) and
 *     returns, so calls can be captured into a HIP graph.
 *   - Shapes: X is [M, K] (tokens x in), W is [N, K] (out x in), Y = X . W^T is
 *     [M, N]; there is no bias.  M, N >= 0; M == 0 or N == 0 is a successful
 *     no-op that enqueues nothing.
 *   - Packed MXFP4 codes are [rows, K/2] bytes: element 2j in the low nibble of
 *     byte j, element 2j+1 in the high nibble; E2M1 code = sign<<3 | exp<<1 |
 *     man.  E8M0 scales are [rows, K/32] bytes, value 2^(s-127), 0xFF = NaN.
 *     E4M3 codes are OCP float8_e4m3fn bytes (max 448, 0x7F/0xFF = NaN).
 *     BF16 is the upper half of an IEEE binary32.
 *   - Numeric rules (the pages name "OCP MXFP4" - "Kimi-K3-Quark-MXFP4-AttnFP8",
 *     section "Model Quantization" - but leave the details open; these are the
 *     readings taken):
 *       MX block: e = max(floor(log2(max|x|)) - 2, -127), scale byte e + 127;
 *       element = round-to-nearest-even(x / 2^e) on {0,.5,1,1.5,2,3,4,6},
 *       saturating at 6, sign kept (negative zero results encode as 0x8); an
 *       all-zero block gets scale 0x00; a block with NaN/Inf gets scale 0xFF and
 *       codes 0.
 *       PTPC row: a = max|x|, s = fl32(a / 448) (s = 1 when a == 0),
 *       code = E4M3fn round-to-nearest-even of fl32(x / s), saturating at 448;
 *       a row with NaN/Inf gets s = NaN and every code 0x7F.
 *       GEMMs accumulate in FP32 and round the result to BF16 (nearest even):
 *       a result beyond BF16's finite range becomes +-inf, one in or below its
 *       subnormal range rounds gradually (to +-0 below 2^-134).  The A8W8
 *       epilogue multiplies the FP32 sum by both FP32 scales in FP64.
 *   - Errors: argument errors are detected on the host before anything is
 *     enqueued and returned as an mx_status; a launch failure returns
 *     MX_ERROR_LAUNCH.  Faults during asynchronous execution surface on the
 *     stream.  No C++ exception crosses this interface.
 *   - Outputs must not alias inputs (not checked).
 */
#ifndef MXGEMM_H
#define MXGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MX_SUCCESS = 0,
    MX_ERROR_INVALID_VALUE = 1,     /* NULL pointer with a non-empty shape, negative size */
    MX_ERROR_UNSUPPORTED_SHAPE = 2, /* K outside the rules stated per entry point        */
    MX_ERROR_MISALIGNED = 3,        /* a pointer misses the alignment stated per entry    */
    MX_ERROR_WORKSPACE = 4,         /* workspace smaller than the size query returned     */
    MX_ERROR_LAUNCH = 5,            /* the HIP runtime refused a kernel launch            */
    MX_ERROR_DEVICE = 6             /* the current device is not a gfx950 GPU             */
} mx_status;

/* Version of this interface (incremented on any ABI change). */
int mx_abi_version(void);

/* Static string naming a status code (never NULL). */
const char *mx_status_string(mx_status status);

/*
 * Dynamic per-token MXFP4 quantization of BF16 activations ("dynamic MXFP4
 * activations with A4W4 dispatch": "Kimi-K3 DSpark O-Proj-only MXFP4", section
 * "Exact quantization coverage").
 *   x_bf16 [M, K]      in   BF16, 16-byte aligned
 *   q      [M, K/2]    out  packed E2M1 codes, 16-byte aligned
 *   s      [M, K/32]   out  E8M0 scales (byte aligned)
 * K > 0 and K % 32 == 0.
 */
mx_status mx_quant_act_bf16(const void *x_bf16, int64_t M, int64_t K,
                            void *q, void *s, void *stream);

/*
 * Offline MXFP4 weight quantization from FP32 (the checkpoint conversion the
 * same section describes: weight (N, K) -> E2M1 codes + (N, K/32) E8M0 scales).
 * Same rules and layouts as mx_quant_act_bf16 with an FP32 input
 * (16-byte aligned).
 */
mx_status mx_quant_weight_f32(const float *w, int64_t N, int64_t K,
                              void *q, void *s, void *stream);

/*
 * Bytes of workspace mx_gemm_a4w4_bf16 needs for this shape: nonzero for the
 * sizes that split K across workgroups - M <= 64, K split into 4 or 8 parts
 * of 2048 K-values, 128-column tiles x parts between 128 and 256 workgroups;
 * 64 < M <= 128 in two 64-row halves, K split into 2 or 4 parts of 4096 or
 * 8192, 2 x tiles x parts between 128 and 256; M > 128 with at most 128
 * output tiles of 128 x 128 and K % 2048 == 0, K split into 2 parts (64 KB per
 * tile) - e.g. 7,340,032 bytes for the (64, 7168, 8192), (128, 7168, 8192)
 * and (256, 7168, 8192) layers, 8 MiB at most - and 0 otherwise.  It depends
 * on the shape only.  The
 * workspace holds the FP32 partial slots through which the workgroups of a
 * tile exchange their partial sums; a slot word reads 0 until written.  It
 * must be zero-filled (e.g. hipMemset) before its first use; every call
 * leaves it all zero again, for any shape.  Calls that share a workspace must
 * not run concurrently: issue them on one stream.
 */
size_t mx_gemm_a4w4_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * A4W4 block-scaled GEMM, Y = dequant(qa, sa) . dequant(qw, sw)^T, BF16 out
 * ("A4W4 dispatch" of "Kimi-K3 DSpark O-Proj-only MXFP4", section "Exact
 * quantization coverage").
 *   qa [M, K/2], sa [M, K/32]   activation codes / scales (from mx_quant_act_bf16)
 *   qw [N, K/2], sw [N, K/32]   weight codes / scales (e.g. from mx_quant_weight_f32)
 *   y_bf16 [M, N]               out
 * K > 0 and K % 128 == 0.  qa, qw 16-byte aligned; sa, sw 4-byte aligned;
 * y_bf16 2-byte aligned.  workspace: at least mx_gemm_a4w4_workspace_bytes(M,
 * N, K) bytes, 16-byte aligned, zero-filled before first use (see there);
 * may be NULL when that size is 0, else MX_ERROR_WORKSPACE.  The split-K
 * kernels sum the K parts of each output in a fixed order, so results
 * do not depend on timing.  Their workgroups wait for each other, so they run
 * only when the whole grid fits the device's CUs at once (one workgroup per
 * CU); otherwise the workspace-free kernels run.  They rely on
 * workgroups being dealt round-robin to the XCDs (the parts of a tile meet in
 * one XCD's L2), and on no other work keeping CUs from the grid for long -
 * in particular, two such launches (of this or of the other split-K entry
 * points) must not run at the same time on different streams, since each
 * would hold CUs the other waits for: a workgroup waiting for a partner
 * gives up after about 0.3 s, so that no launch can hang; the outputs it
 * owns are then NaN, and the workspace must be zero-filled again before its
 * next use.
 */
mx_status mx_gemm_a4w4_bf16(const void *qa, const void *sa, const void *qw, const void *sw,
                            void *y_bf16, int64_t M, int64_t N, int64_t K,
                            void *workspace, size_t workspace_bytes, void *stream);

/*
 * mx_gemm_a4w4_bf16 for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same arguments without a workspace.  The split-K kernel's workspace is a
 * static device array of 8 MiB per GPU (the largest any shape needs), held
 * from the library's load until the process ends; it is zero when loaded and
 * every call leaves it zero again.  A shape whose workspace were larger would
 * return MX_ERROR_WORKSPACE before anything is enqueued.  The call itself
 * allocates nothing.  All calls on one GPU share
 * the array, so calls that overlap on one GPU (other streams, other threads)
 * race: issue them on one stream.  Results equal mx_gemm_a4w4_bf16's bit for
 * bit.
 */
mx_status mx_gemm_a4w4_bf16_noalloc(const void *qa, const void *sa, const void *qw, const void *sw,
                                    void *y_bf16, int64_t M, int64_t N, int64_t K, void *stream);

/*
 * Bytes of workspace mx_linear_a4w4_bf16 needs for this shape: the split-K
 * partial slots (first 8 MiB), then room for the activation codes and scales
 * of the two-launch path; e.g. 8,667,136 for (64, 7168, 8192).  Same rules as
 * mx_gemm_a4w4_workspace_bytes: zero-filled before first use, the first 8 MiB
 * left zero by every call, not shared by concurrent calls; one zero-filled
 * buffer of the larger size may serve both entry points on one stream.
 */
size_t mx_linear_a4w4_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * The A4W4 layer in one call: BF16 activations in, BF16 out, the activations
 * quantized dynamically to MXFP4 on the way ("dynamic MXFP4 activations with
 * A4W4 dispatch": "Kimi-K3 DSpark O-Proj-only MXFP4", section "Exact
 * quantization coverage").  Y = dequant(mx_quant_act_bf16(X)) . dequant(qw,
 * sw)^T, the same value the two calls give.
 *   x_bf16 [M, K]  in  BF16, 16-byte aligned
 *   qw [N, K/2], sw [N, K/32]  weight codes / scales (qw 16-byte, sw 4-byte aligned)
 *   y_bf16 [M, N]  out, 2-byte aligned
 *   workspace  at least mx_linear_a4w4_workspace_bytes(M, N, K) bytes, 256-byte
 *              aligned, zero-filled before first use.
 * K > 0 and K % 128 == 0.  For M <= 8 (K a multiple of 1024 that splits into
 * 2, 4 or 8 parts, enough 128-column tiles for half the GPU, sw 16-byte
 * aligned, the grid resident at once) this is ONE kernel launch: every
 * workgroup quantizes its K part of X into LDS, bit for bit as
 * mx_quant_act_bf16, and runs the split-K GEMM on it, so no activation codes
 * are written to memory.  Other shapes run mx_quant_act_bf16 (codes and
 * scales in the workspace) and mx_gemm_a4w4_bf16 (its split-K partials in the
 * workspace too) in two launches on the same stream: with more rows, every
 * workgroup quantizing all M rows of its K part costs more than the second
 * launch (measured at N = 7168, K = 8192: one launch 8.6 vs 9.9 us at M = 1,
 * 11.4 vs 10.4 us at M = 16).
 */
mx_status mx_linear_a4w4_bf16(const void *x_bf16, const void *qw, const void *sw, void *y_bf16,
                              int64_t M, int64_t N, int64_t K,
                              void *workspace, size_t workspace_bytes, void *stream);

/*
 * Grouped A4W4 GEMM over MoE experts: expert weights and
 * activations both in OCP MXFP4 ("Kimi-K3-Quark-MXFP4-AttnFP8", section
 * "Model Quantization").  Group e multiplies the activation rows
 * offsets[e] .. offsets[e+1]-1 with expert weight e:
 *   Y[r, :] = dequant(qa, sa)[r] . dequant(qw[e], sw[e])^T  for those rows r.
 *   qa [T, K/2], sa [T, K/32]        packed activation codes / scales, T = offsets[G]
 *   qw [G, N, K/2], sw [G, N, K/32]  stacked expert weights (e.g. mx_quant_weight_f32 on [G*N, K])
 *   y_bf16 [T, N]                    out; rows outside every group are not written
 *   offsets [G + 1] int32, DEVICE memory, non-decreasing, offsets[0] = 0: read by the
 *            kernel, so routing computed on the GPU needs no host round trip (capturable)
 *   max_rows  the largest group's row count (or any bound on it), >= 0: it only
 *            picks the kernel - each workgroup takes its group in chunks of 32
 *            rows (max_rows <= 32) or 64 rows (larger), and every row of every
 *            group is written whatever the value; 0 declares every group empty.
 *            Groups are streamed as decode work (the expert weight columns of a
 *            workgroup are re-read from L2 for each chunk): sized for routed
 *            decode tokens, correct for groups of any size.
 * K % 512 == 0 and K <= 16384 (e.g. K = 2048 for an expert down projection,
 * K = 7168 for up / gate); qa, sa, qw, sw 16-byte aligned; y_bf16 2-byte
 * aligned; offsets 4-byte aligned; G <= 65535.  G, N or max_rows == 0: no-op.
 */
mx_status mx_gemm_a4w4_grouped_bf16(const void *qa, const void *sa, const void *qw, const void *sw,
                                    void *y_bf16, const int32_t *offsets, int64_t G, int64_t max_rows,
                                    int64_t N, int64_t K, void *stream);

/*
 * Dynamic per-token FP8 quantization of BF16 activations ("dynamic per-token
 * FP8, computed online": "Kimi-K3-DSpark-FP8-PTPC", section "Phase 1 FP8 PTPC
 * Quantization").
 *   x_bf16 [M, K] in (16-byte aligned); q [M, K] E4M3fn out (8-byte aligned);
 *   s [M] FP32 out (4-byte aligned).  K > 0 and K % 8 == 0.
 */
mx_status ptpc_quant_act_fp8(const void *x_bf16, int64_t M, int64_t K,
                             void *q, float *s, void *stream);

/*
 * Offline per-output-channel FP8 weight quantization from FP32 (the weight
 * side of the same scheme: E4M3 weight + FP32 (out_features, 1) scale).
 *   w [N, K] FP32 in (16-byte aligned); q [N, K] out (8-byte aligned);
 *   s [N] out.  K > 0 and K % 8 == 0.
 */
mx_status ptpc_quant_weight_f32(const float *w, int64_t N, int64_t K,
                                void *q, float *s, void *stream);

/*
 * Bytes of workspace gemm_a8w8_ptpc_bf16 needs for this shape: nonzero for the
 * sizes that split K across workgroups - 33 <= M <= 64, K split into 4 or 8
 * parts of 2048, 128-column tiles x parts between 128 and 256 workgroups
 * (e.g. 7,340,032 bytes for (64, 7168, 8192)); M > 128 with at most 128
 * output tiles of 128 x 128 and K % 256 == 0, K >= 2048: two K parts, 64 KB
 * per tile (7,340,032 bytes for (256, 7168, 8192)); past 256 such tiles, with
 * at most 128 output tiles of 256 x 224, K % 256 == 0 and K >= 2048: two K
 * parts, 224 KB per tile (e.g. 29,360,128 bytes for (1024, 7168, 8192), and
 * at most 29,360,128) - and 0 otherwise.
 * Same rules as mx_gemm_a4w4_workspace_bytes: it depends on the shape only,
 * must be zero-filled before first use, is left all zero by every call, and
 * calls that share a workspace must not run concurrently.
 */
size_t gemm_a8w8_ptpc_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * PTPC A8W8 GEMM: Y[m,n] = sa[m] * sw[n] * sum_k e4m3(qa[m,k]) * e4m3(qw[n,k]),
 * BF16 out (ATOM A8W8 of "Kimi-K3 DSpark O-Proj-only MXFP4", section "Exact
 * quantization coverage"; scales as in "Kimi-K3-DSpark-FP8-PTPC", section
 * "Phase 1 FP8 PTPC Quantization").
 *   qa [M, K], sa [M]; qw [N, K], sw [N] (the (out_features, 1) scale);
 *   y_bf16 [M, N] out.  K > 0 and K % 128 == 0; qa, qw 16-byte aligned;
 *   sa, sw 4-byte aligned; y_bf16 2-byte aligned.
 *   workspace: at least gemm_a8w8_ptpc_workspace_bytes(M, N, K) bytes,
 *   16-byte aligned, zero-filled before first use; may be NULL when that size
 *   is 0, else MX_ERROR_WORKSPACE.  At those sizes the K parts of each
 *   output are summed across workgroups in a fixed order (deterministic), as
 *   in mx_gemm_a4w4_bf16, when the grid fits the device's CUs at once.
 */
mx_status gemm_a8w8_ptpc_bf16(const void *qa, const float *sa, const void *qw, const float *sw,
                              void *y_bf16, int64_t M, int64_t N, int64_t K,
                              void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* MXGEMM_H */
