/*
 * fp8w — FP8 (OCP e4m3fn) weight-only linear layer for AMD MI355X (gfx950).
 *
 * C ABI of libfp8w.so. The method, from "FP8 weight-only (precision:
 * fp8_weights)", section "The contract":
 *   - at build time, once: one symmetric scale per output channel,
 *       scale[n] = amax_k |W[n,k]| / 448   (fp32),
 *       q[n,k]   = e4m3 code of W[n,k] / scale[n], rounded to nearest even and
 *                  clamped to +-448; no higher-precision copy of W is kept;
 *   - per call: y[m,n] = scale[n] * sum_k x[m,k] * value(q[n,k]) + bias[n],
 *     activations stay bf16 / fp16, accumulation and the scale/bias epilogue
 *     are fp32, and the result is rounded to the activation dtype once;
 *   - shapes the fast kernels do not cover go through the dequantised weight
 *     with the same numerics (section "The contract", item "Fallback").
 * The e4m3 format is the OCP one (bias 7, largest finite 448, 0x7F / 0xFF NaN,
 * 0x80 = -0): "B04 - Precision & Quantization", section "The numbers, derived
 * rather than tabulated", and section "Hardware support, and where the vendors
 * diverge" (not the FNUZ variant, whose maximum is 240).
 *
 * Conventions for every entry point:
 *   - Tensors are dense and row-major: W, q and a dequantised weight are
 *     [n, k] (n output channels, k input features), x is [m, k], y is [m, n].
 *   - All tensor pointers are DEVICE pointers owned by the caller. The library
 *     never allocates device memory. Its only state is fp8w_linear_noalloc's
 *     static scratch array (part of the loaded code object) and the cached
 *     device address of it per GPU.
 *   - Work is enqueued on `stream` (0 = the null stream) in stream order.
 *     Only fp8w_quantize synchronizes (on `stream`), to report non-finite
 *     weights. The other calls are asynchronous.
 *   - Arguments are validated before anything is enqueued. An invalid call
 *     returns an error and enqueues nothing.
 *   - Sizes: 0 <= n, k <= 2^31 - 1; 0 <= m <= 1048560; n*k <= 2^62.
 *     A zero-sized call is valid and enqueues nothing, except that k == 0
 *     writes y = bias (or zeros).
 *   - Thread-safe: the scratch address cache is filled once per GPU under a
 *     lock; nothing else is shared between calls (but see fp8w_linear_noalloc
 *     on overlapping calls).
 */
#ifndef FP8W_H
#define FP8W_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#if defined(__GNUC__) || defined(__clang__)
#define FP8W_API __attribute__((visibility("default")))
#else
#define FP8W_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FP8W_BF16 = 0, /* bfloat16, 2 bytes */
    FP8W_FP16 = 1, /* IEEE binary16, 2 bytes */
    FP8W_FP32 = 2  /* IEEE binary32, 4 bytes */
} fp8w_dtype_t;

typedef enum {
    FP8W_SUCCESS = 0,
    FP8W_ERR_INVALID_VALUE = 1, /* bad size, dtype, NULL pointer, aliasing or path request */
    FP8W_ERR_MISALIGNED = 2,    /* a pointer is not aligned to its element size, or a forced fast
                                   path was asked for with pointers it cannot take */
    FP8W_ERR_NONFINITE = 3,     /* fp8w_quantize: some weight is NaN or +-inf */
    FP8W_ERR_WORKSPACE = 4,     /* fallback path needs a larger workspace */
    FP8W_ERR_HIP = 5            /* a HIP runtime call or kernel launch failed */
} fp8w_status_t;

/* Dispatch paths (fp8w_linear_path, fp8w_linear_with_path). */
#define FP8W_PATH_AUTO (-1)
#define FP8W_PATH_GEMV 0     /* m == 1 streaming GEMV (fp32 FMA) */
#define FP8W_PATH_SKINNY 1   /* 1 <= m <= 32, matrix-core (MFMA) skinny GEMM */
#define FP8W_PATH_FALLBACK 2 /* unscaled dequantise to the activation dtype + guarded MFMA GEMM */
#define FP8W_PATH_BATCH 3    /* m > 32: tiled MFMA GEMM that decodes the codes in its main loop */

/*
 * Build-time quantizer ("The contract": scale = amax(|row|) / 448, codes
 * round(w / scale) in e4m3, nearest even, clamped to +-448; "Skill: Write an
 * FP8 Kernel", "Required reasoning process" steps 2 and 4).
 *   w       [n, k] weights, element type w_dtype (FP32, or BF16 / FP16 widened
 *           exactly to fp32), aligned to its element size.
 *   q       [n, k] output codes (uint8, OCP e4m3fn).
 *   scale   [n] output scales (fp32): fl32(amax / 448); 0 for an all-zero row,
 *           whose codes are then all 0x00 (no division takes place).
 *   Each code is the round-to-nearest-even e4m3 encoding of the fp32 quotient
 *   fl32(w / scale), clamped to +-448; -0 and negative values that round to
 *   zero give 0x80.
 * Enqueues one kernel on `stream`, copies the scales back and synchronizes the
 * stream. Returns FP8W_ERR_NONFINITE if any weight is NaN or infinite: the
 * scale of every such row is then NaN and its codes are unspecified.
 * q and scale must not overlap w.
 */
FP8W_API fp8w_status_t fp8w_quantize(const void* w, fp8w_dtype_t w_dtype, int64_t n, int64_t k, uint8_t* q,
                            float* scale, hipStream_t stream);

/*
 * The linear layer, y[m,n] = scale[n] * sum_k x[m,k] * value(q[n,k]) + bias[n]
 * ("The contract"), with fp32 accumulation and one rounding to act_dtype.
 *   x         [m, k] activations, act_dtype = FP8W_BF16 or FP8W_FP16.
 *   q, scale  as written by fp8w_quantize for an [n, k] weight.
 *   bias      [n] in act_dtype, or NULL for none.
 *   y         [m, n] output in act_dtype; must not overlap x, q, scale or bias.
 *   workspace device scratch of fp8w_linear_workspace_bytes(...) bytes (NULL / 0
 *             when that is 0); it must not overlap anything else. The fallback
 *             path needs it (2-byte aligned, FP8W_ERR_WORKSPACE when missing or
 *             short). Skinny and batch shapes whose tiles alone would leave
 *             CUs idle (skinny: m > 16 on layers of 4096 to 8192 channels;
 *             batch: few tiles) use it for fp32 partial sums of a k split
 *             (16-byte aligned); given less, they take a slower single-pass
 *             plan instead, with no error.
 * Dispatch (fp8w_linear_path): the fast kernels take k % 256 == 0 with x, q
 * 16-byte aligned: m == 1 the GEMV, 2 <= m <= 32 the skinny MFMA kernel, m > 32
 * the batch GEMM (which decodes the codes in its main loop, no workspace).
 * Where the fast kernels cannot load the codes (k % 256 != 0 or q not 16-byte
 * aligned), with k % 8 == 0 and x 16-byte aligned: m == 1 takes the GEMV when
 * k >= 256 and q is 8-byte aligned (16-code chunks from each row's first
 * 16-byte boundary when k % 16 == 8, else 8-code chunks); otherwise
 * 1 <= m <= 32 takes the skinny kernel when k >= 512 and q is 4-byte aligned
 * (16-byte loads from the first 16-byte boundary of each workgroup's rows
 * where q is 8-byte aligned and the rows are 16-byte aligned or alternate,
 * else 4-byte loads; the columns outside its ring as extra MFMAs; no
 * workspace). Everything else takes the fallback. Results of different paths and plans agree to
 * within fp32 summation-order rounding; a given call is deterministic.
 * Asynchronous; a failed launch returns FP8W_ERR_HIP.
 */
FP8W_API fp8w_status_t fp8w_linear(const void* x, fp8w_dtype_t act_dtype, int64_t m, int64_t k, const uint8_t* q,
                          const float* scale, const void* bias, int64_t n, void* y, void* workspace,
                          size_t workspace_bytes, hipStream_t stream);

/*
 * fp8w_linear with an explicit path (FP8W_PATH_*), for cross-checking the
 * kernels against one another. FP8W_PATH_GEMV needs m == 1,
 * FP8W_PATH_SKINNY needs m <= 32 and FP8W_PATH_BATCH takes any m, all with
 * k % 256 == 0 (FP8W_ERR_INVALID_VALUE otherwise) and 16-byte aligned x and q
 * (FP8W_ERR_MISALIGNED otherwise); FP8W_PATH_GEMV also takes k % 8 == 0,
 * k >= 256 with x 16-byte and q 8-byte aligned, and FP8W_PATH_SKINNY
 * k % 8 == 0, k >= 512 with x 16-byte and q 4-byte aligned (the shapes
 * fp8w_linear's dispatch sends there when the fast kernels cannot load the codes). FP8W_PATH_FALLBACK takes any shape and needs
 * n * k * element_size(act_dtype) bytes of workspace.
 */
FP8W_API fp8w_status_t fp8w_linear_with_path(const void* x, fp8w_dtype_t act_dtype, int64_t m, int64_t k,
                                    const uint8_t* q, const float* scale, const void* bias, int64_t n,
                                    void* y, void* workspace, size_t workspace_bytes, int path,
                                    hipStream_t stream);

/* Size of the static device scratch buffer of fp8w_linear_noalloc, per GPU. */
#define FP8W_SCRATCH_BYTES ((size_t)32 << 20)

/*
 * fp8w_linear for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc. Same
 * arguments (minus the workspace), dispatch, kernels and results as
 * fp8w_linear given a workspace of FP8W_SCRATCH_BYTES: the workspace is a
 * static device array inside the library (32 MiB on every GPU the library runs
 * on, held until the process ends), so nothing is allocated, by the call or by
 * the caller; the call makes no hipMalloc, hipFree or other allocating call.
 *   - A k split whose fp32 partial sums need more than FP8W_SCRATCH_BYTES runs
 *     its single-pass plan instead (as fp8w_linear does with a short workspace).
 *   - The fallback path needs n * k * 2 bytes for the 16-bit weight; a call
 *     that needs more than FP8W_SCRATCH_BYTES returns FP8W_ERR_WORKSPACE before
 *     anything is enqueued.
 *   - Every call on one GPU shares that GPU's buffer. Each call writes the part
 *     it reads before reading it, so nothing carries over between calls, but
 *     calls that may run at the same time on one GPU (streams not ordered with
 *     each other) race on the buffer and must not be made.
 *   - The first call that needs the buffer on a device looks up its address
 *     there (with that device current; the caller's current device is restored).
 * Asynchronous, like fp8w_linear.
 */
FP8W_API fp8w_status_t fp8w_linear_noalloc(const void* x, fp8w_dtype_t act_dtype, int64_t m, int64_t k,
                                           const uint8_t* q, const float* scale, const void* bias, int64_t n,
                                           void* y, hipStream_t stream);

/*
 * The dequantised weight ("The contract", item "Fallback": q.float() * scale[:, None]).
 *   out[r, j] = out_dtype(fl32(value(q[r,j]) * scale[r]))  when scale != NULL
 *               (FP32 is exactly q.float() * scale; BF16 / FP16 round that
 *               fp32 product to nearest even),
 *   out[r, j] = value(q[r,j])                              when scale == NULL
 *               (exact in every out_dtype; this is what the fallback GEMM uses).
 *   q [n, k] codes; scale [n] fp32 or NULL; out [n, k] of out_dtype
 *   (FP8W_BF16, FP8W_FP16 or FP8W_FP32), not overlapping q or scale.
 * Asynchronous.
 */
FP8W_API fp8w_status_t fp8w_dequantize_fallback(const uint8_t* q, const float* scale, int64_t n, int64_t k, void* out,
                                       fp8w_dtype_t out_dtype, hipStream_t stream);

/*
 * Which path fp8w_linear takes for these sizes and pointers: FP8W_PATH_GEMV,
 * FP8W_PATH_SKINNY, FP8W_PATH_BATCH or FP8W_PATH_FALLBACK; -1 when the
 * arguments are invalid. NULL pointers are treated as 256-byte aligned.
 */
FP8W_API int fp8w_linear_path(int64_t m, int64_t n, int64_t k, fp8w_dtype_t act_dtype, const void* x, const uint8_t* q,
                     const void* y);

/* Workspace bytes fp8w_linear uses for these sizes and pointers: 0 on the GEMV
   and on skinny and batch shapes that do not split k, splits * m * n * 4 on
   those that do, n * k * element_size(act_dtype) on the fallback; 0 when
   invalid. */
FP8W_API size_t fp8w_linear_workspace_bytes(int64_t m, int64_t n, int64_t k, fp8w_dtype_t act_dtype, const void* x,
                                   const uint8_t* q, const void* y);

/* Workspace bytes fp8w_linear_with_path uses for `path` (FP8W_PATH_AUTO or a
   forced path) on these sizes and pointers, the amount fp8w_linear_kernel's
   report assumes: FP8W_PATH_AUTO as fp8w_linear_workspace_bytes;
   FP8W_PATH_FALLBACK n * k * element_size(act_dtype); FP8W_PATH_SKINNY and
   FP8W_PATH_BATCH their k-split partial sums (splits * m * n * 4) only when that
   path is also the one FP8W_PATH_AUTO takes, else 0 (a forced path runs its
   single-pass plan); FP8W_PATH_GEMV 0. 0 when the arguments or the path are
   invalid. */
FP8W_API size_t fp8w_linear_with_path_workspace_bytes(int path, int64_t m, int64_t n, int64_t k,
                                                      fp8w_dtype_t act_dtype, const void* x, const uint8_t* q);

/*
 * Name of the kernel (and its tile parameters) that `path` (FP8W_PATH_AUTO or
 * a forced path) launches for these sizes and pointers, e.g.
 * "pipe_kernel<XR=16,CT=4,KP=1,NS=4>", given the workspace
 * fp8w_linear_workspace_bytes reports. A static or thread-local string, valid
 * until the next call on this thread; NULL when the arguments or the forced
 * path are invalid. For tests and measurement reports.
 */
FP8W_API const char* fp8w_linear_kernel(int path, int64_t m, int64_t n, int64_t k, fp8w_dtype_t act_dtype,
                                        const void* x, const uint8_t* q);

/*
 * Group-wise weight scales along k: one fp32 scale per run of `group`
 * consecutive weights of a row, group = 32, 64 or 128 ("B04 - Precision &
 * Quantization", section "Post-training quantization versus
 * quantization-aware training": per-group granularity, g = 32/64/128; section
 * "The one that matters: quantization is a quality decision": per-channel ->
 * per-group when an outlier inside a row costs accuracy; the Day-98 lab page's
 * "one scale per 32" census). Each group is quantized exactly as
 * fp8w_quantize quantizes a row. Scales are [n, k / group] fp32, row-major;
 * k % group == 0 is required (FP8W_ERR_INVALID_VALUE otherwise).
 */

/* Build-time quantizer with group scales: scale[r, j] = fl32(amax_j / 448) over
   w[r, j*group .. (j+1)*group), codes as in fp8w_quantize (0 for an all-zero
   group). Synchronizes `stream`; FP8W_ERR_NONFINITE if any weight is NaN or
   infinite (that group's scale is then NaN). q and scale must not overlap w. */
FP8W_API fp8w_status_t fp8w_quantize_grouped(const void* w, fp8w_dtype_t w_dtype, int64_t n, int64_t k,
                                             int64_t group, uint8_t* q, float* scale, hipStream_t stream);

/* y[m,n] = sum_j scale[n,j] * sum_{i<group} x[m, j*group+i] * value(q[n, j*group+i]) + bias[n],
   fp32 accumulation (each partial sum of exact products lies inside one
   group and is scaled before it is added), one rounding to act_dtype.
   Arguments as for fp8w_linear; no workspace (see
   fp8w_linear_grouped_with_workspace). Dispatch as fp8w_linear_path (m == 1:
   GEMV; m <= 32: skinny MFMA kernel; m > 32: the batch GEMM, here its single
   pass plan; k % 256 == 0 and 16-byte aligned x and q for all three); everything
   else, and skinny shapes whose k the ring cannot tile, runs a generic kernel
   (any m, n; x 2-byte aligned). Asynchronous. */
FP8W_API fp8w_status_t fp8w_linear_grouped(const void* x, fp8w_dtype_t act_dtype, int64_t m, int64_t k,
                                           const uint8_t* q, const float* scale, int64_t group, const void* bias,
                                           int64_t n, void* y, hipStream_t stream);

/* fp8w_linear_grouped with an explicit FP8W_PATH_* (same requirements as
   fp8w_linear_with_path, FP8W_PATH_BATCH included; FP8W_PATH_FALLBACK is the
   generic kernel). */
FP8W_API fp8w_status_t fp8w_linear_grouped_with_path(const void* x, fp8w_dtype_t act_dtype, int64_t m, int64_t k,
                                                     const uint8_t* q, const float* scale, int64_t group,
                                                     const void* bias, int64_t n, void* y, int path,
                                                     hipStream_t stream);

/* fp8w_linear_grouped with a workspace (and an explicit FP8W_PATH_*, or
   FP8W_PATH_AUTO): on the batch path (m > 32) a plan that splits k over
   workgroups uses fp8w_linear_grouped_workspace_bytes of it (16-byte aligned,
   not overlapping any argument: FP8W_ERR_MISALIGNED / FP8W_ERR_INVALID_VALUE),
   writing fp32 partial sums there and adding them in a second kernel;
   without one (NULL, or fewer bytes) the same call runs its single-pass plan.
   Other paths ignore the workspace. Asynchronous. */
FP8W_API fp8w_status_t fp8w_linear_grouped_with_workspace(const void* x, fp8w_dtype_t act_dtype, int64_t m,
                                                          int64_t k, const uint8_t* q, const float* scale,
                                                          int64_t group, const void* bias, int64_t n, void* y,
                                                          void* workspace, size_t workspace_bytes, int path,
                                                          hipStream_t stream);

/* Workspace bytes fp8w_linear_grouped_with_workspace uses on the path
   FP8W_PATH_AUTO takes: splits * m * n * 4 on batch shapes whose plan splits
   k, else 0 (also when invalid). */
FP8W_API size_t fp8w_linear_grouped_workspace_bytes(int64_t m, int64_t n, int64_t k, int64_t group,
                                                    fp8w_dtype_t act_dtype, const void* x, const uint8_t* q);

/* Path fp8w_linear_grouped takes (FP8W_PATH_GEMV, _SKINNY, _BATCH or
   _FALLBACK, by the rules of fp8w_linear_path), -1 when the arguments are
   invalid. */
FP8W_API int fp8w_linear_grouped_path(int64_t m, int64_t n, int64_t k, int64_t group, fp8w_dtype_t act_dtype,
                                      const void* x, const uint8_t* q);

/* Name of the kernel a grouped call takes (as fp8w_linear_kernel: on the
   batch path, given the workspace fp8w_linear_grouped_workspace_bytes
   reports); NULL when invalid. */
FP8W_API const char* fp8w_linear_grouped_kernel(int path, int64_t m, int64_t n, int64_t k, int64_t group,
                                                fp8w_dtype_t act_dtype, const void* x, const uint8_t* q);

/* The dequantised weight with group scales: out[r, j] = out_dtype(fl32(value(q[r,j])
   * scale[r, j / group])); out_dtype FP8W_FP32 (exactly q.float() * scale),
   FP8W_BF16 or FP8W_FP16 (round to nearest even). out must not overlap q or
   scale. Asynchronous. */
FP8W_API fp8w_status_t fp8w_dequantize_grouped(const uint8_t* q, const float* scale, int64_t group, int64_t n,
                                               int64_t k, void* out, fp8w_dtype_t out_dtype, hipStream_t stream);

/*
 * W8A8: activations quantized too, for batches far above 32 tokens (prefill),
 * where the matrix cores, not the weight stream, bound the layer ("Skill:
 * Write an FP8 Kernel", "Required reasoning process" steps 2, 4 and 5, and
 * "Correctness requirements"; the weight-only contract reserves this for
 * compute-bound GEMMs). Weights are the codes and scales of fp8w_quantize.
 */

/* Per-token activation quantizer: each row of x [m, k] (act_dtype BF16 / FP16)
   quantized exactly as fp8w_quantize quantizes a weight row: sx[t] =
   fl32(amax_t / 448), qx[t, :] the RNE e4m3 codes of x / sx[t], clamped to
   +-448 (0 for an all-zero row). Asynchronous: a row with a NaN or infinite
   value gets a NaN scale (its outputs are then NaN); nothing is reported. */
FP8W_API fp8w_status_t fp8w_quantize_activations(const void* x, fp8w_dtype_t act_dtype, int64_t m, int64_t k,
                                                 uint8_t* qx, float* sx, hipStream_t stream);

/* The W8A8 GEMM: y[t, c] = out_dtype(fl32(fl32(acc * sx[t]) * sw[c]) + bias[c]),
   acc = fp32 sum over k of value(qx[t,k]) * value(qw[c,k]) on the fp8 matrix
   cores (their internal sum is not exactly fp32: measured within ~1e-5 of
   the sum of |terms|). qx [m, k], qw [n, k] (16-byte aligned), k a positive
   multiple of 256 (FP8W_ERR_INVALID_VALUE otherwise); bias [n] in out_dtype or
   NULL; y [m, n] in out_dtype (BF16 / FP16), not overlapping any input.
   Asynchronous. */
FP8W_API fp8w_status_t fp8w_gemm_w8a8(const uint8_t* qx, const float* sx, int64_t m, int64_t k, const uint8_t* qw,
                                      const float* sw, const void* bias, int64_t n, void* y, fp8w_dtype_t out_dtype,
                                      hipStream_t stream);

/* Workspace of fp8w_linear_w8a8: the quantized activations (m*k bytes,
   rounded up to 256) followed by their m fp32 scales. */
FP8W_API size_t fp8w_linear_w8a8_workspace_bytes(int64_t m, int64_t k);

/* fp8w_quantize_activations into the workspace (16-byte aligned, at least
   fp8w_linear_w8a8_workspace_bytes; FP8W_ERR_WORKSPACE otherwise), then
   fp8w_gemm_w8a8 with out_dtype = act_dtype. Asynchronous. */
FP8W_API fp8w_status_t fp8w_linear_w8a8(const void* x, fp8w_dtype_t act_dtype, int64_t m, int64_t k,
                                        const uint8_t* qw, const float* sw, const void* bias, int64_t n, void* y,
                                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Name of the W8A8 GEMM instance for these sizes; NULL when unsupported. */
FP8W_API const char* fp8w_linear_w8a8_kernel(int64_t m, int64_t n, int64_t k);

/*
 * Format interop ("B04 - Precision & Quantization", the format table's
 * E4M3FNUZ row, section "Hardware support, and where the vendors diverge", and
 * its trap list: the same bits decode a factor of two apart on gfx942's FNUZ
 * e4m3 (bias 8, maximum 240, 0x80 NaN, no negative zero) and the OCP e4m3fn
 * this library computes in; tag the format). Translates `count` FNUZ codes
 * into the OCP codes of the same values, round to nearest even, so a
 * checkpoint quantized for gfx942 keeps its scales. All values are kept
 * except the 16 patterns below 2^-6 with an odd mantissa, which lie halfway
 * between OCP subnormals and move 2^-10 to the even one; NaN (0x80) becomes
 * 0x7F. src and dst are device pointers; dst may equal src (in place) but may
 * not otherwise overlap it. Asynchronous.
 */
FP8W_API fp8w_status_t fp8w_fnuz_to_ocp(const uint8_t* src, int64_t count, uint8_t* dst, hipStream_t stream);

/*
 * Measurement aid, not part of the method: read `bytes` bytes at `p` once
 * with the 128-bit streaming loads the linear kernels use, folding them into a
 * word that is written to `sink` (one uint32, device) only for one specific
 * value. Its duration is the streaming-read reference for a weight of that
 * size on this GPU. bytes must be a multiple of 16, p 16-byte aligned.
 * Asynchronous.
 */
FP8W_API fp8w_status_t fp8w_stream_read_probe(const void* p, size_t bytes, uint32_t* sink, hipStream_t stream);

/* Static, NUL-terminated description of a status code. */
FP8W_API const char* fp8w_status_string(fp8w_status_t status);

/* The hipError_t of the most recent FP8W_ERR_HIP returned on this thread (0 if none). */
FP8W_API int fp8w_last_hip_error(void);

/* ABI version of this header: 1. */
FP8W_API int fp8w_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8W_H */
