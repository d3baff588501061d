// Host-side launchers of the fp8w HIP kernels. Internal to the library: the
// public interface is the C ABI in include/fp8w.h. Every launcher enqueues on
// the given stream, returns the launch status, and assumes the C-ABI layer has
// already validated sizes, pointers and alignment.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fp8w {

enum class Act { BF16 = 0, FP16 = 1, FP32 = 2 };

// Build-time quantizer: one workgroup per row; scale[r] = NaN marks a row with
// a non-finite weight.
hipError_t launch_quantize(const void* w, Act w_type, int64_t n, int64_t k, uint8_t* q, float* scale,
                           hipStream_t stream);

// M = 1 streaming GEMV; x 16-byte aligned; k % 16 == 0 and q 16-byte aligned
// (16-code chunks), or k % 8 == 0 and q 8-byte aligned (k % 16 == 8: 16-code
// chunks from each row's first 16-byte boundary; else 8-code chunks).
hipError_t launch_gemv(const void* x, Act act, int64_t k, const uint8_t* q, const float* scale,
                       const void* bias, int64_t n, void* y, hipStream_t stream);

// Name of the GEMV instance launch_gemv picks for this shape and code address
// (16-code chunks; rows of alternating alignment; 8-code chunks).
const char* gemv_kernel_name(int64_t n, int64_t k, const uint8_t* q);

// M = 1..32 MFMA skinny GEMM; x 16-byte aligned; either k % 256 == 0 and q
// 16-byte aligned, or (plan_ring4) k % 8 == 0, k >= 512 and q 4-byte aligned. Shapes that split k use ws (fp32 partial sums, 16-byte
// aligned, not overlapping any operand) when ws_bytes >= skinny_workspace_bytes
// (m, n, k); otherwise they take the single-pass plan. The unaligned-code path never
// splits.
hipError_t launch_skinny(const void* x, Act act, int64_t m, int64_t k, const uint8_t* q, const float* scale,
                         const void* bias, int64_t n, void* y, void* ws, size_t ws_bytes, hipStream_t stream);

// Workspace bytes the 16-byte skinny path uses for split k on this shape (0: none).
size_t skinny_workspace_bytes(int64_t m, int64_t n, int64_t k);

// Name of the kernel and tile launch_skinny picks for this shape (a
// thread-local string; for tests and measurement reports); ring4: the path for
// codes the 16-byte kernels cannot load, at address q.
const char* skinny_kernel_name(int64_t m, int64_t n, int64_t k, bool with_workspace, bool ring4 = false,
                               const uint8_t* q = nullptr);

// The plan for codes the 16-byte kernels cannot load: ok when it takes the
// shape (1..32 tokens, k % 8 == 0, k >= 512); the ring covers kr columns, the
// other k - kr are register-operand MFMAs; cb is the rows' alignment the
// kernel is built for (8: 16-byte loads from a shift of 0 or 8 columns; 4:
// 4-byte loads).
struct Ring4Plan {
    bool ok;
    int xr, ct, kp, ns, cb;
    int64_t kr;
};
Ring4Plan plan_ring4(int64_t m, int64_t n, int64_t k, const uint8_t* q);

// The skinny kernel for layers of fewer than 8192 channels (narrow_kernel):
// activation fragments in VGPRs, codes alone in per-wave LDS rings. plan_narrow
// says whether it takes a shape (ok) and with which tile.
struct NarrowPlan {
    bool ok;
    int mt, w, ns;  // 16-token MFMA tiles, waves, ring stages
    bool ql;        // activation parts loaded by neighbouring lanes, moved by ds_bpermute
};
// split_ok: the caller gives workspace for a k split, which the skinny kernel
// then prefers on the shapes where it measured faster (see plan_narrow).
NarrowPlan plan_narrow(int64_t m, int64_t n, int64_t k, bool split_ok = false);
hipError_t launch_narrow(const NarrowPlan& p, const void* x, Act act, int64_t m, int64_t k, const uint8_t* q,
                         const float* scale, const void* bias, int64_t n, void* y, hipStream_t stream);
const char* narrow_kernel_name(const NarrowPlan& p);

// Sum of fp32 partial sums part[splits, m, n] in split order, then the
// scale/bias epilogue into y (act_type).
hipError_t launch_splitk_reduce(const float* part, int splits, int64_t m, int64_t n, const float* scale,
                                const void* bias, void* y, Act act, hipStream_t stream);

// The linear for m > 32 (any m >= 1): a GEMM over BN x BM tiles that decodes the
// codes in its main loop; k % 256 == 0, x and q 16-byte aligned. Plans that
// split k use ws (fp32 partial sums, 16-byte aligned, not overlapping any
// operand) when ws_bytes >= batch_workspace_bytes(m, n, k); otherwise the
// single-pass plan runs.
hipError_t launch_batch(const void* x, Act act, int64_t m, int64_t k, const uint8_t* q, const float* scale,
                        const void* bias, int64_t n, void* y, void* ws, size_t ws_bytes, hipStream_t stream);

// Workspace bytes the batch path uses for split k on this shape (0: none).
size_t batch_workspace_bytes(int64_t m, int64_t n, int64_t k);

// Name of the batch kernel plan launch_batch picks for this shape.
const char* batch_kernel_name(int64_t m, int64_t n, int64_t k, bool with_workspace);

// Dequantize codes to out_type: value(q) * scale[r] (scale != nullptr) or the
// exact unscaled value (scale == nullptr).
hipError_t launch_dequantize(const uint8_t* q, const float* scale, int64_t n, int64_t k, void* out,
                             Act out_type, hipStream_t stream);

// Name of the fallback's GEMM for this shape (assuming a 16-byte aligned
// workspace).
const char* fallback_kernel_name(int64_t m, int64_t n, int64_t k, const void* x);

// Guarded GEMM over an activation-dtype weight wd [n, k] (any m, n, k, any
// 2-byte alignment) followed by the scale/bias epilogue.
hipError_t launch_fallback_gemm(const void* x, Act act, int64_t m, int64_t k, const void* wd,
                                const float* scale, const void* bias, int64_t n, void* y,
                                hipStream_t stream);

// ---- group-wise scales along k (scale [n, k / group], group 32, 64 or 128)

// Build-time quantizer with one scale per run of `group` weights of a row; a
// group with a non-finite weight gets a NaN scale.
hipError_t launch_quantize_groups(const void* w, Act w_type, int64_t n, int64_t k, int64_t group, uint8_t* q,
                                  float* scale, hipStream_t stream);

// The grouped linear. path 0: M = 1 GEMV (k % 256 == 0, x and q 16-byte
// aligned); path 1: M <= 32 skinny ring where k allows it, else the generic
// kernel; path 2: the generic kernel (any m, n, k % group == 0, x 2-byte and q
// 1-byte aligned); path 3: the batch GEMM (launch_batch_grouped, which alone
// uses ws).
hipError_t launch_linear_grouped(int path, const void* x, Act act, int64_t m, int64_t k, const uint8_t* q,
                                 const float* scale, int64_t group, const void* bias, int64_t n, void* y, void* ws,
                                 size_t ws_bytes, hipStream_t stream);

// The grouped linear above 32 tokens: the batch GEMM with group scales staged
// beside the operands (k % 256 == 0, group 32 / 64 / 128, x and q 16-byte
// aligned). Splits k when the plan asks for it and ws holds
// batch_grouped_workspace_bytes (16-byte aligned), else single pass.
size_t batch_grouped_workspace_bytes(int64_t m, int64_t n, int64_t k, int64_t group);
hipError_t launch_batch_grouped(const void* x, Act act, int64_t m, int64_t k, const uint8_t* q, const float* gs,
                                int64_t group, const void* bias, int64_t n, void* y, void* ws, size_t ws_bytes,
                                hipStream_t stream);
const char* batch_grouped_kernel_name(int64_t m, int64_t n, int64_t k, int64_t group, bool with_workspace);

// Name of the kernel launch_linear_grouped runs for this path and shape.
const char* grouped_kernel_name(int path, int64_t m, int64_t n, int64_t k, int64_t group, bool with_workspace);

// value(q) * scale[r, j / group] rounded to out_type.
hipError_t launch_dequantize_grouped(const uint8_t* q, const float* scale, int64_t group, int64_t n, int64_t k,
                                     void* out, Act out_type, hipStream_t stream);

// W8A8 GEMM: y[t, c] = out(acc * sx[t] * sw[c] + bias[c]) with acc the fp32 sum
// of e4m3 x e4m3 products of qx [m, k] and qw [n, k]; k % 256 == 0, qx and qw
// 16-byte aligned.
hipError_t launch_w8a8(const uint8_t* qx, const float* sx, int64_t m, int64_t k, const uint8_t* qw, const float* sw,
                       const void* bias, int64_t n, void* y, Act out, hipStream_t stream);

// Name of the W8A8 kernel instance for this shape.
const char* w8a8_kernel_name(int64_t m, int64_t n, int64_t k);

// E4M3FNUZ codes -> OCP e4m3fn codes of the same values (dst may equal src).
hipError_t launch_fnuz_to_ocp(const uint8_t* src, int64_t count, uint8_t* dst, hipStream_t stream);

// Plain streaming read of `bytes` bytes (16-byte aligned, multiple of 16): the
// bandwidth reference the linear kernels are read against.
hipError_t launch_read_probe(const void* p, size_t bytes, uint32_t* sink, hipStream_t stream);

}  // namespace fp8w
