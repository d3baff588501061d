// C ABI of libfp8w.so: argument validation, path selection and kernel
// dispatch. Declarations and the contract of each call are in include/fp8w.h.
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "../../include/fp8w.h"
#include "kernels.hpp"

namespace {

thread_local int g_last_hip_error = 0;

constexpr int64_t kMaxNK = (int64_t)0x7fffffff;  // grid dimension and row-count limit
constexpr int64_t kMaxM = (int64_t)65535 * 16;     // fallback token tiles on grid.y
constexpr int64_t kMaxElems = (int64_t)1 << 62;

fp8w_status_t hip_status(hipError_t e)
{
    if (e == hipSuccess)
        return FP8W_SUCCESS;
    g_last_hip_error = (int)e;
    return FP8W_ERR_HIP;
}

bool aligned(const void* p, uintptr_t a)
{
    return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

int elem_bytes(fp8w_dtype_t t)
{
    return t == FP8W_FP32 ? 4 : 2;
}

bool valid_dtype(fp8w_dtype_t t)
{
    return t == FP8W_BF16 || t == FP8W_FP16 || t == FP8W_FP32;
}

bool valid_act(fp8w_dtype_t t)
{
    return t == FP8W_BF16 || t == FP8W_FP16;
}

fp8w::Act act_of(fp8w_dtype_t t)
{
    return t == FP8W_BF16 ? fp8w::Act::BF16 : (t == FP8W_FP16 ? fp8w::Act::FP16 : fp8w::Act::FP32);
}

bool sizes_ok(int64_t m, int64_t n, int64_t k)
{
    if (m < 0 || n < 0 || k < 0 || m > kMaxM || n > kMaxNK || k > kMaxNK)
        return false;
    return n == 0 || k <= kMaxElems / n;
}

// Byte ranges [a, a+na) and [b, b+nb) overlap (empty ranges never do).
bool overlap(const void* a, size_t na, const void* b, size_t nb)
{
    if (!a || !b || na == 0 || nb == 0)
        return false;
    const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
    return pa < pb + nb && pb < pa + na;
}

// The fast kernels' coverage: see fp8w_linear in include/fp8w.h.
bool fast_k(int64_t k)
{
    return k >= 256 && k % 256 == 0;
}

bool fast_shape(int64_t m, int64_t k)
{
    return m >= 1 && m <= 32 && fast_k(k);
}

bool fast_pointers(const void* x, const uint8_t* q)
{
    return aligned(x, 16) && aligned(q, 16);
}

// The skinny kernel's unaligned-code path: 1..32 tokens whose codes the 16-byte
// kernels cannot load (k not a multiple of 256, or q not 16-byte aligned),
// with k % 8 == 0, k >= 512, q 4-byte and x 16-byte aligned.
bool ring4_shape(int64_t m, int64_t k, const void* x, const uint8_t* q)
{
    if (m < 1 || m > 32 || k < 512 || k % 8 != 0 || !aligned(x, 16) || !aligned(q, 4))
        return false;
    return !(fast_k(k) && fast_pointers(x, q));
}

// The GEMV on rows only 8-byte aligned: one token whose codes the 16-byte
// kernels cannot load at their row starts, with k % 8 == 0, k >= 256, q
// 8-byte and x 16-byte aligned.
bool gemv8_shape(int64_t m, int64_t k, const void* x, const uint8_t* q)
{
    if (m != 1 || k < 256 || k % 8 != 0 || !aligned(x, 16) || !aligned(q, 8))
        return false;
    return !(fast_k(k) && fast_pointers(x, q));
}

// The per-channel linear: GEMV, skinny MFMA, the batch GEMM above 32 tokens,
// or the fallback.
int auto_path(int64_t m, int64_t k, const void* x, const uint8_t* q)
{
    if (m >= 1 && fast_k(k) && fast_pointers(x, q))
        return m == 1 ? FP8W_PATH_GEMV : m <= 32 ? FP8W_PATH_SKINNY : FP8W_PATH_BATCH;
    if (gemv8_shape(m, k, x, q))
        return FP8W_PATH_GEMV;
    return ring4_shape(m, k, x, q) ? FP8W_PATH_SKINNY : FP8W_PATH_FALLBACK;
}

// The grouped linear: the same split by tokens, without the unaligned-code path.
int auto_path_grouped(int64_t m, int64_t k, const void* x, const uint8_t* q)
{
    if (!fast_k(k) || !fast_pointers(x, q) || m < 1)
        return FP8W_PATH_FALLBACK;
    return m == 1 ? FP8W_PATH_GEMV : m <= 32 ? FP8W_PATH_SKINNY : FP8W_PATH_BATCH;
}

// Workspace bytes the skinny path uses for this call (the unaligned-code path: none).
size_t skinny_workspace(int64_t m, int64_t n, int64_t k, const void* x, const uint8_t* q)
{
    return ring4_shape(m, k, x, q) ? 0 : fp8w::skinny_workspace_bytes(m, n, k);
}

size_t fallback_workspace(int64_t n, int64_t k, fp8w_dtype_t act)
{
    return (size_t)n * (size_t)k * (size_t)elem_bytes(act);
}

fp8w_status_t check_linear(const void* x, fp8w_dtype_t act, int64_t m, int64_t k, const uint8_t* q,
                           const float* scale, const void* bias, int64_t n, const void* y)
{
    if (!valid_act(act) || !sizes_ok(m, n, k))
        return FP8W_ERR_INVALID_VALUE;
    if (m == 0 || n == 0)
        return FP8W_SUCCESS;
    if (!y || !scale || (k > 0 && (!x || !q)))
        return FP8W_ERR_INVALID_VALUE;
    if (!aligned(x, 2) || !aligned(y, 2) || !aligned(bias, 2) || !aligned(scale, 4))
        return FP8W_ERR_MISALIGNED;
    const size_t eb = 2;
    const size_t ybytes = (size_t)m * (size_t)n * eb;
    if (overlap(y, ybytes, x, (size_t)m * (size_t)k * eb) || overlap(y, ybytes, q, (size_t)n * (size_t)k) ||
        overlap(y, ybytes, scale, (size_t)n * 4) || overlap(y, ybytes, bias, bias ? (size_t)n * eb : 0))
        return FP8W_ERR_INVALID_VALUE;
    return FP8W_SUCCESS;
}

// Whether `need` bytes of workspace at ws overlap any operand of the call.
bool ws_overlaps(const void* ws, size_t need, const void* x, int64_t m, int64_t k, const uint8_t* q,
                 const float* scale, const void* bias, int64_t n, const void* y)
{
    return overlap(ws, need, y, (size_t)m * (size_t)n * 2) || overlap(ws, need, x, (size_t)m * (size_t)k * 2) ||
           overlap(ws, need, q, (size_t)n * (size_t)k) || overlap(ws, need, scale, (size_t)n * 4) ||
           overlap(ws, need, bias, bias ? (size_t)n * 2 : 0);
}

fp8w_status_t run_linear(const void* x, fp8w_dtype_t act, int64_t m, int64_t k, const uint8_t* q,
                         const float* scale, const void* bias, int64_t n, void* y, void* ws, size_t ws_bytes,
                         int path, hipStream_t stream)
{
    fp8w_status_t st = check_linear(x, act, m, k, q, scale, bias, n, y);
    if (st != FP8W_SUCCESS)
        return st;
    if (path == FP8W_PATH_AUTO)
        path = auto_path(m, k, x, q);
    if (path == FP8W_PATH_GEMV) {
        if (m != 1 && m != 0)
            return FP8W_ERR_INVALID_VALUE;
        // k % 256 == 0 with x and q 16-byte aligned, or rows 8-byte aligned
        // (k % 8 == 0, x 16-byte and q 8-byte aligned: launch_gemv picks the chunking)
        if (!(fast_k(k) && fast_pointers(x, q))) {
            if (k < 256 || k % 8 != 0)
                return FP8W_ERR_INVALID_VALUE;
            if (!aligned(x, 16) || !aligned(q, 8))
                return FP8W_ERR_MISALIGNED;
        }
    } else if (path == FP8W_PATH_SKINNY) {
        // the 16-byte kernels (k % 256 == 0, x and q 16-byte aligned) or the
        // unaligned-code path (k % 8 == 0, k >= 512, x 16-byte and q 4-byte aligned)
        if (m > 32)
            return FP8W_ERR_INVALID_VALUE;
        if (!(fast_k(k) && fast_pointers(x, q))) {
            if (k < 512 || k % 8 != 0)
                return fast_k(k) ? FP8W_ERR_MISALIGNED : FP8W_ERR_INVALID_VALUE;
            if (!aligned(x, 16) || !aligned(q, 4))
                return FP8W_ERR_MISALIGNED;
        }
    } else if (path == FP8W_PATH_BATCH) {
        if (!fast_k(k))
            return FP8W_ERR_INVALID_VALUE;
        if (!fast_pointers(x, q))
            return FP8W_ERR_MISALIGNED;
    } else if (path != FP8W_PATH_FALLBACK) {
        return FP8W_ERR_INVALID_VALUE;
    }
    if (m == 0 || n == 0)
        return FP8W_SUCCESS;

    const fp8w::Act a = act_of(act);
    if (path == FP8W_PATH_GEMV)
        return hip_status(fp8w::launch_gemv(x, a, k, q, scale, bias, n, y, stream));
    if (path == FP8W_PATH_BATCH) {
        // split k on plans that use it, when the caller's workspace is large enough
        const size_t need = fp8w::batch_workspace_bytes(m, n, k);
        const bool use_ws = need > 0 && ws && ws_bytes >= need;
        if (use_ws) {
            if (!aligned(ws, 16))
                return FP8W_ERR_MISALIGNED;
            if (ws_overlaps(ws, need, x, m, k, q, scale, bias, n, y))
                return FP8W_ERR_INVALID_VALUE;
        }
        return hip_status(fp8w::launch_batch(x, a, m, k, q, scale, bias, n, y, use_ws ? ws : nullptr,
                                             use_ws ? ws_bytes : 0, stream));
    }
    if (path == FP8W_PATH_SKINNY) {
        // split k on shapes that use it, when the caller's workspace is large enough
        const size_t need = skinny_workspace(m, n, k, x, q);
        const bool use_ws = need > 0 && ws && ws_bytes >= need;
        if (use_ws) {
            if (!aligned(ws, 16))
                return FP8W_ERR_MISALIGNED;
            if (ws_overlaps(ws, need, x, m, k, q, scale, bias, n, y))
                return FP8W_ERR_INVALID_VALUE;
        }
        return hip_status(fp8w::launch_skinny(x, a, m, k, q, scale, bias, n, y, use_ws ? ws : nullptr,
                                              use_ws ? ws_bytes : 0, stream));
    }

    const size_t need = fallback_workspace(n, k, act);
    if (need > 0) {
        if (!ws || ws_bytes < need)
            return FP8W_ERR_WORKSPACE;
        if (!aligned(ws, 2))
            return FP8W_ERR_MISALIGNED;
        if (ws_overlaps(ws, need, x, m, k, q, scale, bias, n, y))
            return FP8W_ERR_INVALID_VALUE;
        st = hip_status(fp8w::launch_dequantize(q, nullptr, n, k, ws, a, stream));
        if (st != FP8W_SUCCESS)
            return st;
    }
    return hip_status(fp8w::launch_fallback_gemm(x, a, m, k, ws, scale, bias, n, y, stream));
}

// ---- group-wise scales
bool valid_group(int64_t k, int64_t group)
{
    return (group == 32 || group == 64 || group == 128) && k % group == 0;
}

size_t group_scale_bytes(int64_t n, int64_t k, int64_t group)
{
    return (size_t)n * (size_t)(k / group) * 4;
}

fp8w_status_t run_linear_grouped(const void* x, fp8w_dtype_t act, int64_t m, int64_t k, const uint8_t* q,
                                 const float* scale, int64_t group, const void* bias, int64_t n, void* y, void* ws,
                                 size_t ws_bytes, int path, hipStream_t stream)
{
    if (!valid_act(act) || !sizes_ok(m, n, k) || !valid_group(k, group))
        return FP8W_ERR_INVALID_VALUE;
    if (path < FP8W_PATH_AUTO || path > FP8W_PATH_BATCH)
        return FP8W_ERR_INVALID_VALUE;
    if (path == FP8W_PATH_AUTO)
        path = auto_path_grouped(m, k, x, q);
    if (path == FP8W_PATH_GEMV || path == FP8W_PATH_SKINNY) {
        if (path == FP8W_PATH_GEMV && m != 1 && m != 0)
            return FP8W_ERR_INVALID_VALUE;
        if (m > 32 || k % 256 != 0 || k == 0)
            return FP8W_ERR_INVALID_VALUE;
    } else if (path == FP8W_PATH_BATCH && !fast_k(k)) {
        return FP8W_ERR_INVALID_VALUE;
    }
    if (m == 0 || n == 0)
        return FP8W_SUCCESS;
    if (!y || (k > 0 && (!x || !q || !scale)))
        return FP8W_ERR_INVALID_VALUE;
    if (!aligned(x, 2) || !aligned(y, 2) || !aligned(bias, 2) || !aligned(scale, 4))
        return FP8W_ERR_MISALIGNED;
    if (path != FP8W_PATH_FALLBACK && !fast_pointers(x, q))
        return FP8W_ERR_MISALIGNED;
    const size_t ybytes = (size_t)m * (size_t)n * 2;
    if (overlap(y, ybytes, x, (size_t)m * (size_t)k * 2) || overlap(y, ybytes, q, (size_t)n * (size_t)k) ||
        overlap(y, ybytes, scale, group_scale_bytes(n, k, group)) ||
        overlap(y, ybytes, bias, bias ? (size_t)n * 2 : 0))
        return FP8W_ERR_INVALID_VALUE;
    // the batch path splits k on plans that use it, when the caller's workspace is large enough
    const size_t need = path == FP8W_PATH_BATCH ? fp8w::batch_grouped_workspace_bytes(m, n, k, group) : 0;
    const bool use_ws = need > 0 && ws && ws_bytes >= need;
    if (use_ws) {
        if (!aligned(ws, 16))
            return FP8W_ERR_MISALIGNED;
        if (overlap(ws, need, y, ybytes) || overlap(ws, need, x, (size_t)m * (size_t)k * 2) ||
            overlap(ws, need, q, (size_t)n * (size_t)k) || overlap(ws, need, scale, group_scale_bytes(n, k, group)) ||
            overlap(ws, need, bias, bias ? (size_t)n * 2 : 0))
            return FP8W_ERR_INVALID_VALUE;
    }
    return hip_status(fp8w::launch_linear_grouped(path, x, act_of(act), m, k, q, scale, group, bias, n, y,
                                                  use_ws ? ws : nullptr, use_ws ? ws_bytes : 0, stream));
}

// ---- scratch of the no-allocation entry point (fp8w_linear_noalloc)
// Every GPU the library runs on holds its own copy of this array, at its own
// address, until the process ends. In host code `scratch` names only a
// host-side handle, not a device address: the address is looked up once per
// device with hipGetSymbolAddress (that device current) and kept, and only that
// pointer is ever handed to kernels.
static __device__ __align__(256) uint8_t scratch[FP8W_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;

// Device address of the scratch array on the GPU that `stream` runs on.
fp8w_status_t scratch_for(hipStream_t stream, void** out)
{
    int dev = 0;
    hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_status(e);
    if (dev < 0 || dev >= kMaxDevices)
        return FP8W_ERR_INVALID_VALUE;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            int cur = 0;
            e = hipGetDevice(&cur);
            if (e != hipSuccess)
                return hip_status(e);
            if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
                return hip_status(e);
            void* addr = nullptr;
            e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
            const hipError_t back = cur != dev ? hipSetDevice(cur) : hipSuccess;
            if (e != hipSuccess)
                return hip_status(e);
            if (back != hipSuccess)
                return hip_status(back);
            if (!addr)
                return hip_status(hipErrorInvalidSymbol);
            p = addr;
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return FP8W_SUCCESS;
}

}  // namespace

extern "C" {

fp8w_status_t fp8w_linear_noalloc(const void* x, fp8w_dtype_t act_dtype, int64_t m, int64_t k, const uint8_t* q,
                                  const float* scale, const void* bias, int64_t n, void* y, hipStream_t stream)
{
    fp8w_status_t st = check_linear(x, act_dtype, m, k, q, scale, bias, n, y);
    if (st != FP8W_SUCCESS || m == 0 || n == 0)
        return st;
    const int path = auto_path(m, k, x, q);
    size_t need = 0;
    if (path == FP8W_PATH_FALLBACK) {
        need = fallback_workspace(n, k, act_dtype);
        if (need > FP8W_SCRATCH_BYTES)  // the 16-bit weight would not fit: rejected before anything runs
            return FP8W_ERR_WORKSPACE;
    } else if (path == FP8W_PATH_SKINNY) {
        need = skinny_workspace(m, n, k, x, q);
    } else if (path == FP8W_PATH_BATCH) {
        need = fp8w::batch_workspace_bytes(m, n, k);
    }
    void* ws = nullptr;
    if (need > 0 && (st = scratch_for(stream, &ws)) != FP8W_SUCCESS)
        return st;
    // a k split whose partial sums would not fit takes its single-pass plan, as
    // fp8w_linear does when given fewer bytes
    return run_linear(x, act_dtype, m, k, q, scale, bias, n, y, ws, ws ? (size_t)FP8W_SCRATCH_BYTES : 0,
                      FP8W_PATH_AUTO, stream);
}

fp8w_status_t fp8w_quantize_grouped(const void* w, fp8w_dtype_t w_dtype, int64_t n, int64_t k, int64_t group,
                                    uint8_t* q, float* scale, hipStream_t stream)
{
    if (!valid_dtype(w_dtype) || !sizes_ok(0, n, k) || !valid_group(k, group))
        return FP8W_ERR_INVALID_VALUE;
    if (n == 0 || k == 0)
        return FP8W_SUCCESS;
    if (!w || !q || !scale)
        return FP8W_ERR_INVALID_VALUE;
    const size_t eb = (size_t)elem_bytes(w_dtype);
    if (!aligned(w, eb) || !aligned(scale, 4))
        return FP8W_ERR_MISALIGNED;
    const size_t wbytes = (size_t)n * (size_t)k * eb, qbytes = (size_t)n * (size_t)k;
    const size_t sbytes = group_scale_bytes(n, k, group);
    if (overlap(q, qbytes, w, wbytes) || overlap(scale, sbytes, w, wbytes) || overlap(scale, sbytes, q, qbytes))
        return FP8W_ERR_INVALID_VALUE;

    fp8w_status_t st =
        hip_status(fp8w::launch_quantize_groups(w, act_of(w_dtype), n, k, group, q, scale, stream));
    if (st != FP8W_SUCCESS)
        return st;
    std::vector<float> host(sbytes / 4);
    st = hip_status(hipMemcpyAsync(host.data(), scale, sbytes, hipMemcpyDeviceToHost, stream));
    if (st != FP8W_SUCCESS)
        return st;
    st = hip_status(hipStreamSynchronize(stream));
    if (st != FP8W_SUCCESS)
        return st;
    for (float s : host)
        if (!isfinite(s))
            return FP8W_ERR_NONFINITE;
    return FP8W_SUCCESS;
}

fp8w_status_t fp8w_linear_grouped(const void* x, fp8w_dtype_t act_dtype, int64_t m, int64_t k, const uint8_t* q,
                                  const float* scale, int64_t group, const void* bias, int64_t n, void* y,
                                  hipStream_t stream)
{
    return run_linear_grouped(x, act_dtype, m, k, q, scale, group, bias, n, y, nullptr, 0, FP8W_PATH_AUTO, stream);
}

fp8w_status_t fp8w_linear_grouped_with_path(const void* x, fp8w_dtype_t act_dtype, int64_t m, int64_t k,
                                            const uint8_t* q, const float* scale, int64_t group, const void* bias,
                                            int64_t n, void* y, int path, hipStream_t stream)
{
    return run_linear_grouped(x, act_dtype, m, k, q, scale, group, bias, n, y, nullptr, 0, path, stream);
}

fp8w_status_t fp8w_linear_grouped_with_workspace(const void* x, fp8w_dtype_t act_dtype, int64_t m, int64_t k,
                                                 const uint8_t* q, const float* scale, int64_t group,
                                                 const void* bias, int64_t n, void* y, void* workspace,
                                                 size_t workspace_bytes, int path, hipStream_t stream)
{
    return run_linear_grouped(x, act_dtype, m, k, q, scale, group, bias, n, y, workspace, workspace_bytes, path,
                              stream);
}

size_t fp8w_linear_grouped_workspace_bytes(int64_t m, int64_t n, int64_t k, int64_t group, fp8w_dtype_t act_dtype,
                                           const void* x, const uint8_t* q)
{
    if (!valid_act(act_dtype) || !sizes_ok(m, n, k) || !valid_group(k, group))
        return 0;
    if (auto_path_grouped(m, k, x, q) != FP8W_PATH_BATCH)
        return 0;
    return fp8w::batch_grouped_workspace_bytes(m, n, k, group);
}

int fp8w_linear_grouped_path(int64_t m, int64_t n, int64_t k, int64_t group, fp8w_dtype_t act_dtype,
                             const void* x, const uint8_t* q)
{
    if (!valid_act(act_dtype) || !sizes_ok(m, n, k) || !valid_group(k, group))
        return -1;
    return auto_path_grouped(m, k, x, q);
}

const char* fp8w_linear_grouped_kernel(int path, int64_t m, int64_t n, int64_t k, int64_t group,
                                       fp8w_dtype_t act_dtype, const void* x, const uint8_t* q)
{
    if (!valid_act(act_dtype) || !sizes_ok(m, n, k) || !valid_group(k, group))
        return nullptr;
    if (path == FP8W_PATH_AUTO)
        path = auto_path_grouped(m, k, x, q);
    if (path == FP8W_PATH_GEMV || path == FP8W_PATH_SKINNY) {
        if ((path == FP8W_PATH_GEMV && m != 1) || m < 1 || m > 32 || k % 256 != 0 || k == 0)
            return nullptr;
        return fp8w::grouped_kernel_name(path, m, n, k, group, false);
    }
    if (path == FP8W_PATH_BATCH)
        return m >= 1 && fast_k(k) ? fp8w::grouped_kernel_name(3, m, n, k, group, auto_path_grouped(m, k, x, q) == FP8W_PATH_BATCH) : nullptr;
    if (path == FP8W_PATH_FALLBACK)
        return fp8w::grouped_kernel_name(2, m, n, k, group, false);
    return nullptr;
}

fp8w_status_t fp8w_quantize_activations(const void* x, fp8w_dtype_t act_dtype, int64_t m, int64_t k, uint8_t* qx,
                                        float* sx, hipStream_t stream)
{
    if (!valid_act(act_dtype) || !sizes_ok(m, 0, k))
        return FP8W_ERR_INVALID_VALUE;
    if (m == 0)
        return FP8W_SUCCESS;
    if (!sx || (k > 0 && (!x || !qx)))
        return FP8W_ERR_INVALID_VALUE;
    if (!aligned(x, 2) || !aligned(sx, 4))
        return FP8W_ERR_MISALIGNED;
    const size_t xbytes = (size_t)m * (size_t)k * 2, qbytes = (size_t)m * (size_t)k;
    if (overlap(qx, qbytes, x, xbytes) || overlap(sx, (size_t)m * 4, x, xbytes) ||
        overlap(sx, (size_t)m * 4, qx, qbytes))
        return FP8W_ERR_INVALID_VALUE;
    return hip_status(fp8w::launch_quantize(x, act_of(act_dtype), m, k, qx, sx, stream));
}

// Every check of the W8A8 GEMM's arguments, run before anything is enqueued
// (fp8w_linear_w8a8 runs it on its workspace pointers before it launches the
// activation quantizer).
static fp8w_status_t check_gemm_w8a8(const uint8_t* qx, const float* sx, int64_t m, int64_t k, const uint8_t* qw,
                                     const float* sw, const void* bias, int64_t n, const void* y,
                                     fp8w_dtype_t out_dtype)
{
    if (!valid_act(out_dtype) || !sizes_ok(m, n, k) || k == 0 || k % 256 != 0)
        return FP8W_ERR_INVALID_VALUE;
    if (m == 0 || n == 0)
        return FP8W_SUCCESS;
    if (!qx || !sx || !qw || !sw || !y)
        return FP8W_ERR_INVALID_VALUE;
    if (!aligned(qx, 16) || !aligned(qw, 16) || !aligned(sx, 4) || !aligned(sw, 4) || !aligned(y, 2) ||
        !aligned(bias, 2))
        return FP8W_ERR_MISALIGNED;
    const size_t ybytes = (size_t)m * (size_t)n * 2;
    if (overlap(y, ybytes, qx, (size_t)m * (size_t)k) || overlap(y, ybytes, qw, (size_t)n * (size_t)k) ||
        overlap(y, ybytes, sx, (size_t)m * 4) || overlap(y, ybytes, sw, (size_t)n * 4) ||
        overlap(y, ybytes, bias, bias ? (size_t)n * 2 : 0))
        return FP8W_ERR_INVALID_VALUE;
    return FP8W_SUCCESS;
}

fp8w_status_t fp8w_gemm_w8a8(const uint8_t* qx, const float* sx, int64_t m, int64_t k, const uint8_t* qw,
                             const float* sw, const void* bias, int64_t n, void* y, fp8w_dtype_t out_dtype,
                             hipStream_t stream)
{
    const fp8w_status_t st = check_gemm_w8a8(qx, sx, m, k, qw, sw, bias, n, y, out_dtype);
    if (st != FP8W_SUCCESS || m == 0 || n == 0)
        return st;
    return hip_status(fp8w::launch_w8a8(qx, sx, m, k, qw, sw, bias, n, y, act_of(out_dtype), stream));
}

size_t fp8w_linear_w8a8_workspace_bytes(int64_t m, int64_t k)
{
    if (!sizes_ok(m, 0, k))
        return 0;
    return (((size_t)m * (size_t)k + 255) & ~(size_t)255) + (size_t)m * 4;
}

fp8w_status_t fp8w_linear_w8a8(const void* x, fp8w_dtype_t act_dtype, int64_t m, int64_t k, const uint8_t* qw,
                               const float* sw, const void* bias, int64_t n, void* y, void* workspace,
                               size_t workspace_bytes, hipStream_t stream)
{
    if (!valid_act(act_dtype) || !sizes_ok(m, n, k) || k == 0 || k % 256 != 0)
        return FP8W_ERR_INVALID_VALUE;
    if (m == 0 || n == 0)
        return FP8W_SUCCESS;
    const size_t need = fp8w_linear_w8a8_workspace_bytes(m, k);
    if (!workspace || workspace_bytes < need)
        return FP8W_ERR_WORKSPACE;
    if (!aligned(workspace, 16))
        return FP8W_ERR_MISALIGNED;
    if (!x || !y || !aligned(x, 2) || !aligned(y, 2))
        return x && y ? FP8W_ERR_MISALIGNED : FP8W_ERR_INVALID_VALUE;
    if (overlap(workspace, need, x, (size_t)m * (size_t)k * 2) || overlap(workspace, need, y, (size_t)m * (size_t)n * 2) ||
        overlap(workspace, need, qw, (size_t)n * (size_t)k) || overlap(workspace, need, sw, (size_t)n * 4) ||
        overlap(workspace, need, bias, bias ? (size_t)n * 2 : 0) ||
        overlap(y, (size_t)m * (size_t)n * 2, x, (size_t)m * (size_t)k * 2))
        return FP8W_ERR_INVALID_VALUE;
    uint8_t* qx = static_cast<uint8_t*>(workspace);
    float* sx = reinterpret_cast<float*>(qx + (need - (size_t)m * 4));
    fp8w_status_t st = check_gemm_w8a8(qx, sx, m, k, qw, sw, bias, n, y, act_dtype);
    if (st != FP8W_SUCCESS)
        return st;
    st = fp8w_quantize_activations(x, act_dtype, m, k, qx, sx, stream);
    if (st != FP8W_SUCCESS)
        return st;
    return fp8w_gemm_w8a8(qx, sx, m, k, qw, sw, bias, n, y, act_dtype, stream);
}

const char* fp8w_linear_w8a8_kernel(int64_t m, int64_t n, int64_t k)
{
    if (!sizes_ok(m, n, k) || m < 1 || n < 1 || k == 0 || k % 256 != 0)
        return nullptr;
    return fp8w::w8a8_kernel_name(m, n, k);
}

fp8w_status_t fp8w_fnuz_to_ocp(const uint8_t* src, int64_t count, uint8_t* dst, hipStream_t stream)
{
    if (count < 0 || count > kMaxElems)
        return FP8W_ERR_INVALID_VALUE;
    if (count == 0)
        return FP8W_SUCCESS;
    if (!src || !dst)
        return FP8W_ERR_INVALID_VALUE;
    if (src != dst && overlap(src, (size_t)count, dst, (size_t)count))
        return FP8W_ERR_INVALID_VALUE;
    return hip_status(fp8w::launch_fnuz_to_ocp(src, count, dst, stream));
}

fp8w_status_t fp8w_dequantize_grouped(const uint8_t* q, const float* scale, int64_t group, int64_t n, int64_t k,
                                      void* out, fp8w_dtype_t out_dtype, hipStream_t stream)
{
    if (!valid_dtype(out_dtype) || !sizes_ok(0, n, k) || !valid_group(k, group))
        return FP8W_ERR_INVALID_VALUE;
    if (n == 0 || k == 0)
        return FP8W_SUCCESS;
    if (!q || !scale || !out)
        return FP8W_ERR_INVALID_VALUE;
    const size_t eb = (size_t)elem_bytes(out_dtype);
    if (!aligned(out, eb) || !aligned(scale, 4))
        return FP8W_ERR_MISALIGNED;
    const size_t obytes = (size_t)n * (size_t)k * eb;
    if (overlap(out, obytes, q, (size_t)n * (size_t)k) || overlap(out, obytes, scale, group_scale_bytes(n, k, group)))
        return FP8W_ERR_INVALID_VALUE;
    return hip_status(fp8w::launch_dequantize_grouped(q, scale, group, n, k, out, act_of(out_dtype), stream));
}

fp8w_status_t fp8w_quantize(const void* w, fp8w_dtype_t w_dtype, int64_t n, int64_t k, uint8_t* q, float* scale,
                            hipStream_t stream)
{
    if (!valid_dtype(w_dtype) || !sizes_ok(0, n, k))
        return FP8W_ERR_INVALID_VALUE;
    if (n == 0)
        return FP8W_SUCCESS;
    if (!scale || (k > 0 && (!w || !q)))
        return FP8W_ERR_INVALID_VALUE;
    const size_t eb = (size_t)elem_bytes(w_dtype);
    if (!aligned(w, eb) || !aligned(scale, 4))
        return FP8W_ERR_MISALIGNED;
    const size_t wbytes = (size_t)n * (size_t)k * eb;
    if (overlap(q, (size_t)n * (size_t)k, w, wbytes) || overlap(scale, (size_t)n * 4, w, wbytes) ||
        overlap(scale, (size_t)n * 4, q, (size_t)n * (size_t)k))
        return FP8W_ERR_INVALID_VALUE;

    fp8w_status_t st = hip_status(fp8w::launch_quantize(w, act_of(w_dtype), n, k, q, scale, stream));
    if (st != FP8W_SUCCESS)
        return st;
    std::vector<float> host((size_t)n);
    st = hip_status(hipMemcpyAsync(host.data(), scale, (size_t)n * 4, hipMemcpyDeviceToHost, stream));
    if (st != FP8W_SUCCESS)
        return st;
    st = hip_status(hipStreamSynchronize(stream));
    if (st != FP8W_SUCCESS)
        return st;
    for (float s : host)
        if (!isfinite(s))
            return FP8W_ERR_NONFINITE;
    return FP8W_SUCCESS;
}

fp8w_status_t fp8w_linear(const void* x, fp8w_dtype_t act_dtype, int64_t m, int64_t k, const uint8_t* q,
                          const float* scale, const void* bias, int64_t n, void* y, void* workspace,
                          size_t workspace_bytes, hipStream_t stream)
{
    return run_linear(x, act_dtype, m, k, q, scale, bias, n, y, workspace, workspace_bytes, FP8W_PATH_AUTO,
                      stream);
}

fp8w_status_t fp8w_linear_with_path(const void* x, fp8w_dtype_t act_dtype, int64_t m, int64_t k,
                                    const uint8_t* q, const float* scale, const void* bias, int64_t n, void* y,
                                    void* workspace, size_t workspace_bytes, int path, hipStream_t stream)
{
    if (path < FP8W_PATH_AUTO || path > FP8W_PATH_BATCH)
        return FP8W_ERR_INVALID_VALUE;
    return run_linear(x, act_dtype, m, k, q, scale, bias, n, y, workspace, workspace_bytes, path, stream);
}

fp8w_status_t fp8w_dequantize_fallback(const uint8_t* q, const float* scale, int64_t n, int64_t k, void* out,
                                       fp8w_dtype_t out_dtype, hipStream_t stream)
{
    if (!valid_dtype(out_dtype) || !sizes_ok(0, n, k))
        return FP8W_ERR_INVALID_VALUE;
    if (n == 0 || k == 0)
        return FP8W_SUCCESS;
    if (!q || !out)
        return FP8W_ERR_INVALID_VALUE;
    const size_t eb = (size_t)elem_bytes(out_dtype);
    if (!aligned(out, eb) || !aligned(scale, 4))
        return FP8W_ERR_MISALIGNED;
    const size_t obytes = (size_t)n * (size_t)k * eb;
    if (overlap(out, obytes, q, (size_t)n * (size_t)k) || overlap(out, obytes, scale, scale ? (size_t)n * 4 : 0))
        return FP8W_ERR_INVALID_VALUE;
    return hip_status(fp8w::launch_dequantize(q, scale, n, k, out, act_of(out_dtype), stream));
}

int fp8w_linear_path(int64_t m, int64_t n, int64_t k, fp8w_dtype_t act_dtype, const void* x, const uint8_t* q,
                     const void* y)
{
    (void)y;
    if (!valid_act(act_dtype) || !sizes_ok(m, n, k))
        return -1;
    return auto_path(m, k, x, q);
}

size_t fp8w_linear_workspace_bytes(int64_t m, int64_t n, int64_t k, fp8w_dtype_t act_dtype, const void* x,
                                   const uint8_t* q, const void* y)
{
    const int p = fp8w_linear_path(m, n, k, act_dtype, x, q, y);
    if (p == FP8W_PATH_SKINNY)
        return skinny_workspace(m, n, k, x, q);
    if (p == FP8W_PATH_BATCH)
        return fp8w::batch_workspace_bytes(m, n, k);
    if (p != FP8W_PATH_FALLBACK)
        return 0;
    return fallback_workspace(n, k, act_dtype);
}

size_t fp8w_linear_with_path_workspace_bytes(int path, int64_t m, int64_t n, int64_t k, fp8w_dtype_t act_dtype,
                                             const void* x, const uint8_t* q)
{
    if (!valid_act(act_dtype) || !sizes_ok(m, n, k))
        return 0;
    const int autop = auto_path(m, k, x, q);
    if (path == FP8W_PATH_AUTO)
        path = autop;
    if (path == FP8W_PATH_FALLBACK)
        return fallback_workspace(n, k, act_dtype);
    if (path == FP8W_PATH_SKINNY && autop == FP8W_PATH_SKINNY)
        return skinny_workspace(m, n, k, x, q);
    if (path == FP8W_PATH_BATCH && autop == FP8W_PATH_BATCH)
        return fp8w::batch_workspace_bytes(m, n, k);
    return 0;
}

const char* fp8w_linear_kernel(int path, int64_t m, int64_t n, int64_t k, fp8w_dtype_t act_dtype, const void* x,
                               const uint8_t* q)
{
    if (!valid_act(act_dtype) || !sizes_ok(m, n, k))
        return nullptr;
    if (path == FP8W_PATH_AUTO)
        path = auto_path(m, k, x, q);
    if (path == FP8W_PATH_SKINNY && ring4_shape(m, k, x, q))
        return fp8w::skinny_kernel_name(m, n, k, false, true, q);
    if (path == FP8W_PATH_GEMV && gemv8_shape(m, k, x, q))  // the chunking follows k and q's alignment
        return fp8w::gemv_kernel_name(n, k, q);
    if (path == FP8W_PATH_GEMV || path == FP8W_PATH_SKINNY) {
        if ((path == FP8W_PATH_GEMV && m != 1) || m < 1 || m > 32 || !fast_k(k))
            return nullptr;
        // 16-code chunks: a call here needs 16-byte aligned codes
        return path == FP8W_PATH_GEMV ? fp8w::gemv_kernel_name(n, k, nullptr)
                                      : fp8w::skinny_kernel_name(m, n, k, true);
    }
    if (path == FP8W_PATH_BATCH)  // the workspace fp8w_linear_workspace_bytes reports exists only on the batch path
        return m >= 1 && fast_k(k) ? fp8w::batch_kernel_name(m, n, k, auto_path(m, k, x, q) == FP8W_PATH_BATCH)
                                   : nullptr;
    if (path == FP8W_PATH_FALLBACK)
        return fp8w::fallback_kernel_name(m, n, k, x);
    return nullptr;
}

const char* fp8w_status_string(fp8w_status_t status)
{
    switch (status) {
    case FP8W_SUCCESS:
        return "success";
    case FP8W_ERR_INVALID_VALUE:
        return "invalid value (size, dtype, NULL pointer, overlapping buffers or path request)";
    case FP8W_ERR_MISALIGNED:
        return "misaligned pointer";
    case FP8W_ERR_NONFINITE:
        return "non-finite weight (NaN or infinity)";
    case FP8W_ERR_WORKSPACE:
        return "workspace missing or too small for the fallback path (fp8w_linear_noalloc: the call needs more "
               "than the library's static scratch buffer holds)";
    case FP8W_ERR_HIP:
        return "HIP runtime error";
    }
    return "unknown status";
}

fp8w_status_t fp8w_stream_read_probe(const void* p, size_t bytes, uint32_t* sink, hipStream_t stream)
{
    if (bytes == 0)
        return FP8W_SUCCESS;
    if (!p || !sink || bytes % 16 != 0 || bytes / 16 > (size_t)1 << 40)
        return FP8W_ERR_INVALID_VALUE;
    if (!aligned(p, 16) || !aligned(sink, 4))
        return FP8W_ERR_MISALIGNED;
    return hip_status(fp8w::launch_read_probe(p, bytes, sink, stream));
}

int fp8w_last_hip_error(void)
{
    return g_last_hip_error;
}

int fp8w_abi_version(void)
{
    return 1;
}

}  // extern "C"
