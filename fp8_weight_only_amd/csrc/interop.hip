// E4M3FNUZ codes carried over to OCP e4m3fn codes.
//
// "B04 - Precision & Quantization": the format table's FNUZ row and the
// section "Hardware support, and where the vendors diverge". gfx942 stores
// e4m3 with bias 8 (maximum 240, 0x80 is its only NaN, there is no negative
// zero); the OCP format this library computes in has bias 7 (maximum 448,
// 0x7F/0xFF NaN, 0x80 = -0). The same bits decode a factor of two apart, so a
// checkpoint's codes are translated, not reinterpreted: each code becomes the
// OCP code of the same value, and the per-channel scales stay as they are.
//
// The FNUZ value of every finite pattern other than 0x7F/0xFF is exactly half
// its OCP value, so it is the hardware OCP decode times 0.5 (exact); 0x7F/0xFF
// are +-240 = OCP 0x77/0xF7. The OCP code of that value is the hardware
// round-to-nearest-even conversion (no value is out of range). The 16 patterns
// below 2^-6 with an odd mantissa fall exactly between two OCP subnormals and
// round to the even one (2^-10 away); every other value is kept exactly. NaN
// (0x80) becomes the OCP NaN 0x7F.
#include "common.hpp"
#include "kernels.hpp"

namespace fp8w {
namespace {

__device__ __forceinline__ uint32_t fnuz_to_ocp1(uint32_t c)
{
    if (c == 0x80u)
        return 0x7Fu;
    if ((c & 0x7Fu) == 0x7Fu)
        return (c & 0x80u) | 0x77u;
    const f32x2 v = __builtin_amdgcn_cvt_pk_f32_fp8(c, false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(0.5f * v.x, 0.0f, 0, false) & 0xFFu;
}

__device__ __forceinline__ uint32_t fnuz_to_ocp4(uint32_t w)
{
    return fnuz_to_ocp1(w & 0xFFu) | (fnuz_to_ocp1((w >> 8) & 0xFFu) << 8) |
           (fnuz_to_ocp1((w >> 16) & 0xFFu) << 16) | (fnuz_to_ocp1(w >> 24) << 24);
}

// 16 codes per thread where src and dst are 16-byte aligned (grid-stride), the
// rest one byte per thread.
__global__ __launch_bounds__(256) void fnuz_to_ocp_kernel(const uint8_t* src, uint8_t* dst, int64_t count,
                                                          int64_t head, int64_t vec_chunks)
{
    const int64_t stride = (int64_t)gridDim.x * 256;
    const int64_t t0 = (int64_t)blockIdx.x * 256 + threadIdx.x;
    for (int64_t i = t0; i < vec_chunks; i += stride) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(src + head + 16 * i);
        u32x4 o;
        o.x = fnuz_to_ocp4(v.x);
        o.y = fnuz_to_ocp4(v.y);
        o.z = fnuz_to_ocp4(v.z);
        o.w = fnuz_to_ocp4(v.w);
        *reinterpret_cast<u32x4*>(dst + head + 16 * i) = o;
    }
    const int64_t tail0 = head + 16 * vec_chunks;
    for (int64_t i = t0; i < head + (count - tail0); i += stride) {
        const int64_t e = i < head ? i : tail0 + (i - head);
        dst[e] = (uint8_t)fnuz_to_ocp1(src[e]);
    }
}

}  // namespace

hipError_t launch_fnuz_to_ocp(const uint8_t* src, int64_t count, uint8_t* dst, hipStream_t stream)
{
    if (count == 0)
        return hipSuccess;
    // the vector part starts where both pointers are 16-byte aligned, if they agree modulo 16
    int64_t head = 0, vec = 0;
    const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
    if ((a & 15) == (b & 15)) {
        head = (int64_t)((16 - (a & 15)) & 15);
        if (head > count)
            head = count;
        vec = (count - head) / 16;
    } else {
        head = count;
    }
    const int64_t work = vec > 0 ? vec : count;
    const int64_t blocks64 = (work + 255) / 256;
    const unsigned blocks = (unsigned)(blocks64 < 4096 ? (blocks64 > 0 ? blocks64 : 1) : 4096);
    hipLaunchKernelGGL(fnuz_to_ocp_kernel, dim3(blocks), dim3(256), 0, stream, src, dst, count, head, vec);
    return hipGetLastError();
}

}  // namespace fp8w
