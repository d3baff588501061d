// Build-time per-output-channel e4m3 quantizer.
//
// "FP8 weight-only (precision: fp8_weights)", section "The contract": one
// symmetric scale per output channel (a row of the [out, in] weight),
// scale = amax(|row|) / 448, codes = round-to-nearest-even(w / scale) in e4m3,
// clamped to +-448, computed once at build time. "Skill: Write an FP8 Kernel",
// "Required reasoning process" steps 2 and 4: amax over the row with a block
// reduction, the scale to a separate buffer, a saturating conversion; step 7:
// an all-zero row (scale 0) needs no division (its codes are all 0x00).
//
// One workgroup of 256 threads per row. Pass 1 reduces |w| to the row's amax
// (and flags NaN/inf); pass 2 encodes, from registers when the row fits (k up
// to 16384 with 16-byte alignment, the activation rows of the W8A8 path
// included), otherwise re-reading the row (mostly from L2).
// The quotient w / scale is an IEEE fp32 division (the compiler's correctly
// rounded sequence; no fast-math) and the result is clamped to +-448 in fp32
// before the hardware RNE conversion, so the conversion never sees an
// out-of-range value and the codes do not depend on its saturation mode.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace fp8w {
namespace {

constexpr int kThreads = 256;

// Weight element readers: fp32 as is, bf16/fp16 widened exactly.
struct WF32 {
    static constexpr int kBytes = 4;
    __device__ __forceinline__ static float at(const void* p, int64_t i)
    {
        return static_cast<const float*>(p)[i];
    }
    // 4 consecutive elements from a 16-byte aligned address
    __device__ __forceinline__ static void load4(const void* p, int64_t i, float* o)
    {
        const f32x4 d = *reinterpret_cast<const f32x4*>(static_cast<const float*>(p) + i);
        o[0] = d.x;
        o[1] = d.y;
        o[2] = d.z;
        o[3] = d.w;
    }
    // 16 consecutive elements from a 16-byte aligned address
    __device__ __forceinline__ static void load16(const void* p, int64_t i, float* o)
    {
        const f32x4* v = reinterpret_cast<const f32x4*>(static_cast<const float*>(p) + i);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const f32x4 d = v[j];
            o[4 * j + 0] = d.x;
            o[4 * j + 1] = d.y;
            o[4 * j + 2] = d.z;
            o[4 * j + 3] = d.w;
        }
    }
};

template <typename A>
struct W16 {
    static constexpr int kBytes = 2;
    __device__ __forceinline__ static float at(const void* p, int64_t i)
    {
        return A::to_f32(static_cast<const uint16_t*>(p)[i]);
    }
    // 4 consecutive elements from an 8-byte aligned address
    __device__ __forceinline__ static void load4(const void* p, int64_t i, float* o)
    {
        const u32x2 d = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(p) + i);
        o[0] = A::lo_f32(d.x);
        o[1] = A::hi_f32(d.x);
        o[2] = A::lo_f32(d.y);
        o[3] = A::hi_f32(d.y);
    }
    __device__ __forceinline__ static void load16(const void* p, int64_t i, float* o)
    {
        const u32x4* v = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(p) + i);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const u32x4 d = v[j];
            const uint32_t w4[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                o[8 * j + 2 * e + 0] = A::lo_f32(w4[e]);
                o[8 * j + 2 * e + 1] = A::hi_f32(w4[e]);
            }
        }
    }
};

__device__ __forceinline__ float clamp448(float t)
{
    return fminf(fmaxf(t, -448.0f), 448.0f);
}

// Four fp32 values -> four e4m3 codes in one dword (byte 0 = first value).
__device__ __forceinline__ uint32_t encode4(float a, float b, float c, float d)
{
    uint32_t p = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(a), clamp448(b), 0, false);
    p = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(c), clamp448(d), p, true);
    return p;
}

__device__ __forceinline__ uint8_t encode1(float a)
{
    return (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(clamp448(a), 0.0f, 0, false) & 0xffu);
}

// VEC: k % 16 == 0 and w, q 16-byte aligned, so every thread moves 16 elements
// per iteration (four or two 128-bit loads in, one 128-bit store out).
// U > 0 (VEC only, k <= U * 16 * kThreads): the row is read once and held in
// registers (U chunks of 16 elements per thread) between the amax and the
// encode, instead of a second read of the row; the arithmetic is the same.
template <typename W, bool VEC, int U = 0>
__global__ __launch_bounds__(kThreads) void quantize_rows_kernel(const void* __restrict__ w, int64_t k,
                                                                 uint8_t* __restrict__ q,
                                                                 float* __restrict__ scale)
{
    static_assert(U == 0 || VEC, "the register-resident row needs the vector path");
    __shared__ float wave_amax[kThreads / kWave];
    const int tid = threadIdx.x;
    const int64_t r = blockIdx.x;
    const int64_t base = r * k;

    // pass 1: amax and the non-finite flag
    float amax = 0.0f;
    int bad = 0;
    float held[U > 0 ? U : 1][16];
    if constexpr (U > 0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t j = ((int64_t)u * kThreads + tid) * 16;
            if (j < k) {
                W::load16(w, base + j, held[u]);
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const float a = fabsf(held[u][e]);
                    bad |= !(a <= 3.402823466e38f);
                    amax = fmaxf(amax, a);
                }
            }
        }
    } else if (VEC) {
        for (int64_t j = (int64_t)tid * 16; j < k; j += kThreads * 16) {
            float v[16];
            W::load16(w, base + j, v);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float a = fabsf(v[e]);
                bad |= !(a <= 3.402823466e38f);
                amax = fmaxf(amax, a);
            }
        }
    } else {
        for (int64_t j = tid; j < k; j += kThreads) {
            const float a = fabsf(W::at(w, base + j));
            bad |= !(a <= 3.402823466e38f);
            amax = fmaxf(amax, a);
        }
    }
    bad = __syncthreads_or(bad);
    amax = wave_max(amax);
    if ((tid & (kWave - 1)) == 0)
        wave_amax[tid / kWave] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(wave_amax[0], wave_amax[1]), fmaxf(wave_amax[2], wave_amax[3]));

    const float s = amax / 448.0f;
    if (tid == 0)
        scale[r] = bad ? __builtin_nanf("") : s;
    if (bad)
        return;  // uniform over the workgroup; the host reports the error

    // pass 2: codes
    auto encode16 = [&](const float* v) {
        u32x4 out = {0u, 0u, 0u, 0u};
        if (s != 0.0f) {
            out.x = encode4(v[0] / s, v[1] / s, v[2] / s, v[3] / s);
            out.y = encode4(v[4] / s, v[5] / s, v[6] / s, v[7] / s);
            out.z = encode4(v[8] / s, v[9] / s, v[10] / s, v[11] / s);
            out.w = encode4(v[12] / s, v[13] / s, v[14] / s, v[15] / s);
        }
        return out;
    };
    if constexpr (U > 0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t j = ((int64_t)u * kThreads + tid) * 16;
            if (j < k)
                *reinterpret_cast<u32x4*>(q + base + j) = encode16(held[u]);
        }
    } else if (VEC) {
        for (int64_t j = (int64_t)tid * 16; j < k; j += kThreads * 16) {
            float v[16];
            if (s != 0.0f)
                W::load16(w, base + j, v);
            *reinterpret_cast<u32x4*>(q + base + j) = encode16(v);
        }
    } else {
        for (int64_t j = tid; j < k; j += kThreads)
            q[base + j] = (s != 0.0f) ? encode1(W::at(w, base + j) / s) : (uint8_t)0;
    }
}

template <typename W>
hipError_t launch_typed(const void* w, int elem_bytes, int64_t n, int64_t k, uint8_t* q, float* scale,
                        hipStream_t stream)
{
    const bool vec = (k % 16 == 0) && ((reinterpret_cast<uintptr_t>(w) & 15) == 0) &&
                     ((reinterpret_cast<uintptr_t>(q) & 15) == 0) && ((k * elem_bytes) % 16 == 0);
    const dim3 grid((unsigned)n), block(kThreads);
    constexpr int64_t kChunk = 16 * kThreads;  // elements per register-resident chunk
    if (vec && k <= kChunk)
        hipLaunchKernelGGL((quantize_rows_kernel<W, true, 1>), grid, block, 0, stream, w, k, q, scale);
    else if (vec && k <= 2 * kChunk)
        hipLaunchKernelGGL((quantize_rows_kernel<W, true, 2>), grid, block, 0, stream, w, k, q, scale);
    else if (vec && k <= 4 * kChunk)
        hipLaunchKernelGGL((quantize_rows_kernel<W, true, 4>), grid, block, 0, stream, w, k, q, scale);
    else if (vec)
        hipLaunchKernelGGL((quantize_rows_kernel<W, true>), grid, block, 0, stream, w, k, q, scale);
    else
        hipLaunchKernelGGL((quantize_rows_kernel<W, false>), grid, block, 0, stream, w, k, q, scale);
    return hipGetLastError();
}

// ---------------------------------------------------------------- group scales
// One scale per run of G weights of a row (G = 32, 64 or 128; k % G == 0):
// "B04 - Precision & Quantization", section "Post-training quantization versus
// quantization-aware training" (per-group granularity), and the Day-98 lab
// page's "one scale per 32" census. Each group is quantized as the contract
// quantizes a row: scale = fl32(amax / 448), codes the RNE e4m3 of the IEEE
// quotient clamped to +-448, an all-zero group gets scale 0 and codes 0x00. A
// group with a NaN or infinite weight gets a NaN scale (codes unspecified).
//
// VEC: each thread takes 4 consecutive weights, so a group is G / 4 adjacent
// lanes of one wave and its amax is a butterfly over those lanes. Every lane
// runs every shuffle (lanes past the row's end carry zeros): k % G == 0, so a
// lane group is either wholly inside the row or wholly past it.
template <typename W, int G, bool VEC>
__global__ __launch_bounds__(kThreads) void quantize_groups_kernel(const void* __restrict__ w, int64_t k,
                                                                   uint8_t* __restrict__ q,
                                                                   float* __restrict__ scale)
{
    static_assert(G == 32 || G == 64 || G == 128, "group size");
    const int tid = threadIdx.x;
    const int64_t r = blockIdx.x;
    const int64_t base = r * k;
    const int64_t ng = k / G;
    if (VEC) {
        constexpr int LG = G / 4;  // lanes per group
        for (int64_t j0 = 0; j0 < k; j0 += kThreads * 4) {
            const int64_t j = j0 + (int64_t)tid * 4;
            const bool in = j < k;
            float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            if (in)
                W::load4(w, base + j, v);
            float amax = 0.0f;
            int bad = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float a = fabsf(v[e]);
                bad |= !(a <= 3.402823466e38f);
                amax = fmaxf(amax, a);
            }
#pragma unroll
            for (int off = 1; off < LG; off <<= 1) {
                amax = fmaxf(amax, __shfl_xor(amax, off, kWave));
                bad |= __shfl_xor(bad, off, kWave);
            }
            if (!in)
                continue;
            const float s = amax / 448.0f;
            if ((tid & (LG - 1)) == 0)
                scale[r * ng + j / G] = bad ? __builtin_nanf("") : s;
            if (bad)
                continue;
            const uint32_t out = (s != 0.0f) ? encode4(v[0] / s, v[1] / s, v[2] / s, v[3] / s) : 0u;
            *reinterpret_cast<uint32_t*>(q + base + j) = out;
        }
    } else {
        // any alignment: one thread per group
        for (int64_t g = tid; g < ng; g += kThreads) {
            const int64_t g0 = base + g * G;
            float amax = 0.0f;
            int bad = 0;
            for (int e = 0; e < G; ++e) {
                const float a = fabsf(W::at(w, g0 + e));
                bad |= !(a <= 3.402823466e38f);
                amax = fmaxf(amax, a);
            }
            const float s = amax / 448.0f;
            scale[r * ng + g] = bad ? __builtin_nanf("") : s;
            if (bad)
                continue;
            for (int e = 0; e < G; ++e)
                q[g0 + e] = (s != 0.0f) ? encode1(W::at(w, g0 + e) / s) : (uint8_t)0;
        }
    }
}

template <typename W, int G>
hipError_t launch_groups_g(const void* w, int64_t n, int64_t k, uint8_t* q, float* scale, hipStream_t stream)
{
    const bool vec = ((reinterpret_cast<uintptr_t>(w) & (4 * W::kBytes - 1)) == 0) &&
                     ((reinterpret_cast<uintptr_t>(q) & 3) == 0);
    const dim3 grid((unsigned)n), block(kThreads);
    if (vec)
        hipLaunchKernelGGL((quantize_groups_kernel<W, G, true>), grid, block, 0, stream, w, k, q, scale);
    else
        hipLaunchKernelGGL((quantize_groups_kernel<W, G, false>), grid, block, 0, stream, w, k, q, scale);
    return hipGetLastError();
}

template <typename W>
hipError_t launch_groups_typed(const void* w, int64_t n, int64_t k, int64_t group, uint8_t* q, float* scale,
                               hipStream_t stream)
{
    switch (group) {
    case 32: return launch_groups_g<W, 32>(w, n, k, q, scale, stream);
    case 64: return launch_groups_g<W, 64>(w, n, k, q, scale, stream);
    case 128: return launch_groups_g<W, 128>(w, n, k, q, scale, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_quantize_groups(const void* w, Act w_type, int64_t n, int64_t k, int64_t group, uint8_t* q,
                                  float* scale, hipStream_t stream)
{
    if (n == 0 || k == 0)
        return hipSuccess;
    switch (w_type) {
    case Act::FP32:
        return launch_groups_typed<WF32>(w, n, k, group, q, scale, stream);
    case Act::BF16:
        return launch_groups_typed<W16<Bf16>>(w, n, k, group, q, scale, stream);
    case Act::FP16:
        return launch_groups_typed<W16<F16>>(w, n, k, group, q, scale, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_quantize(const void* w, Act w_type, int64_t n, int64_t k, uint8_t* q, float* scale,
                           hipStream_t stream)
{
    if (n == 0)
        return hipSuccess;
    switch (w_type) {
    case Act::FP32:
        return launch_typed<WF32>(w, 4, n, k, q, scale, stream);
    case Act::BF16:
        return launch_typed<W16<Bf16>>(w, 2, n, k, q, scale, stream);
    case Act::FP16:
        return launch_typed<W16<F16>>(w, 2, n, k, q, scale, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace fp8w
