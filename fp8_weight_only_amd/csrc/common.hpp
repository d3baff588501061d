// Device-side helpers shared by the fp8w HIP kernels (gfx950 / CDNA4 only).
//
// The weight codes are OCP e4m3fn bytes (bias 7, largest finite 448, 0x7F/0xFF
// NaN), the format fixed by "B04 - Precision & Quantization", section "The
// numbers, derived rather than tabulated". gfx950's conversion instructions
// implement exactly this format (v_cvt_pk_f32_fp8, v_cvt_scalef32_pk_{bf16,f16}_fp8,
// v_cvt_pk_fp8_f32), so decoding is one instruction per two codes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8w {

// Note: __builtin_bit_cast is only ever applied to whole values here, never to
// a vector element expression such as v.y (clang lowers that form to a read of
// element 0).
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

// ------------------------------------------------------------------ loads
// 16 codes in one 128-bit load that bypasses reuse-oriented caching: the weight
// stream is read exactly once per call ("FP8 weight-only (precision:
// fp8_weights)", "Dequantise in registers": 128-bit loads of 16 codes, streamed).
__device__ __forceinline__ u32x4 load_stream16(const uint8_t* p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ u32x4 load16(const void* p)
{
    return *reinterpret_cast<const u32x4*>(p);
}

// ------------------------------------------------------------------ e4m3 decode
// Four codes (one dword, byte 0 first) to four fp32 values; exact.
__device__ __forceinline__ void decode4_f32(uint32_t w, float& v0, float& v1, float& v2, float& v3)
{
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
    v0 = lo.x;
    v1 = lo.y;
    v2 = hi.x;
    v3 = hi.y;
}

// ------------------------------------------------------------------ activation types
// Activations, biases and outputs travel as 16-bit patterns; these traits give
// the exact widening to fp32, the round-to-nearest-even narrowing, and the
// exact decode of four e4m3 codes into two packed 16-bit pairs (every e4m3 value
// is representable in bf16 and in fp16).
struct Bf16 {
    typedef bf16x8 vec8;
    __device__ __forceinline__ static float to_f32(uint16_t b)
    {
        return __builtin_bit_cast(float, (uint32_t)b << 16);
    }
    __device__ __forceinline__ static float lo_f32(uint32_t pair)
    {
        return __builtin_bit_cast(float, pair << 16);
    }
    __device__ __forceinline__ static float hi_f32(uint32_t pair)
    {
        return __builtin_bit_cast(float, pair & 0xffff0000u);
    }
    __device__ __forceinline__ static uint16_t from_f32(float f)
    {
        return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
    }
    __device__ __forceinline__ static u32x2 decode4(uint32_t w)
    {
        const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
        const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
        u32x2 r;
        r.x = __builtin_bit_cast(uint32_t, lo);
        r.y = __builtin_bit_cast(uint32_t, hi);
        return r;
    }
    __device__ __forceinline__ static f32x4 mfma(u32x4 a, u32x4 b, f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
};

struct F16 {
    typedef f16x8 vec8;
    __device__ __forceinline__ static float to_f32(uint16_t b)
    {
        return static_cast<float>(__builtin_bit_cast(_Float16, b));
    }
    __device__ __forceinline__ static float lo_f32(uint32_t pair)
    {
        return static_cast<float>(__builtin_bit_cast(_Float16, (uint16_t)(pair & 0xffffu)));
    }
    __device__ __forceinline__ static float hi_f32(uint32_t pair)
    {
        return static_cast<float>(__builtin_bit_cast(_Float16, (uint16_t)(pair >> 16)));
    }
    __device__ __forceinline__ static uint16_t from_f32(float f)
    {
        return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
    }
    __device__ __forceinline__ static u32x2 decode4(uint32_t w)
    {
        const f16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
        const f16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
        u32x2 r;
        r.x = __builtin_bit_cast(uint32_t, lo);
        r.y = __builtin_bit_cast(uint32_t, hi);
        return r;
    }
    __device__ __forceinline__ static f32x4 mfma(u32x4 a, u32x4 b, f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
};

// ------------------------------------------------------------------ reductions
__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        v += __shfl_xor(v, off, kWave);
    return v;
}

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        v = fmaxf(v, __shfl_xor(v, off, kWave));
    return v;
}

// ------------------------------------------------------------------ epilogue
// y = round_to_dtype(scale * acc + bias), in fp32 with one final rounding
// ("FP8 weight-only (precision: fp8_weights)", "The contract").
template <typename Act>
__device__ __forceinline__ uint16_t epilogue(float acc, float scale, const uint16_t* bias, int64_t ch)
{
    const float b = bias ? Act::to_f32(bias[ch]) : 0.0f;
    return Act::from_f32(__builtin_fmaf(scale, acc, b));
}

// The same with scale and bias already in registers: the streaming kernels
// fetch them when they start, so that the end of every workgroup does not
// wait for one more memory round trip.
template <typename Act>
__device__ __forceinline__ uint16_t epilogue(float acc, float scale, uint16_t bias_bits)
{
    return Act::from_f32(__builtin_fmaf(scale, acc, Act::to_f32(bias_bits)));
}

// Raw bias bits of channel ch (+0.0 without a bias), widened only where the
// epilogue uses them so that the load is not waited for early. The load is
// unconditional (a pointer select, no branch): without a bias it reads a zero
// held in device memory.
static __device__ uint16_t kNoBias = 0;  // never written; global address space

__device__ __forceinline__ uint16_t bias_bits(const uint16_t* bias, int64_t ch)
{
    const uint16_t* p = bias ? bias + ch : &kNoBias;
    return *p;
}

}  // namespace fp8w
