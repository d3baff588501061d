// Fallback for shapes the fast kernels do not cover (k % 256 != 0, m > 32,
// unaligned pointers): "FP8 weight-only (precision: fp8_weights)", section
// "The contract", item "Fallback": take the dequantised weight through a plain
// GEMM with the same numerics.
//
// Same numerics here means: the codes are decoded *unscaled* into the
// activation dtype (exact, since every e4m3 value is a bf16 and an fp16
// value), the GEMM multiplies exactly in that dtype and accumulates in fp32 on
// the matrix cores, and the scale and bias are applied in the fp32 epilogue
// with one final rounding, exactly as on the fast path; only the summation
// order differs. Folding the scale into the bf16 weight instead would round
// every weight a second time.
//
// dequantize_kernel also serves the exported dequantize entry point
// (q.float() * scale[:, None], optionally rounded to bf16 / fp16).
#include "common.hpp"
#include "kernels.hpp"

namespace fp8w {
namespace {

constexpr int kDqThreads = 256;

struct OutF32 {
    __device__ __forceinline__ static void store(void* p, int64_t i, float v)
    {
        static_cast<float*>(p)[i] = v;
    }
    // 8 values to a 32-byte aligned address
    __device__ __forceinline__ static void store8(void* p, int64_t i, const float* v)
    {
        f32x4* d = reinterpret_cast<f32x4*>(static_cast<float*>(p) + i);
        d[0] = f32x4{v[0], v[1], v[2], v[3]};
        d[1] = f32x4{v[4], v[5], v[6], v[7]};
    }
};
template <typename A>
struct Out16 {
    __device__ __forceinline__ static void store(void* p, int64_t i, float v)
    {
        static_cast<uint16_t*>(p)[i] = A::from_f32(v);
    }
    // 8 values to a 16-byte aligned address
    __device__ __forceinline__ static void store8(void* p, int64_t i, const float* v)
    {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            w[e] = (uint32_t)A::from_f32(v[2 * e]) | ((uint32_t)A::from_f32(v[2 * e + 1]) << 16);
        *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(p) + i) = u32x4{w[0], w[1], w[2], w[3]};
    }
};

// One workgroup per row. VEC: k % 8 == 0, q 8-byte and out 16/32-byte aligned,
// so 8 codes per thread per iteration are one 64-bit load and one or two
// 128-bit stores. value(q) * scale is one fp32 multiply; with
// scale == nullptr the value is stored unscaled (exact in every out type).
template <typename O, bool VEC>
__global__ __launch_bounds__(kDqThreads) void dequantize_kernel(const uint8_t* __restrict__ q,
                                                                const float* __restrict__ scale, int64_t k,
                                                                void* __restrict__ out)
{
    const int64_t r = blockIdx.x;
    const int64_t base = r * k;
    const float s = scale ? scale[r] : 1.0f;
    const bool scaled = scale != nullptr;
    if (VEC) {
        for (int64_t j = (int64_t)threadIdx.x * 8; j < k; j += kDqThreads * 8) {
            const u32x2 c = *reinterpret_cast<const u32x2*>(q + base + j);
            float v[8];
            decode4_f32(c.x, v[0], v[1], v[2], v[3]);
            decode4_f32(c.y, v[4], v[5], v[6], v[7]);
            if (scaled) {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    v[e] = v[e] * s;
            }
            O::store8(out, base + j, v);
        }
    } else {
        for (int64_t j = threadIdx.x; j < k; j += kDqThreads) {
            float v0, v1, v2, v3;
            decode4_f32((uint32_t)q[base + j], v0, v1, v2, v3);
            O::store(out, base + j, scaled ? v0 * s : v0);
        }
    }
}

// Guarded MFMA GEMM: y[m, n] = epilogue(sum_k x[m,k] * wd[n,k]) with wd in the
// activation dtype. Workgroup = 16 channels x 16 tokens (grid.y over token
// tiles), WAVES waves split k in 32-wide steps, partials reduced through LDS
// in a fixed order. VEC: k % 8 == 0 and x, wd 16-byte aligned, so every
// 8-element group that lies inside the row is one 128-bit load; groups past
// the end of k (or past n / m) read as zeros.
template <typename A, int WAVES, bool VEC>
__global__ __launch_bounds__(WAVES* kWave) void fallback_gemm_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wd, const float* __restrict__ scale,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ y, int64_t m, int64_t n, int64_t k)
{
    __shared__ f32x4 part[WAVES][kWave];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x >> 6;
    const int i = lane & 15;
    const int g = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * 16;
    const int64_t m0 = (int64_t)blockIdx.y * 16;
    const bool chok = n0 + i < n;
    const bool tokok = m0 + i < m;
    const uint16_t* wrow = wd + (chok ? n0 + i : 0) * k;
    const uint16_t* xrow = x + (tokok ? m0 + i : 0) * k;

    const int64_t steps = (k + 31) / 32;
    const int64_t per = (steps + WAVES - 1) / WAVES;
    const int64_t s0 = (int64_t)wave * per;
    const int64_t s1 = (s0 + per < steps) ? s0 + per : steps;

    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int64_t s = s0; s < s1; ++s) {
        const int64_t kk = s * 32 + 8 * g;
        u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
        if (VEC) {
            if (kk < k) {  // k % 8 == 0: the group is either whole or absent
                if (chok)
                    a = load16(wrow + kk);
                if (tokok)
                    b = load16(xrow + kk);
            }
        } else {
            uint16_t av[8], bv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const bool in = kk + e < k;
                av[e] = (in && chok) ? wrow[kk + e] : (uint16_t)0;
                bv[e] = (in && tokok) ? xrow[kk + e] : (uint16_t)0;
            }
            a = u32x4{(uint32_t)av[0] | ((uint32_t)av[1] << 16), (uint32_t)av[2] | ((uint32_t)av[3] << 16),
                      (uint32_t)av[4] | ((uint32_t)av[5] << 16), (uint32_t)av[6] | ((uint32_t)av[7] << 16)};
            b = u32x4{(uint32_t)bv[0] | ((uint32_t)bv[1] << 16), (uint32_t)bv[2] | ((uint32_t)bv[3] << 16),
                      (uint32_t)bv[4] | ((uint32_t)bv[5] << 16), (uint32_t)bv[6] | ((uint32_t)bv[7] << 16)};
        }
        acc = A::mfma(a, b, acc);
    }

    part[wave][lane] = acc;
    __syncthreads();
    if (wave != 0)
        return;
    f32x4 sum = part[0][lane];
#pragma unroll
    for (int w = 1; w < WAVES; ++w)
        sum += part[w][lane];
    const int64_t tok = m0 + i;
    if (tok >= m)
        return;
    const float v[4] = {sum.x, sum.y, sum.z, sum.w};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int64_t c = n0 + 4 * g + r;
        if (c < n)
            y[tok * n + c] = epilogue<A>(v[r], scale[c], bias, c);
    }
}

template <typename O>
hipError_t dq_launch(const uint8_t* q, const float* scale, int64_t n, int64_t k, void* out, int out_bytes,
                     hipStream_t stream)
{
    const bool vec = (k % 8 == 0) && ((reinterpret_cast<uintptr_t>(q) & 7) == 0) &&
                     ((reinterpret_cast<uintptr_t>(out) & (uintptr_t)(out_bytes * 8 - 1)) == 0);
    const dim3 grid((unsigned)n), block(kDqThreads);
    if (vec)
        hipLaunchKernelGGL((dequantize_kernel<O, true>), grid, block, 0, stream, q, scale, k, out);
    else
        hipLaunchKernelGGL((dequantize_kernel<O, false>), grid, block, 0, stream, q, scale, k, out);
    return hipGetLastError();
}

template <typename A>
hipError_t gemm_launch(const void* x, int64_t m, int64_t k, const void* wd, const float* scale,
                       const void* bias, int64_t n, void* y, hipStream_t stream)
{
    constexpr int WAVES = 8;
    const bool vec = (k % 8 == 0) && ((reinterpret_cast<uintptr_t>(x) & 15) == 0) &&
                     ((reinterpret_cast<uintptr_t>(wd) & 15) == 0);
    const dim3 grid((unsigned)((n + 15) / 16), (unsigned)((m + 15) / 16)), block(WAVES * kWave);
    const uint16_t* xp = static_cast<const uint16_t*>(x);
    const uint16_t* wp = static_cast<const uint16_t*>(wd);
    const uint16_t* bp = static_cast<const uint16_t*>(bias);
    uint16_t* yp = static_cast<uint16_t*>(y);
    if (vec)
        hipLaunchKernelGGL((fallback_gemm_kernel<A, WAVES, true>), grid, block, 0, stream, xp, wp, scale, bp, yp,
                           m, n, k);
    else
        hipLaunchKernelGGL((fallback_gemm_kernel<A, WAVES, false>), grid, block, 0, stream, xp, wp, scale, bp,
                           yp, m, n, k);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dequantize(const uint8_t* q, const float* scale, int64_t n, int64_t k, void* out,
                             Act out_type, hipStream_t stream)
{
    if (n == 0 || k == 0)
        return hipSuccess;
    switch (out_type) {
    case Act::FP32:
        return dq_launch<OutF32>(q, scale, n, k, out, 4, stream);
    case Act::BF16:
        return dq_launch<Out16<Bf16>>(q, scale, n, k, out, 2, stream);
    case Act::FP16:
        return dq_launch<Out16<F16>>(q, scale, n, k, out, 2, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_fallback_gemm(const void* x, Act act, int64_t m, int64_t k, const void* wd,
                                const float* scale, const void* bias, int64_t n, void* y, hipStream_t stream)
{
    if (n == 0 || m == 0)
        return hipSuccess;
    if (act == Act::BF16)
        return gemm_launch<Bf16>(x, m, k, wd, scale, bias, n, y, stream);
    if (act == Act::FP16)
        return gemm_launch<F16>(x, m, k, wd, scale, bias, n, y, stream);
    return hipErrorInvalidValue;
}

}  // namespace fp8w
