// Fallback for shapes the fast kernels do not cover (k % 256 != 0 or k < 256,
// unaligned pointers) at any m, and for calls that force it: "FP8 weight-only
// (precision: fp8_weights)", section "The contract", item "Fallback": take the
// dequantised weight through a plain GEMM with the same numerics.
//
// Same numerics here means: the codes are decoded *unscaled* into the
// activation dtype (exact, since every e4m3 value is a bf16 and an fp16
// value), the GEMM multiplies exactly in that dtype and accumulates in fp32 on
// the matrix cores, and the scale and bias are applied in the fp32 epilogue
// with one final rounding, exactly as on the fast path; only the summation
// order differs. Folding the scale into the bf16 weight instead would round
// every weight a second time.
//
// The GEMM: when k % 8 == 0 and x and the workspace are 16-byte aligned (every
// row then starts on a 16-byte boundary; this covers k = 8200) wpipe_kernel
// streams the dequantised weight through the same direct-to-LDS ring as the
// fast skinny kernel; any other shape takes fallback_gemm_kernel, which reads
// element by element where it must.
//
// dequantize_kernel also serves the exported dequantize entry point
// (q.float() * scale[:, None], optionally rounded to bf16 / fp16).
#include <stdio.h>

#include "common.hpp"
#include "kernels.hpp"
#include "ring.hpp"

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
    // 8 values to a 16-byte aligned address, as a streaming (non-temporal)
    // store: the dequantised weight is read back once, right away, by the
    // fallback GEMM, which measured faster when these writes had drained to HBM
    // instead of lingering dirty in the memory-side cache
    __device__ __forceinline__ static void store8(void* p, int64_t i, const float* v)
    {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            w[e] = (uint32_t)A::from_f32(v[2 * e]) | ((uint32_t)A::from_f32(v[2 * e + 1]) << 16);
        __builtin_nontemporal_store(u32x4{w[0], w[1], w[2], w[3]},
                                    reinterpret_cast<u32x4*>(static_cast<uint16_t*>(p) + i));
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

// ---------------------------------------------------------------- wpipe_kernel
// XR activation rows per token tile (grid.y over tiles of XR tokens), CT waves
// of 16 channels, NS stage buffers; one stage is 128 k: per wave 16 weight
// rows x 256 bytes, plus XR activation rows x 256 bytes for the workgroup.
template <int XR, int CT, int NS>
struct WCfg {
    static_assert(XR % 4 == 0 && XR >= 4 && XR <= 32, "activation rows");
    static constexpr int MT = XR > 16 ? 2 : 1;
    static constexpr int W = CT;
    static constexpr int WROW = 16 * 256;
    static constexpr int XPART = XR * 256;
    static constexpr int STAGE = W * WROW + XPART;
    static constexpr int XLOADS = XR / 4;             // one 1 KB load holds 4 activation rows
    static constexpr int XPW = (XLOADS + W - 1) / W;  // duplicates fill the last round
    static constexpr int LOADS = 4 + XPW;
};

template <typename A, int XR, int CT, int NS>
struct WPipe {
    using C = WCfg<XR, CT, NS>;
    static constexpr int MT = C::MT;
    const uint16_t* x;
    const uint16_t* wd;
    int64_t m, n, k, n0, m0, S, rot;
    int lane, wave;

    // Stage s (staggered by rot, as in the fast kernel) into buf. Weight load j
    // puts rows 4j..4j+3 of this wave's tile, row r = 4j + l / 16 at slot l % 16
    // holding chunk (slot - r) mod 16 (8 values each); activation load p puts
    // token rows 4p..4p+3 the same way.
    __device__ __forceinline__ void issue(int64_t s, uint8_t* buf) const
    {
        int64_t sr = s + rot;  // s < S and rot < S
        sr = sr < S ? sr : sr - S;
        const int64_t kb = sr * 128;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 4 * j + (lane >> 4);
            const int chunk = ((lane & 15) - r) & 15;
            int64_t row = n0 + 16 * wave + r;
            row = row < n ? row : n - 1;
            __builtin_amdgcn_global_load_lds((const void*)(wd + row * k + kb + chunk * 8),
                                             FP8W_LDS(buf + wave * C::WROW + j * 1024), 16, 0, 2 /* non-temporal */);
        }
#pragma unroll
        for (int u = 0; u < C::XPW; ++u) {
            const int p = (wave * C::XPW + u) % C::XLOADS;
            const int t = 4 * p + (lane >> 4);
            const int chunk = ((lane & 15) - t) & 15;
            int64_t tok = m0 + t;
            tok = tok < m ? tok : m - 1;
            __builtin_amdgcn_global_load_lds((const void*)(x + tok * k + kb + chunk * 8),
                                             FP8W_LDS(buf + C::W * C::WROW + p * 1024), 16, 0, 0);
        }
    }

    // MFMA jj of the stage covers k 32jj .. 32jj + 31: lane (i, g) takes weights
    // 32jj + 8g .. +7 of channel i and the same activations of token i (+ 16 mt).
    __device__ __forceinline__ void compute(const uint8_t* buf, f32x4* acc) const
    {
        const int i = lane & 15, g = lane >> 4;
        const uint8_t* wb = buf + wave * C::WROW;
        const uint8_t* xb = buf + C::W * C::WROW;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const u32x4 a = *reinterpret_cast<const u32x4*>(wb + 16 * (16 * i + ((4 * jj + g + i) & 15)));
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int t = (i + 16 * mt) < XR ? (i + 16 * mt) : XR - 1;
                const u32x4 b = *reinterpret_cast<const u32x4*>(xb + 16 * (16 * t + ((4 * jj + g + t) & 15)));
                acc[mt] = A::mfma(a, b, acc[mt]);
            }
        }
    }
};

// The ring covers k_main = k - k % (128 * NS) (at least 128 * NS); the tail,
// fewer than 128 * NS values, is added in fp32 before the epilogue.
template <typename A, int XR, int CT, int NS>
__global__ __launch_bounds__(CT* kWave) void wpipe_kernel(const uint16_t* __restrict__ x,
                                                         const uint16_t* __restrict__ wd,
                                                         const float* __restrict__ scale,
                                                         const uint16_t* __restrict__ bias,
                                                         uint16_t* __restrict__ y, int64_t m, int64_t n, int64_t k)
{
    using P = WPipe<A, XR, CT, NS>;
    using C = typename P::C;
    constexpr int MT = C::MT;
    __shared__ __attribute__((aligned(1024))) uint8_t b0[C::STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t b1[C::STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t b2[NS > 2 ? C::STAGE : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t b3[NS > 3 ? C::STAGE : 16];
    P p;
    p.x = x;
    p.wd = wd;
    p.m = m;
    p.n = n;
    p.k = k;
    p.lane = threadIdx.x & (kWave - 1);
    p.wave = threadIdx.x / kWave;
    p.n0 = (int64_t)blockIdx.x * (16 * CT);
    p.m0 = (int64_t)blockIdx.y * XR;
    const int64_t k_main = k - k % (128 * NS);
    p.S = k_main / 128;
    p.rot = (int64_t)(blockIdx.x / 8) % p.S;

    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
        acc[mt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    run_ring<NS, C::LOADS>(p, p.S, b0, b1, b2, b3, acc);

    // D[4g + r][i]: channel 4g + r of this wave's tile, token i (+ 16 mt)
    const int i = p.lane & 15, g = p.lane >> 4;
    const int64_t ch0 = p.n0 + 16 * p.wave + 4 * g;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int64_t tok = p.m0 + i + 16 * mt;
        if (i + 16 * mt >= XR || tok >= m)
            continue;
        float v[4] = {acc[mt].x, acc[mt].y, acc[mt].z, acc[mt].w};
        const uint16_t* xr = x + tok * k;
        for (int64_t e = k_main; e < k; ++e) {
            const float xv = A::to_f32(xr[e]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t ch = ch0 + r < n ? ch0 + r : n - 1;
                v[r] = __builtin_fmaf(xv, A::to_f32(wd[ch * k + e]), v[r]);
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (ch0 + r < n)
                y[tok * n + ch0 + r] = epilogue<A>(v[r], scale[ch0 + r], bias, ch0 + r);
    }
}

template <typename A, int XR>
hipError_t wpipe_launch(const uint16_t* x, int64_t m, int64_t k, const uint16_t* wd, const float* scale,
                        const uint16_t* bias, int64_t n, uint16_t* y, int ns, hipStream_t stream)
{
    constexpr int CT = 4;
    const dim3 grid((unsigned)((n + 16 * CT - 1) / (16 * CT)), (unsigned)((m + XR - 1) / XR)), block(CT * kWave);
    if (ns == 2)
        hipLaunchKernelGGL((wpipe_kernel<A, XR, CT, 2>), grid, block, 0, stream, x, wd, scale, bias, y, m, n, k);
    else
        hipLaunchKernelGGL((wpipe_kernel<A, XR, CT, 4>), grid, block, 0, stream, x, wd, scale, bias, y, m, n, k);
    return hipGetLastError();
}

// Ring depth wpipe_kernel uses for this shape, 0 when it does not apply: rows
// must start on 16-byte boundaries and the ring needs at least NS stages.
int wpipe_stages(int64_t k, const void* x, const void* wd)
{
    if (k % 8 != 0 || (reinterpret_cast<uintptr_t>(x) & 15) != 0 || (reinterpret_cast<uintptr_t>(wd) & 15) != 0)
        return 0;
    if (k >= 128 * 4)
        return 4;
    return k >= 256 ? 2 : 0;
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
    const int ns = wpipe_stages(k, x, wd);
    if (ns != 0) {
        const uint16_t* xp = static_cast<const uint16_t*>(x);
        const uint16_t* wp = static_cast<const uint16_t*>(wd);
        const uint16_t* bp = static_cast<const uint16_t*>(bias);
        uint16_t* yp = static_cast<uint16_t*>(y);
        if (m <= 4)
            return wpipe_launch<A, 4>(xp, m, k, wp, scale, bp, n, yp, ns, stream);
        if (m <= 8)
            return wpipe_launch<A, 8>(xp, m, k, wp, scale, bp, n, yp, ns, stream);
        if (m <= 16)
            return wpipe_launch<A, 16>(xp, m, k, wp, scale, bp, n, yp, ns, stream);
        return wpipe_launch<A, 32>(xp, m, k, wp, scale, bp, n, yp, ns, stream);
    }
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

const char* fallback_kernel_name(int64_t m, int64_t n, int64_t k, const void* x)
{
    thread_local char name[96];
    const void* aligned_ws = reinterpret_cast<const void*>((uintptr_t)256);  // a workspace of the usual alignment
    const int ns = wpipe_stages(k, x, aligned_ws);
    if (ns == 0)
        return "dequantize_kernel+fallback_gemm_kernel";
    const int xr = m <= 4 ? 4 : m <= 8 ? 8 : m <= 16 ? 16 : 32;
    snprintf(name, sizeof name, "dequantize_kernel+wpipe_kernel<XR=%d,CT=4,NS=%d>", xr, ns);
    return name;
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
