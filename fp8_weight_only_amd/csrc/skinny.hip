// M = 2..32 fp8-weight skinny GEMM on the matrix cores.
//
// "FP8 weight-only (precision: fp8_weights)", section "Dequantise in
// registers": from M = 2 the per-row FMA work of a GEMV turns ALU-bound, so the
// small-batch kernel runs the dot products on the matrix unit in the
// activations' type, with the weight as the 16-channel operand and the tokens
// as the narrow one; both operands use the same k permutation; each code is
// converted once (exactly: every e4m3 value is a bf16 and an fp16 value) and
// reused for every token; k is split across waves and the partial sums are
// reduced through on-chip memory. The epilogue is the contract's: fp32
// accumulate, scale and bias in fp32, one rounding.
//
// gfx950 form: v_mfma_f32_16x16x32_{bf16,f16}. For a 16x16x32 step lane l holds
// A[l % 16][8*(l/16) .. 8*(l/16)+7] (A = 16 channels x 32 k), B[8*(l/16) ..][l % 16]
// (B = 32 k x 16 tokens) and returns D[4*(l/16) + r][l % 16], r = 0..3.
//
// Per 64-k step a lane (i = l % 16, g = l / 16) makes one 128-bit streaming
// load of the 16 codes W[n0+i][kb+16g .. kb+16g+15]; codes 0..7 feed the first
// MFMA and 8..15 the second, and the activations x[j][...] of token j = i use
// the same two 8-element k groups, so A and B agree on the k permutation. One
// workgroup owns 16 output channels over the whole of k; its WAVES waves take
// contiguous k ranges and their 16x16 fp32 partial tiles are summed in a fixed
// order through LDS (deterministic, no atomics). M <= 16 pads the token
// operand with zeros; 16 < M <= 32 uses a second token tile (MT = 2) on the
// same decoded weight registers.
#include "common.hpp"
#include "kernels.hpp"

namespace fp8w {
namespace {

template <typename A, int MT, int WAVES, int U>
__global__ __launch_bounds__(WAVES* kWave) void skinny_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ q, const float* __restrict__ scale,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ y, int m, int64_t n, int64_t k)
{
    __shared__ f32x4 part[WAVES][MT][kWave];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x >> 6;
    const int i = lane & 15;
    const int g = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * 16;

    const int64_t ch = (n0 + i < n) ? n0 + i : n - 1;
    const uint8_t* qrow = q + ch * k + 16 * g;
    const uint16_t* xrow[MT];
    bool xok[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        const int j = i + 16 * t;
        xok[t] = j < m;
        xrow[t] = x + (int64_t)(xok[t] ? j : 0) * k + 16 * g;
    }

    const int64_t steps = k >> 6;
    const int64_t per = (steps + WAVES - 1) / WAVES;
    const int64_t s0 = (int64_t)wave * per;
    const int64_t s1 = (s0 + per < steps) ? s0 + per : steps;

    f32x4 acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t)
        acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    const u32x4 zero = {0u, 0u, 0u, 0u};
    for (int64_t s = s0; s < s1; s += U) {
        u32x4 cw[U];
        u32x4 xb[U][MT][2];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool ok = s + u < s1;
            const int64_t kb = (s + u) * 64;
            cw[u] = ok ? load_stream16(qrow + kb) : zero;
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const bool xk = ok && xok[t];
                xb[u][t][0] = xk ? load16(xrow[t] + kb) : zero;
                xb[u][t][1] = xk ? load16(xrow[t] + kb + 8) : zero;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const u32x2 d0 = A::decode4(cw[u].x);
            const u32x2 d1 = A::decode4(cw[u].y);
            const u32x2 d2 = A::decode4(cw[u].z);
            const u32x2 d3 = A::decode4(cw[u].w);
            const u32x4 a0 = {d0.x, d0.y, d1.x, d1.y};
            const u32x4 a1 = {d2.x, d2.y, d3.x, d3.y};
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                acc[t] = A::mfma(a0, xb[u][t][0], acc[t]);
                acc[t] = A::mfma(a1, xb[u][t][1], acc[t]);
            }
        }
    }

#pragma unroll
    for (int t = 0; t < MT; ++t)
        part[wave][t][lane] = acc[t];
    __syncthreads();
    if (wave != 0)
        return;

#pragma unroll
    for (int t = 0; t < MT; ++t) {
        f32x4 sum = part[0][t][lane];
#pragma unroll
        for (int w = 1; w < WAVES; ++w)
            sum += part[w][t][lane];
        const int tok = i + 16 * t;
        if (tok >= m)
            continue;
        const float v[4] = {sum.x, sum.y, sum.z, sum.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t c = n0 + 4 * g + r;
            if (c < n)
                y[(int64_t)tok * n + c] = epilogue<A>(v[r], scale[c], bias, c);
        }
    }
}

template <typename A, int MT>
hipError_t launch_mt(const void* x, int m, int64_t k, const uint8_t* q, const float* scale, const void* bias,
                     int64_t n, void* y, hipStream_t stream)
{
    constexpr int WAVES = 8, U = 4;
    const dim3 grid((unsigned)((n + 15) / 16)), block(WAVES * kWave);
    hipLaunchKernelGGL((skinny_kernel<A, MT, WAVES, U>), grid, block, 0, stream,
                       static_cast<const uint16_t*>(x), q, scale, static_cast<const uint16_t*>(bias),
                       static_cast<uint16_t*>(y), m, n, k);
    return hipGetLastError();
}

template <typename A>
hipError_t launch_typed(const void* x, int64_t m, int64_t k, const uint8_t* q, const float* scale,
                        const void* bias, int64_t n, void* y, hipStream_t stream)
{
    if (m <= 16)
        return launch_mt<A, 1>(x, (int)m, k, q, scale, bias, n, y, stream);
    return launch_mt<A, 2>(x, (int)m, k, q, scale, bias, n, y, stream);
}

}  // namespace

hipError_t launch_skinny(const void* x, Act act, int64_t m, int64_t k, const uint8_t* q,
                         const float* scale, const void* bias, int64_t n, void* y, hipStream_t stream)
{
    if (n == 0 || m == 0)
        return hipSuccess;
    if (m > 32)
        return hipErrorInvalidValue;
    if (act == Act::BF16)
        return launch_typed<Bf16>(x, m, k, q, scale, bias, n, y, stream);
    if (act == Act::FP16)
        return launch_typed<F16>(x, m, k, q, scale, bias, n, y, stream);
    return hipErrorInvalidValue;
}

}  // namespace fp8w
