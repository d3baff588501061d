// M = 1 fp8-weight GEMV: y[n] = scale[n] * sum_k x[k] * value(q[n,k]) + bias[n].
//
// "FP8 weight-only (precision: fp8_weights)", section "Dequantise in
// registers": 128-bit streaming loads of 16 codes, exact hardware conversion of
// each code to fp32, fp32 FMA, a cross-lane reduction and the scale in the
// epilogue ("The contract": fp32 accumulation, scale and bias in fp32, one
// rounding). Batch-1 decode is bound by the bytes of the weight stream ("B04 -
// Precision & Quantization", "Worked example: batch-1 decode is a bandwidth
// problem"), so everything here serves to keep enough 128-bit code loads in
// flight on all 256 CUs.
//
// Layout: one wave (64 lanes) owns ROWS consecutive output rows. Lane l of the
// wave reads the 16-code chunks l, l+64, l+128, ... of each of its rows, so one
// load instruction covers 1 KiB of one row; ROWS x U chunk loads per lane are
// issued before any of them is consumed. The activation chunk a lane needs is
// the same for all ROWS rows and is read once per chunk (L2/L1 resident: the
// whole x vector is a few KiB). Four waves per workgroup; consecutive
// workgroups stream consecutive row blocks.
#include "common.hpp"
#include "kernels.hpp"

namespace fp8w {
namespace {

constexpr int kWavesPerBlock = 4;

template <typename A, int ROWS, int U>
__global__ __launch_bounds__(kWavesPerBlock * kWave) void gemv_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ q, const float* __restrict__ scale,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ y, int64_t n, int64_t k)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t row0 = ((int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6)) * ROWS;
    if (row0 >= n)
        return;
    const int64_t nch = k >> 4;  // 16-code chunks per row

    const uint8_t* qr[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; ++r)
        qr[r] = q + (row0 + r < n ? row0 + r : n - 1) * k;

    float acc[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; ++r)
        acc[r] = 0.0f;

    for (int64_t c0 = 0; c0 < nch; c0 += kWave * U) {
        u32x4 code[ROWS][U];
        u32x4 xv[U][2];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t c = c0 + lane + kWave * u;
            const bool ok = c < nch;
#pragma unroll
            for (int r = 0; r < ROWS; ++r)
                code[r][u] = ok ? load_stream16(qr[r] + c * 16) : u32x4{0u, 0u, 0u, 0u};
            xv[u][0] = ok ? load16(x + c * 16) : u32x4{0u, 0u, 0u, 0u};
            xv[u][1] = ok ? load16(x + c * 16 + 8) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float xf[16];
            const uint32_t xw[8] = {xv[u][0].x, xv[u][0].y, xv[u][0].z, xv[u][0].w,
                                    xv[u][1].x, xv[u][1].y, xv[u][1].z, xv[u][1].w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                xf[2 * e + 0] = A::lo_f32(xw[e]);
                xf[2 * e + 1] = A::hi_f32(xw[e]);
            }
#pragma unroll
            for (int r = 0; r < ROWS; ++r) {
                const uint32_t cw[4] = {code[r][u].x, code[r][u].y, code[r][u].z, code[r][u].w};
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    float w0, w1, w2, w3;
                    decode4_f32(cw[d], w0, w1, w2, w3);
                    acc[r] = __builtin_fmaf(xf[4 * d + 0], w0, acc[r]);
                    acc[r] = __builtin_fmaf(xf[4 * d + 1], w1, acc[r]);
                    acc[r] = __builtin_fmaf(xf[4 * d + 2], w2, acc[r]);
                    acc[r] = __builtin_fmaf(xf[4 * d + 3], w3, acc[r]);
                }
            }
        }
    }

    float mine = 0.0f;
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
        const float s = wave_sum(acc[r]);
        if (lane == r)
            mine = s;
    }
    const int64_t row = row0 + lane;
    if (lane < ROWS && row < n)
        y[row] = epilogue<A>(mine, scale[row], bias, row);
}

template <typename A>
hipError_t launch_typed(const void* x, int64_t k, const uint8_t* q, const float* scale, const void* bias,
                        int64_t n, void* y, hipStream_t stream)
{
    constexpr int ROWS = 4, U = 4;
    const int64_t rows_per_block = (int64_t)kWavesPerBlock * ROWS;
    const dim3 grid((unsigned)((n + rows_per_block - 1) / rows_per_block)), block(kWavesPerBlock * kWave);
    hipLaunchKernelGGL((gemv_kernel<A, ROWS, U>), grid, block, 0, stream,
                       static_cast<const uint16_t*>(x), q, scale, static_cast<const uint16_t*>(bias),
                       static_cast<uint16_t*>(y), n, k);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv(const void* x, Act act, int64_t k, const uint8_t* q, const float* scale,
                       const void* bias, int64_t n, void* y, hipStream_t stream)
{
    if (n == 0)
        return hipSuccess;
    if (act == Act::BF16)
        return launch_typed<Bf16>(x, k, q, scale, bias, n, y, stream);
    if (act == Act::FP16)
        return launch_typed<F16>(x, k, q, scale, bias, n, y, stream);
    return hipErrorInvalidValue;
}

}  // namespace fp8w
