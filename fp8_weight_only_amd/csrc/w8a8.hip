// W8A8: both operands e4m3, for batches far above the skinny kernels' 32 tokens
// (prefill), where the layer is bound by the matrix cores, not by the weight
// stream.
//
// "Skill: Write an FP8 Kernel", "Required reasoning process": step 2 (scale =
// amax / 448, codes of x / scale, saturating), step 4 (per-token activation
// scales: one amax per row of x), step 5 (fp32 accumulation; epilogue
// acc * scale_A[m] * scale_B[n], bias in fp32, one rounding to the output
// type) and its correctness requirements (scale_A by the row, scale_B by the
// column; scale = 0 needs no division). The activation quantizer is the
// weight quantizer run on the rows of x (launch_quantize); the weights are the
// per-channel codes and scales of fp8w_quantize.
//
// The GEMM uses gfx950's v_mfma_f32_32x32x64_f8f6f4 (e4m3 x e4m3, fp32
// accumulate; lane l holds 32 consecutive k of row l % 32, k half l / 32, and
// D[8j + 4(l / 32) + r][l % 32] at accumulator 4j + r). The weight rows are the
// A operand (channels) and the token rows the B operand, so a lane's four
// consecutive D rows are four consecutive channels of one token: one 8-byte
// store per fragment row. A workgroup of four waves owns BN channels x BM
// tokens; stages of 64 k of both tiles travel HBM/L2 -> LDS by direct
// global-to-LDS loads through the same NS-stage ring as the weight-only
// kernels (csrc/ring.hpp). In LDS every 64-byte row keeps its four 16-byte
// chunks rotated by row / 4, so the 16 lanes of each ds_read_b128 phase
// (rows i .. i+15, same chunk) hit 16 distinct bank groups.
#include <stdio.h>

#include "common.hpp"
#include "kernels.hpp"
#include "ring.hpp"

namespace fp8w {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int BN, int BM, int NS>
struct W8Cfg {
    static constexpr int FN = BN / 64;  // 32-channel fragments per wave (two waves along n)
    static constexpr int FM = BM / 64;  // 32-token fragments per wave (two waves along m)
    static constexpr int ABYTES = BN * 64;
    static constexpr int STAGE = (BN + BM) * 64;
    static constexpr int BLOCKS = (BN + BM) / 16;  // 1 KB load instructions per stage
    static constexpr int LOADS = BLOCKS / 4;       // per wave
    static_assert(BLOCKS % 4 == 0, "blocks split over four waves");
    static_assert(LOADS * (NS - 2) < 64, "vmcnt range");
};

template <int BN, int BM, int NS>
struct W8Pipe {
    using C = W8Cfg<BN, BM, NS>;
    const uint8_t* qw;  // [n, k]
    const uint8_t* qx;  // [m, k]
    int64_t n, m, k, n0, m0;
    int lane, wave, wn, wm;

    // Block b of the stage holds rows 16b .. 16b + 15 of the weight tile (b <
    // BN / 16) or of the token tile; lane l brings 16 bytes of row 16b + l / 4,
    // the chunk that belongs at slot l % 4 (chunk (slot - row / 4) mod 4).
    __device__ __forceinline__ void issue(int64_t s, uint8_t* buf) const
    {
        const int64_t kb = s * 64;
#pragma unroll
        for (int u = 0; u < C::LOADS; ++u) {
            const int b = wave * C::LOADS + u;
            const int r = 16 * b + (lane >> 2);  // row within the combined tile
            const int slot = lane & 3;
            const int chunk = (slot - (r >> 2)) & 3;
            const uint8_t* src;
            if (r < BN) {
                int64_t row = n0 + r;
                row = row < n ? row : n - 1;
                src = qw + row * k + kb + 16 * chunk;
            } else {
                int64_t row = m0 + (r - BN);
                row = row < m ? row : m - 1;
                src = qx + row * k + kb + 16 * chunk;
            }
            __builtin_amdgcn_global_load_lds((const void*)src, FP8W_LDS(buf + 1024 * b), 16, 0, 0);
        }
    }

    __device__ __forceinline__ i32x8 frag(const uint8_t* base, int row) const
    {
        const int h = lane >> 5;  // k half
        const uint8_t* p = base + 64 * row;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(p + 16 * ((2 * h + (row >> 2)) & 3));
        const u32x4 hi = *reinterpret_cast<const u32x4*>(p + 16 * ((2 * h + 1 + (row >> 2)) & 3));
        i32x8 v;
        v[0] = (int)lo.x;
        v[1] = (int)lo.y;
        v[2] = (int)lo.z;
        v[3] = (int)lo.w;
        v[4] = (int)hi.x;
        v[5] = (int)hi.y;
        v[6] = (int)hi.z;
        v[7] = (int)hi.w;
        return v;
    }

    __device__ __forceinline__ void compute(const uint8_t* buf, f32x16* acc) const
    {
        const int i = lane & 31;
        i32x8 a[C::FN], b[C::FM];
#pragma unroll
        for (int f = 0; f < C::FN; ++f)
            a[f] = frag(buf, wn * (BN / 2) + 32 * f + i);
#pragma unroll
        for (int f = 0; f < C::FM; ++f)
            b[f] = frag(buf + C::ABYTES, wm * (BM / 2) + 32 * f + i);
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
            for (int fm = 0; fm < C::FM; ++fm)
                acc[fn * C::FM + fm] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    a[fn], b[fm], acc[fn * C::FM + fm], 0, 0, 0, 0, 0, 0);
    }
};

// y[t, c] = out(fl32(fl32(acc * scale_x[t]) * scale_w[c]) + bias[c]).
// Requires k % (64 * NS) == 0; qw, qx 16-byte aligned.
template <typename A, int BN, int BM, int NS>
__global__ __launch_bounds__(256) void w8a8_kernel(const uint8_t* __restrict__ qx, const float* __restrict__ sx,
                                                  const uint8_t* __restrict__ qw, const float* __restrict__ sw,
                                                  const uint16_t* __restrict__ bias, uint16_t* __restrict__ y,
                                                  int64_t m, int64_t n, int64_t k)
{
    using P = W8Pipe<BN, BM, NS>;
    using C = typename P::C;
    __shared__ __attribute__((aligned(1024))) uint8_t b0[C::STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t b1[C::STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t b2[NS > 2 ? C::STAGE : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t b3[NS > 3 ? C::STAGE : 16];

    P p;
    p.qw = qw;
    p.qx = qx;
    p.n = n;
    p.m = m;
    p.k = k;
    p.n0 = (int64_t)blockIdx.x * BN;
    p.m0 = (int64_t)blockIdx.y * BM;
    p.lane = threadIdx.x & (kWave - 1);
    p.wave = threadIdx.x / kWave;
    p.wn = p.wave & 1;
    p.wm = p.wave >> 1;

    f32x16 acc[C::FN * C::FM];
#pragma unroll
    for (int f = 0; f < C::FN * C::FM; ++f)
        acc[f] = f32x16{0.0f};

    run_ring<NS, C::LOADS>(p, k / 64, b0, b1, b2, b3, acc);

    // epilogue: lane (i, h) holds channels c0 + 8j + 4h + r (r = 0..3) of token t
    const int i = p.lane & 31, h = p.lane >> 5;
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm) {
        const int64_t t = p.m0 + p.wm * (BM / 2) + 32 * fm + i;
        if (t >= m)
            continue;
        const float st = sx[t];
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn) {
            const f32x16 d = acc[fn * C::FM + fm];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t c0 = p.n0 + p.wn * (BN / 2) + 32 * fn + 8 * j + 4 * h;
                uint16_t o[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int64_t c = c0 + r < n ? c0 + r : n - 1;
                    const float v = (d[4 * j + r] * st) * sw[c];
                    o[r] = A::from_f32(v + A::to_f32(bias_bits(bias, c)));
                }
                uint16_t* dst = y + t * n + c0;
                if (c0 + 3 < n && ((reinterpret_cast<uintptr_t>(dst) & 7) == 0)) {
                    u32x2 pk;
                    pk.x = (uint32_t)o[0] | ((uint32_t)o[1] << 16);
                    pk.y = (uint32_t)o[2] | ((uint32_t)o[3] << 16);
                    *reinterpret_cast<u32x2*>(dst) = pk;
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (c0 + r < n)
                            dst[r] = o[r];
                }
            }
        }
    }
}

template <typename A, int BN, int BM, int NS>
hipError_t launch_w8(const uint8_t* qx, const float* sx, int64_t m, int64_t k, const uint8_t* qw, const float* sw,
                     const void* bias, int64_t n, void* y, hipStream_t stream)
{
    const dim3 grid((unsigned)((n + BN - 1) / BN), (unsigned)((m + BM - 1) / BM)), block(256);
    hipLaunchKernelGGL((w8a8_kernel<A, BN, BM, NS>), grid, block, 0, stream, qx, sx, qw, sw,
                       static_cast<const uint16_t*>(bias), static_cast<uint16_t*>(y), m, n, k);
    return hipGetLastError();
}

// 256 x 256 tiles when they still give a workgroup per CU, 128 x 128 otherwise.
bool w8a8_large_tile(int64_t m, int64_t n)
{
    return ((n + 255) / 256) * ((m + 255) / 256) >= 256;
}

}  // namespace

hipError_t launch_w8a8(const uint8_t* qx, const float* sx, int64_t m, int64_t k, const uint8_t* qw, const float* sw,
                       const void* bias, int64_t n, void* y, Act out, hipStream_t stream)
{
    if (m == 0 || n == 0)
        return hipSuccess;
    const bool large = w8a8_large_tile(m, n);
    if (out == Act::BF16)
        return large ? launch_w8<Bf16, 256, 256, 4>(qx, sx, m, k, qw, sw, bias, n, y, stream)
                     : launch_w8<Bf16, 128, 128, 4>(qx, sx, m, k, qw, sw, bias, n, y, stream);
    if (out == Act::FP16)
        return large ? launch_w8<F16, 256, 256, 4>(qx, sx, m, k, qw, sw, bias, n, y, stream)
                     : launch_w8<F16, 128, 128, 4>(qx, sx, m, k, qw, sw, bias, n, y, stream);
    return hipErrorInvalidValue;
}

const char* w8a8_kernel_name(int64_t m, int64_t n)
{
    return w8a8_large_tile(m, n) ? "w8a8_kernel<BN=256,BM=256,NS=4>" : "w8a8_kernel<BN=128,BM=128,NS=4>";
}

}  // namespace fp8w
