// M = 2..32 fp8-weight skinny GEMM on the matrix cores (v_mfma_f32_16x16x32_{bf16,f16}).
//
// "FP8 weight-only (precision: fp8_weights)", section "Dequantise in
// registers": from M = 2 a GEMV's per-row FMA work turns ALU-bound, so the
// small-batch kernel runs the dot products on the matrix unit in the
// activations' type, with the weight as the channel operand and the tokens as
// the narrow one; both operands use the same k permutation; each code is
// converted once (exactly: every e4m3 value is a bf16 and an fp16 value) and
// reused for every token; k is split across waves and the partial sums are
// reduced through LDS. The epilogue is the contract's: fp32 accumulation,
// scale and bias in fp32, one rounding.
//
// gfx950 MFMA 16x16x32 lane layout: lane l holds A[l % 16][8*(l/16) + e] and
// B[8*(l/16) + e][l % 16] (e = 0..7) and returns D[4*(l/16) + r][l % 16]
// (r = 0..3). Loaded naively (lane l reads 16 bytes of row l % 16), each
// quarter-wave would touch 16 different rows, and the vector memory unit's
// per-cache-line work, not HBM, would set the speed. Two layouts avoid that:
//
// * seg_kernel (M <= 8, and 17..32 on wide layers): one MFMA covers MP = 16/SEG
//   channels x MP tokens x SEG k-segments. A row i = MP*s + c and B column
//   j = MP*s + t; only the D blocks with matching segment (s == s') are kept and
//   summed over s at the end. Lane (i, g) reads the 16 codes of channel c at
//   kb + 16*SEG*g + 16*s, so a quarter-wave reads 16*SEG contiguous bytes per
//   channel (64 B for M <= 4). T channel groups per wave share the activation
//   fragments; W waves split k.
// * lds_kernel (M = 9..32): codes and activations are read with fully
//   coalesced loads (a quarter-wave reads 256 contiguous bytes of one row),
//   written to a per-wave LDS tile and read back in the MFMA layout.
//
// One workgroup owns a block of output channels over the whole of k (no
// cross-workgroup reduction: on MI355X the eight XCDs have separate L2s and a
// device-scope handoff between workgroups costs more than it saves).
#include "common.hpp"
#include "kernels.hpp"

namespace fp8w {
namespace {

// ---------------------------------------------------------------- seg_kernel
template <typename A, int SEG, int T, int W, int U, int MT>
__global__ __launch_bounds__(W* kWave) void seg_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ q, const float* __restrict__ scale,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ y, int m, int64_t n, int64_t k)
{
    constexpr int MP = 16 / SEG;     // channels (and tokens) per MFMA
    constexpr int SPAN = 64 * SEG;   // k covered by one MFMA pair
    __shared__ float red[W][MT][T][16 * 16];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x >> 6;
    const int i = lane & 15, g = lane >> 4;
    const int c = i % MP, s = i / MP;
    const int64_t n0 = (int64_t)blockIdx.x * (MP * T);
    const int64_t lane_k = 16 * SEG * g + 16 * s;

    const uint8_t* qp[T];
#pragma unroll
    for (int tg = 0; tg < T; ++tg) {
        const int64_t r = n0 + MP * tg + c;
        qp[tg] = q + (r < n ? r : n - 1) * k + lane_k;
    }
    const uint16_t* xp[MT];
    bool xok[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int tok = c + MP * mt;
        xok[mt] = tok < m;
        xp[mt] = x + (int64_t)(xok[mt] ? tok : 0) * k + lane_k;
    }

    const int64_t steps = k / SPAN;
    const int64_t per = (steps + W - 1) / W;
    const int64_t s0 = (int64_t)wave * per;
    const int64_t s1 = (s0 + per < steps) ? s0 + per : steps;

    f32x4 acc[MT][T];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int tg = 0; tg < T; ++tg)
            acc[mt][tg] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    const u32x4 zero = {0u, 0u, 0u, 0u};
    int64_t st = s0;
    for (; st + U <= s1; st += U) {
        u32x4 cw[U][T];
        u32x4 xb[U][MT][2];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t off = (st + u) * SPAN;
#pragma unroll
            for (int tg = 0; tg < T; ++tg)
                cw[u][tg] = load_stream16(qp[tg] + off);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                xb[u][mt][0] = xok[mt] ? load16(xp[mt] + off) : zero;
                xb[u][mt][1] = xok[mt] ? load16(xp[mt] + off + 8) : zero;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int tg = 0; tg < T; ++tg) {
                const u32x2 d0 = A::decode4(cw[u][tg].x), d1 = A::decode4(cw[u][tg].y);
                const u32x2 d2 = A::decode4(cw[u][tg].z), d3 = A::decode4(cw[u][tg].w);
                const u32x4 a0 = {d0.x, d0.y, d1.x, d1.y};
                const u32x4 a1 = {d2.x, d2.y, d3.x, d3.y};
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    acc[mt][tg] = A::mfma(a0, xb[u][mt][0], acc[mt][tg]);
                    acc[mt][tg] = A::mfma(a1, xb[u][mt][1], acc[mt][tg]);
                }
            }
    }
    for (; st < s1; ++st) {
        const int64_t off = st * SPAN;
        u32x4 xb[MT][2];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            xb[mt][0] = xok[mt] ? load16(xp[mt] + off) : zero;
            xb[mt][1] = xok[mt] ? load16(xp[mt] + off + 8) : zero;
        }
#pragma unroll
        for (int tg = 0; tg < T; ++tg) {
            const u32x4 cw = load_stream16(qp[tg] + off);
            const u32x2 d0 = A::decode4(cw.x), d1 = A::decode4(cw.y);
            const u32x2 d2 = A::decode4(cw.z), d3 = A::decode4(cw.w);
            const u32x4 a0 = {d0.x, d0.y, d1.x, d1.y};
            const u32x4 a1 = {d2.x, d2.y, d3.x, d3.y};
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                acc[mt][tg] = A::mfma(a0, xb[mt][0], acc[mt][tg]);
                acc[mt][tg] = A::mfma(a1, xb[mt][1], acc[mt][tg]);
            }
        }
    }

    // D[4g + r][i] of every (token tile, channel group) to LDS, row-major 16x16
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int tg = 0; tg < T; ++tg) {
            const float v[4] = {acc[mt][tg].x, acc[mt][tg].y, acc[mt][tg].z, acc[mt][tg].w};
#pragma unroll
            for (int r = 0; r < 4; ++r)
                red[wave][mt][tg][(4 * g + r) * 16 + i] = v[r];
        }
    __syncthreads();

    // this workgroup's outputs: MT*MP tokens x T*MP channels; sum over waves
    // and matching segments in a fixed order
    constexpr int NOUT = MT * MP * T * MP;
    for (int o = threadIdx.x; o < NOUT; o += W * kWave) {
        const int cc = o % MP;
        const int tg = (o / MP) % T;
        const int t = (o / (MP * T)) % MP;
        const int mt = o / (MP * T * MP);
        const int tok = t + MP * mt;
        const int64_t ch = n0 + MP * tg + cc;
        if (tok >= m || ch >= n)
            continue;
        float sum = 0.0f;
        for (int w = 0; w < W; ++w)
#pragma unroll
            for (int ss = 0; ss < SEG; ++ss)
                sum += red[w][mt][tg][(MP * ss + cc) * 16 + MP * ss + t];
        y[(int64_t)tok * n + ch] = epilogue<A>(sum, scale[ch], bias, ch);
    }
}

// ---------------------------------------------------------------- lds_kernel
constexpr int kCodeRow = 256 + 16;  // LDS code tile row stride (bytes): 256 codes + pad
constexpr int kActRow = 512 + 16;   // LDS activation tile row stride (bytes): 256 values + pad

template <typename A, int MT, int W>
__global__ __launch_bounds__(W* kWave) void lds_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ q, const float* __restrict__ scale,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ y, int m, int64_t n, int64_t k)
{
    __shared__ __attribute__((aligned(16))) uint8_t ctile_all[W][16 * kCodeRow];
    __shared__ __attribute__((aligned(16))) uint8_t xtile_all[W][MT * 16 * kActRow];
    __shared__ f32x4 part[W][MT][kWave];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x >> 6;
    const int i = lane & 15, g = lane >> 4;
    uint8_t* ctile = ctile_all[wave];
    uint8_t* xtile = xtile_all[wave];
    const int64_t n0 = (int64_t)blockIdx.x * 16;

    // coalesced roles: code row 4j + (lane >> 4) at byte (lane & 15) * 16;
    // activation row 2j + (lane >> 5) at element (lane & 31) * 8
    const int cr0 = lane >> 4, co = (lane & 15) * 16;
    const uint8_t* qrow[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t r = n0 + 4 * j + cr0;
        qrow[j] = q + (r < n ? r : n - 1) * k + co;
    }
    const int xt0 = lane >> 5, xo = (lane & 31) * 8;
    constexpr int XJ = MT * 8;
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < XJ; ++j)  // rows of tokens >= m stay zero
        *reinterpret_cast<u32x4*>(xtile + (2 * j + xt0) * kActRow + xo * 2) = zero;

    const int64_t steps = k >> 8;  // 256-k super-steps
    const int64_t per = (steps + W - 1) / W;
    const int64_t s0 = (int64_t)wave * per;
    const int64_t s1 = (s0 + per < steps) ? s0 + per : steps;

    f32x4 acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t)
        acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    for (int64_t st = s0; st < s1; ++st) {
        const int64_t kb = st * 256;
        u32x4 cv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            cv[j] = load_stream16(qrow[j] + kb);
        u32x4 xv[XJ];
#pragma unroll
        for (int j = 0; j < XJ; ++j) {
            const int tok = 2 * j + xt0;
            xv[j] = tok < m ? load16(x + (int64_t)tok * k + kb + xo) : zero;
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int j = 0; j < 4; ++j)
            *reinterpret_cast<u32x4*>(ctile + (4 * j + cr0) * kCodeRow + co) = cv[j];
#pragma unroll
        for (int j = 0; j < XJ; ++j) {
            const int tok = 2 * j + xt0;
            if (tok < m)
                *reinterpret_cast<u32x4*>(xtile + tok * kActRow + xo * 2) = xv[j];
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            // codes kb + 64g + 16j .. +15 of channel i: MFMA pair (j, 0/1)
            const u32x4 c16 = *reinterpret_cast<const u32x4*>(ctile + i * kCodeRow + 64 * g + 16 * j);
            const u32x2 d0 = A::decode4(c16.x), d1 = A::decode4(c16.y);
            const u32x2 d2 = A::decode4(c16.z), d3 = A::decode4(c16.w);
            const u32x4 a0 = {d0.x, d0.y, d1.x, d1.y};
            const u32x4 a1 = {d2.x, d2.y, d3.x, d3.y};
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const uint8_t* xpp = xtile + (i + 16 * t) * kActRow + (64 * g + 16 * j) * 2;
                const u32x4 b0 = *reinterpret_cast<const u32x4*>(xpp);
                const u32x4 b1 = *reinterpret_cast<const u32x4*>(xpp + 16);
                acc[t] = A::mfma(a0, b0, acc[t]);
                acc[t] = A::mfma(a1, b1, acc[t]);
            }
        }
        __builtin_amdgcn_wave_barrier();
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
        for (int w = 1; w < W; ++w)
            sum += part[w][t][lane];
        const int tok = i + 16 * t;
        if (tok >= m)
            continue;
        const float v[4] = {sum.x, sum.y, sum.z, sum.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t ch = n0 + 4 * g + r;
            if (ch < n)
                y[(int64_t)tok * n + ch] = epilogue<A>(v[r], scale[ch], bias, ch);
        }
    }
}

// ---------------------------------------------------------------- dispatch
template <typename A, int SEG, int T, int W, int U, int MT>
hipError_t launch_seg(const void* x, int m, int64_t k, const uint8_t* q, const float* scale, const void* bias,
                      int64_t n, void* y, hipStream_t stream)
{
    constexpr int C = (16 / SEG) * T;  // channels per workgroup
    const dim3 grid((unsigned)((n + C - 1) / C)), block(W * kWave);
    hipLaunchKernelGGL((seg_kernel<A, SEG, T, W, U, MT>), grid, block, 0, stream,
                       static_cast<const uint16_t*>(x), q, scale, static_cast<const uint16_t*>(bias),
                       static_cast<uint16_t*>(y), m, n, k);
    return hipGetLastError();
}

template <typename A, int MT, int W>
hipError_t launch_lds(const void* x, int m, int64_t k, const uint8_t* q, const float* scale, const void* bias,
                      int64_t n, void* y, hipStream_t stream)
{
    const dim3 grid((unsigned)((n + 15) / 16)), block(W * kWave);
    hipLaunchKernelGGL((lds_kernel<A, MT, W>), grid, block, 0, stream, static_cast<const uint16_t*>(x), q, scale,
                       static_cast<const uint16_t*>(bias), static_cast<uint16_t*>(y), m, n, k);
    return hipGetLastError();
}

// Tile choice per batch size, from sweeps on MI355X (k % 256 == 0 here). A
// workgroup always covers the whole of k, so layers with few channels
// (n < 8192) keep 16 channels per workgroup to give every CU work.
template <typename A>
hipError_t launch_typed(const void* x, int64_t m, int64_t k, const uint8_t* q, const float* scale,
                        const void* bias, int64_t n, void* y, hipStream_t stream)
{
    const int mi = (int)m;
    if (m <= 4)
        return launch_seg<A, 4, 4, 4, 2, 1>(x, mi, k, q, scale, bias, n, y, stream);
    if (m <= 8) {
        if (n >= 8192)
            return launch_seg<A, 2, 4, 4, 1, 1>(x, mi, k, q, scale, bias, n, y, stream);
        return launch_seg<A, 2, 2, 8, 2, 1>(x, mi, k, q, scale, bias, n, y, stream);
    }
    if (m <= 16)
        return launch_lds<A, 1, 4>(x, mi, k, q, scale, bias, n, y, stream);
    if (n >= 8192)
        return launch_seg<A, 1, 2, 4, 1, 2>(x, mi, k, q, scale, bias, n, y, stream);
    return launch_lds<A, 2, 4>(x, mi, k, q, scale, bias, n, y, stream);
}

}  // namespace

hipError_t launch_skinny(const void* x, Act act, int64_t m, int64_t k, const uint8_t* q,
                         const float* scale, const void* bias, int64_t n, void* y, hipStream_t stream)
{
    if (n == 0 || m == 0)
        return hipSuccess;
    if (m > 32 || k % 256 != 0)
        return hipErrorInvalidValue;
    if (act == Act::BF16)
        return launch_typed<Bf16>(x, m, k, q, scale, bias, n, y, stream);
    if (act == Act::FP16)
        return launch_typed<F16>(x, m, k, q, scale, bias, n, y, stream);
    return hipErrorInvalidValue;
}

}  // namespace fp8w
