// Skinny GEMM (M = 2..32) for layers too narrow to give every CU more than one
// 16-channel tile: the matrix-core kernel whose LDS carries weight codes only.
//
// "FP8 weight-only (precision: fp8_weights)", section "Dequantise in
// registers": from M = 2 the small-batch kernel runs the dot products on the
// matrix unit in the activations' type, the weight as the channel operand and
// the tokens as the narrow one; each code is converted once (exactly) and
// reused for every token; k is split across waves and their partial sums are
// reduced through LDS. The epilogue is the contract's: fp32 accumulation,
// scale and bias in fp32, one rounding.
//
// Why a second kernel. On a layer of 4096 channels there are only 256 tiles of
// 16 channels, one per CU, so each workgroup must read the whole activation
// block: at 16 tokens, 2 bytes of activations per code byte. Staged through the
// same LDS ring as the codes (pipe_kernel), the activations took two thirds of
// every stage and left a few KB of the weight stream in flight per CU; the
// kernel then waited on HBM latency most of the time. Here each wave loads its
// activation fragments straight into VGPRs, already in the MFMA operand layout,
// and the LDS holds codes only, in a ring per wave: with k = 4096, all 64 KB of
// a CU's codes can be in flight at once.
//
// Layout (gfx950, v_mfma_f32_16x16x32_{bf16,f16}: lane l = i + 16 g holds
// A[i][8g + e], B[8g + e][i], returns D[4g + r][i]). A workgroup owns 16
// channels over the whole of k and has W waves; stage s of wave w is the 256 k
// starting at (s W + w) 256. Per stage a wave
//   * loads its 16 code rows x 256 bytes with four direct global-to-LDS loads
//     (1 KB each: a quarter-wave reads 256 contiguous bytes of one row; the
//     lane-to-address map rotates each row's 16-byte chunks by the row index so
//     the reads below hit distinct banks), into its own region of stage buffer
//     s mod NS;
//   * loads, per 16-token tile, eight 16-byte activation fragments into
//     registers: for MFMA pair j (0..3) and half h, lane (i, g) takes token i's
//     elements 16 (4j + g) + 8h .. + 7, so the lanes of a token cover one
//     128-byte line with the two halves. Those lanes are 16 apart, so a
//     quarter-wave (four neighbouring lanes, four tokens) touches four lines
//     per instruction. With QL the same fragments are loaded by lane 4i + g
//     instead (a quarter-wave reads one token's line) and moved to lane i + 16g
//     with ds_bpermute just before their MFMA: four LDS-crossbar moves per
//     fragment, paid back from 10 tokens on;
//   * reads chunk 4j + g of code row i from LDS for pair j, decodes it to two
//     8-element operands and issues two MFMAs per token tile. MFMA (j, h)
//     pairs k slot 8g + e with k = 64j + 16g + 8h + e in both operands.
// The waves never read each other's LDS, so the ring needs no barriers: a wave
// waits only for its own loads (vmcnt, which counts the direct-to-LDS loads
// too, in issue order). At the end the W partial sums meet in LDS and wave 0
// adds them in wave order and applies the epilogue.
#include <stdio.h>

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "ring.hpp"

namespace fp8w {
namespace {

// f(std::integral_constant<int, I>) for I = B .. E-1, unrolled at compile time
// (the ring's buffer and wait-count indices must be constants).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f)
{
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

template <int MT_, int W, int NS>
struct NarrowCfg {
    static_assert(MT_ == 1 || MT_ == 2, "16-token tiles");
    static_assert(W >= 1 && W <= 16, "waves");
    static_assert(NS >= 2 && NS <= 8, "stages");
    static constexpr int MT = MT_;              // 16-token MFMA tiles
    static constexpr int CODE = 16 * 256;        // code bytes per wave and stage
    static constexpr int BUF = W * CODE;         // one stage buffer (all waves)
    static constexpr int XL = 8 * MT;            // activation loads per wave and stage
    static constexpr int LOADS = 4 + XL;         // load instructions per wave and stage
    static_assert(LOADS * (NS - 2) < 64, "vmcnt range");
};

// QL: each token's activation fragments are loaded by four neighbouring lanes
// (lane 4 t + g takes token t's part g), so each quarter of a load instruction
// reads one 128-byte line instead of four; before each MFMA the parts move to
// the operand layout's lanes (t + 16 g) with ds_bpermute. Lanes of tokens past
// m load nothing (their columns of D are never stored).
template <typename A, int MT_, int W, int NS, bool QL>
struct Narrow {
    using C = NarrowCfg<MT_, W, NS>;
    static constexpr int MT = C::MT;
    // The waits count every load instruction of a stage, so no instruction may
    // be skipped by a whole wave: with one token tile, token 0's lanes always
    // load (m >= 1). A second tile's QL loads could all be masked off.
    static_assert(!QL || MT == 1, "QL loads with one token tile");

    const uint8_t* q;     // row n0 of the codes
    const uint16_t* xrow[MT];  // this lane's token rows (QL: the loading lane's)
    bool xon[MT];         // QL: this lane loads for a token below m
    int64_t n, k, n0;
    int64_t S, rot;       // stages per wave; this workgroup's first stage
    int lane, wave;

    // Issue stage s (any s < S) into buffer `buf` and registers xv.
    __device__ __forceinline__ void issue(int64_t s, uint8_t* buf, u32x4 (&xv)[4][2][MT]) const
    {
        int64_t sr = s + rot;  // s < S and rot < S
        sr = sr < S ? sr : sr - S;
        const int64_t kb = (sr * W + wave) * 256;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 4 * j + (lane >> 4);
            const int chunk = ((lane & 15) - r) & 15;
            int64_t row = n0 + r;
            row = row < n ? row : n - 1;
            const uint8_t* src = q + row * k + kb + chunk * 16;
            __builtin_amdgcn_global_load_lds((const void*)src, FP8W_LDS(buf + wave * C::CODE + j * 1024), 16, 0,
                                             2 /* non-temporal */);
        }
        const int g = QL ? (lane & 3) : (lane >> 4);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    if (!QL || xon[mt])
                        xv[j][h][mt] = load16(xrow[mt] + kb + 64 * j + 16 * g + 8 * h);
                }
    }

    // QL: lane t + 16 g takes the part its token's loading lane 4 t + g holds
    __device__ __forceinline__ static u32x4 to_operand(const u32x4 v, int src)
    {
        if constexpr (!QL)
            return v;
        u32x4 r;
        r.x = __builtin_amdgcn_ds_bpermute(src, (int)v.x);
        r.y = __builtin_amdgcn_ds_bpermute(src, (int)v.y);
        r.z = __builtin_amdgcn_ds_bpermute(src, (int)v.z);
        r.w = __builtin_amdgcn_ds_bpermute(src, (int)v.w);
        return r;
    }

    __device__ __forceinline__ void compute(const uint8_t* buf, const u32x4 (&xv)[4][2][MT], f32x4* acc) const
    {
        const int i = lane & 15, g = lane >> 4;
        const int src = (4 * i + g) << 2;  // QL: byte address of lane 4 i + g
        const uint8_t* cb = buf + wave * C::CODE + 256 * i;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const u32x4 c16 = *reinterpret_cast<const u32x4*>(cb + 16 * ((4 * j + g + i) & 15));
            const u32x2 d0 = A::decode4(c16.x), d1 = A::decode4(c16.y);
            const u32x2 d2 = A::decode4(c16.z), d3 = A::decode4(c16.w);
            const u32x4 a0 = {d0.x, d0.y, d1.x, d1.y};
            const u32x4 a1 = {d2.x, d2.y, d3.x, d3.y};
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                acc[mt] = A::mfma(a0, to_operand(xv[j][0][mt], src), acc[mt]);
                acc[mt] = A::mfma(a1, to_operand(xv[j][1][mt], src), acc[mt]);
            }
        }
    }
};

// Requires k % (W * 256 * NS) == 0 and m <= 16 * MT. One workgroup per 16 channels.
// The output pointer comes last, so that the sizes lie in the 56 bytes of
// arguments the wave finds preloaded in SGPRs.
template <typename A, int MT_, int W, int NS, bool QL>
__global__ __launch_bounds__(W* kWave) void narrow_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ q, const float* __restrict__ scale,
    const uint16_t* __restrict__ bias, int m, int64_t n, int64_t k, uint16_t* __restrict__ y)
{
    using P = Narrow<A, MT_, W, NS, QL>;
    using C = typename P::C;
    constexpr int MT = C::MT;
    constexpr int LOADS = C::LOADS;
    // one distinct array per stage buffer, so that the compiler can tell the
    // buffers apart and adds no waits of its own for the direct-to-LDS loads
    __shared__ __attribute__((aligned(1024))) uint8_t b0[C::BUF];
    __shared__ __attribute__((aligned(1024))) uint8_t b1[C::BUF];
    __shared__ __attribute__((aligned(1024))) uint8_t b2[NS > 2 ? C::BUF : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t b3[NS > 3 ? C::BUF : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t b4[NS > 4 ? C::BUF : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t b5[NS > 5 ? C::BUF : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t b6[NS > 6 ? C::BUF : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t b7[NS > 7 ? C::BUF : 16];
    __shared__ f32x4 red[W][MT][kWave];
    uint8_t* const bufs[8] = {b0, b1, b2, b3, b4, b5, b6, b7};

    P p;
    p.q = q;
    p.n = n;
    p.k = k;
    p.lane = threadIdx.x & (kWave - 1);
    p.wave = threadIdx.x / kWave;
    p.n0 = (int64_t)blockIdx.x * 16;
    const int i = p.lane & 15, g = p.lane >> 4;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int t = (QL ? (p.lane >> 2) : i) + 16 * mt;
        p.xon[mt] = t < m;
        p.xrow[mt] = x + (int64_t)(t < m ? t : m - 1) * k;  // rows past m: a real row, results discarded
    }
    const int64_t S = k / (W * 256);
    p.S = S;
    // workgroups are dealt to the eight XCDs in turn: consecutive workgroups of
    // one XCD start at consecutive stages
    p.rot = (int64_t)(blockIdx.x / 8) % S;

    // epilogue operands of this lane's four channels, fetched before the ring
    float sc[4];
    uint16_t bi[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        int64_t ch = p.n0 + 4 * g + r;
        ch = ch < n ? ch : n - 1;
        sc[r] = scale[ch];
        bi[r] = bias_bits(bias, ch);
    }

    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
        acc[mt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    u32x4 xv[NS][4][2][MT];

    // NS - 1 stages in flight before the first is used
    static_for<0, NS - 1>([&](auto uc) {
        constexpr int u = decltype(uc)::value;
        p.issue(u, bufs[u], xv[u]);
    });
    int64_t s0 = 0;
    for (; s0 + NS < S; s0 += NS) {
        static_for<0, NS>([&](auto uc) {
            constexpr int u = decltype(uc)::value;
            constexpr int nx = (u + NS - 1) % NS;
            wait_loads_at_most<LOADS*(NS - 2)>();  // stage s0 + u has landed
            __builtin_amdgcn_sched_barrier(0);
            p.issue(s0 + u + NS - 1, bufs[nx], xv[nx]);
            __builtin_amdgcn_sched_barrier(0);
            p.compute(bufs[u], xv[u], acc);
        });
    }
    // the last NS stages: issue the final one, then drain
    static_for<0, NS>([&](auto uc) {
        constexpr int u = decltype(uc)::value;
        if constexpr (u == 0) {
            wait_loads_at_most<LOADS*(NS - 2)>();
            __builtin_amdgcn_sched_barrier(0);
            p.issue(S - 1, bufs[NS - 1], xv[NS - 1]);
            __builtin_amdgcn_sched_barrier(0);
        } else {
            wait_loads_at_most<LOADS*(NS - 1 - u)>();
        }
        p.compute(bufs[u], xv[u], acc);
    });

    // partial sums of the W waves, added in wave order by wave 0
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
        red[p.wave][mt][p.lane] = acc[mt];
    __syncthreads();
    if (p.wave != 0)
        return;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        f32x4 sum = red[0][mt][p.lane];
#pragma unroll
        for (int w = 1; w < W; ++w)
            sum += red[w][mt][p.lane];
        const int tok = i + 16 * mt;
        if (tok >= m)
            continue;
        const float v[4] = {sum.x, sum.y, sum.z, sum.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t ch = p.n0 + 4 * g + r;
            if (ch < n)
                y[(int64_t)tok * n + ch] = epilogue<A>(v[r], sc[r], bi[r]);
        }
    }
}

template <typename A, int MT, int W, int NS, bool QL>
hipError_t launch_narrow_cfg(const void* x, int m, int64_t k, const uint8_t* q, const float* scale,
                             const void* bias, int64_t n, void* y, hipStream_t stream)
{
    const dim3 grid((unsigned)((n + 15) / 16)), block(W * kWave);
    hipLaunchKernelGGL((narrow_kernel<A, MT, W, NS, QL>), grid, block, 0, stream, static_cast<const uint16_t*>(x), q,
                       scale, static_cast<const uint16_t*>(bias), m, n, k, static_cast<uint16_t*>(y));
    return hipGetLastError();
}

}  // namespace

// Where it runs, from A/B sweeps against pipe_kernel / seg_kernel / the k split
// on MI355X (weights rotated through 1 GiB): layers under 8192 channels with
//   * k a multiple of 4096, 2..9 tokens: four waves, four-stage rings (the
//     whole k = 4096 in flight); 0.1-1.1 us faster on 1024- to 4096-channel
//     layers, e.g. [4096, 4096] at 4 tokens 6.7 -> 5.7 us, at 9: 7.2 -> 6.3;
//   * k a multiple of 4096, 10..16 tokens: eight waves, two-stage rings, QL
//     loads; [4096, 4096] at 16 tokens 7.2 -> 6.5 us, [4096, 8192] 11.5 ->
//     10.1, [2048, 4096] 6.9 -> 5.9 (the activation loads of four tokens'
//     lanes each touched four 128-byte lines per quarter-wave);
//   * k a multiple of 7168 (the 14336-wide down projection), 2..5 tokens:
//     seven waves, four-stage rings; [4096, 14336] at 4 tokens 12.3 us;
//   * k a multiple of 7168, 6..16 tokens: seven waves, two-stage rings, QL
//     loads; [4096, 14336] at 8 / 12 / 16 tokens 13.8 / 16.2 / 17.5 (the
//     last on pipe_kernel) -> 13.0 / 14.6 / 16.2 us;
//   * 17..24 tokens, k <= 8192 a multiple of 2048: two token tiles, four
//     waves, two stages; [4096, 4096] at 17 tokens 9.7 (k split) -> 8.4 us,
//     [2048, 8192] at 22 tokens 16.7 -> 14.7 (at 32 tokens and on long k the
//     k split stays faster; QL loads measured 0.6-1 us slower here).
NarrowPlan plan_narrow(int64_t m, int64_t n, int64_t k, bool split_ok)
{
    NarrowPlan p{};
    if (m < 2 || m > 24 || n < 1 || n >= 8192 || k < 256 || k % 256 != 0)
        return p;
    // with workspace, 12..16 tokens on layers of 4096+ channels with k % 7168 == 0,
    // k % 2048 == 0 and k % 4096 != 0 (the 14336-wide down projection) take
    // the skinny kernel's four-way k split (13.9 / 14.3 us at 12 / 16 tokens
    // on [4096, 14336], against 14.6 / 16.2 here)
    if (split_ok && m >= 12 && m <= 16 && n >= 4096 && k % 7168 == 0 && k % 2048 == 0 && k % 4096 != 0)
        return p;
    if (m <= 16 && k % 4096 == 0) {
        p = m >= 10 ? NarrowPlan{true, 1, 8, 2, true} : NarrowPlan{true, 1, 4, 4, false};
    } else if (m <= 16 && k % 7168 == 0) {
        p = m >= 6 ? NarrowPlan{true, 1, 7, 2, true} : NarrowPlan{true, 1, 7, 4, false};
    } else if (m >= 17 && k % 2048 == 0 && k <= 8192) {
        p = NarrowPlan{true, 2, 4, 2, false};
    }
    return p;
}

template <typename A>
static hipError_t launch_narrow_typed(const NarrowPlan& p, const void* x, int m, int64_t k, const uint8_t* q,
                                      const float* scale, const void* bias, int64_t n, void* y, hipStream_t stream)
{
    const int key = (p.ql ? 1000 : 0) + p.mt * 100 + p.w * 10 + p.ns;
    switch (key) {
    case 144: return launch_narrow_cfg<A, 1, 4, 4, false>(x, m, k, q, scale, bias, n, y, stream);
    case 174: return launch_narrow_cfg<A, 1, 7, 4, false>(x, m, k, q, scale, bias, n, y, stream);
    case 242: return launch_narrow_cfg<A, 2, 4, 2, false>(x, m, k, q, scale, bias, n, y, stream);
    case 1182: return launch_narrow_cfg<A, 1, 8, 2, true>(x, m, k, q, scale, bias, n, y, stream);
    case 1172: return launch_narrow_cfg<A, 1, 7, 2, true>(x, m, k, q, scale, bias, n, y, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_narrow(const NarrowPlan& p, const void* x, Act act, int64_t m, int64_t k, const uint8_t* q,
                         const float* scale, const void* bias, int64_t n, void* y, hipStream_t stream)
{
    if (!p.ok || m < 1 || m > 16 * p.mt || n < 1 || k < 256 || k % ((int64_t)p.w * 256 * p.ns) != 0)
        return hipErrorInvalidValue;
    if ((n + 15) / 16 > INT32_MAX)
        return hipErrorInvalidValue;
    if (act == Act::BF16)
        return launch_narrow_typed<Bf16>(p, x, (int)m, k, q, scale, bias, n, y, stream);
    if (act == Act::FP16)
        return launch_narrow_typed<F16>(p, x, (int)m, k, q, scale, bias, n, y, stream);
    return hipErrorInvalidValue;
}

const char* narrow_kernel_name(const NarrowPlan& p)
{
    thread_local char name[64];
    snprintf(name, sizeof name, "narrow_kernel<MT=%d,W=%d,NS=%d%s>", p.mt, p.w, p.ns, p.ql ? ",QL" : "");
    return name;
}

}  // namespace fp8w
