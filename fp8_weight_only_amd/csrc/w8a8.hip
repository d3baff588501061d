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
// store per fragment row.
//
// A workgroup of WN x WM waves owns BN channels x BM tokens (256 x 256 down to
// 128 x 64, by the shape); each wave owns BN / WN channels x BM / WM tokens.
// Stages of 64 k of both tiles travel HBM/L2 -> LDS by direct global-to-LDS
// loads through a ring of NS stage buffers (the waits and barrier of
// csrc/ring.hpp). In LDS every 64-byte row keeps its four 16-byte chunks
// rotated by row / 4, so the 16 lanes of each ds_read_b128 phase (rows
// i .. i+15, same chunk) hit 16 distinct bank groups.
//
// Latency hiding: with eight waves (two per SIMD) one wave's MFMAs run while
// the other waits for LDS or the barrier. With four waves (one per SIMD, the
// 128 x 64 tile) the ring prefetches fragments instead: the fragments of
// stage s + 1 are read into a second register set while the MFMAs of stage s
// run, one read issued after each MFMA (scheduling-group barriers hold that
// order). The epilogue's operands (the workgroup's channel scales and biases
// and its token scales) are fetched once when the workgroup starts and pass
// through LDS, so the end of a tile waits for no global load. Tiles are dealt
// so that the workgroups resident on one XCD at a time cover a compact block
// of the output (rows of four tiles along the tokens), and share more of
// their operand rows in that XCD's L2; each XCD's workgroups start at their
// own eighth of k.
#include <stdio.h>

#include <type_traits>
#include <utility>

#include "common.hpp"
#include "kernels.hpp"
#include "ring.hpp"

namespace fp8w {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int BN, int BM, int NS, int WN, int WM>
struct W8Cfg {
    static constexpr int W = WN * WM;            // waves
    static constexpr int FN = BN / WN / 32;      // 32-channel fragments per wave
    static constexpr int FM = BM / WM / 32;      // 32-token fragments per wave
    static constexpr int ABYTES = BN * 64;
    static constexpr int STAGE = (BN + BM) * 64;
    static constexpr int BLOCKS = (BN + BM) / 16;  // 1 KB load instructions per stage
    static constexpr int LOADS = BLOCKS / W;       // per wave
    static_assert(FN >= 1 && FM >= 1, "at least one fragment each way per wave");
    static_assert(BLOCKS % W == 0, "blocks split evenly over the waves");
    static_assert(LOADS * (NS - 2) < 64, "vmcnt range");
};

template <int BN, int BM, int NS, int WN, int WM>
struct W8Pipe {
    using C = W8Cfg<BN, BM, NS, WN, WM>;
    const uint8_t* qw;  // [n, k]
    const uint8_t* qx;  // [m, k]
    int64_t n, m, k, n0, m0;
    int64_t S, rot;  // stages; the k stage this workgroup starts at
    int lane, wave, wn, wm;

    // Stage s covers k stage (s + rot) mod S. Block b of the stage holds rows
    // 16b .. 16b + 15 of the weight tile (b < BN / 16) or of the token tile;
    // lane l brings 16 bytes of row 16b + l / 4, the chunk that belongs at
    // slot l % 4 (chunk (slot - row / 4) mod 4).
    __device__ __forceinline__ void issue(int64_t s, uint8_t* buf) const
    {
        int64_t sr = s + rot;  // s < S and rot < S
        sr = sr < S ? sr : sr - S;
        const int64_t kb = sr * 64;
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

    // fragments of this wave's channel (a) and token (b) tiles from a stage buffer
    __device__ __forceinline__ void read(const uint8_t* buf, i32x8* a, i32x8* b) const
    {
        const int i = lane & 31;
#pragma unroll
        for (int f = 0; f < C::FN; ++f)
            a[f] = frag(buf, wn * (BN / WN) + 32 * f + i);
#pragma unroll
        for (int f = 0; f < C::FM; ++f)
            b[f] = frag(buf + C::ABYTES, wm * (BM / WM) + 32 * f + i);
    }

    __device__ __forceinline__ void mma(const i32x8* a, const i32x8* b, f32x16* acc) const
    {
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
            for (int fm = 0; fm < C::FM; ++fm)
                acc[fn * C::FM + fm] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    a[fn], b[fm], acc[fn * C::FM + fm], 0, 0, 0, 0, 0, 0);
    }

    // one stage with no prefetch (run_ring's step; eight-wave tiles)
    __device__ __forceinline__ void compute(const uint8_t* buf, f32x16* acc) const
    {
        i32x8 a[C::FN], b[C::FM];
        read(buf, a, b);
        mma(a, b, acc);
    }

    // MFMAs on (a, b) while the next stage's fragments are read from nbuf into
    // (na, nb): one MFMA, then one ds_read_b128, in turn (four-wave tiles)
    __device__ __forceinline__ void step(const uint8_t* nbuf, const i32x8* a, const i32x8* b, i32x8* na, i32x8* nb,
                                         f32x16* acc) const
    {
        read(nbuf, na, nb);
        mma(a, b, acc);
        constexpr int NR = 2 * (C::FN + C::FM);  // ds_read_b128 per stage
        constexpr int NM = C::FN * C::FM;
        constexpr int PER = NR / NM > 0 ? NR / NM : 1;
#pragma unroll
        for (int j = 0; j < NM; ++j) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            if (j * PER < NR)
                __builtin_amdgcn_sched_group_barrier(0x100, PER, 0);  // then LDS reads
        }
    }
};

// Calls f(integral_constant<int, I>) for I = 0 .. N-1, unrolled at compile time.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, I...>)
{
    (f(std::integral_constant<int, I>{}), ...);
}

template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f)
{
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// y[t, c] = out(fl32(fl32(acc * scale_x[t]) * scale_w[c]) + bias[c]).
// Requires k % (64 * NS) == 0 (k / 64 stages, a multiple of the NS-stage
// ring); qw, qx 16-byte aligned.
template <typename A, int BN, int BM, int NS, int WN, int WM, int GM = 4>
__global__ __launch_bounds__(WN* WM * kWave) void w8a8_kernel(const uint8_t* __restrict__ qx,
                                                             const float* __restrict__ sx,
                                                             const uint8_t* __restrict__ qw,
                                                             const float* __restrict__ sw,
                                                             const uint16_t* __restrict__ bias,
                                                             uint16_t* __restrict__ y, int64_t m, int64_t n,
                                                             int64_t k)
{
    static_assert(NS == 4 || NS == 6 || NS == 8, "an even number of stages, 4 to 8");
    using P = W8Pipe<BN, BM, NS, WN, WM>;
    using C = typename P::C;
    constexpr int L = C::LOADS;
    constexpr int NT = C::W * kWave;
    static_assert(C::W == 4 || (C::W == 8 && NS == 4), "eight-wave tiles run the four-stage ring");
    static_assert(BN <= NT && BM <= NT, "one epilogue operand per thread");
    // one array per stage buffer: the compiler can then tell the buffer being
    // read from the ones the direct-to-LDS loads are writing, and inserts no
    // waits of its own
    __shared__ __attribute__((aligned(1024))) uint8_t b0[C::STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t b1[C::STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t b2[C::STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t b3[C::STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t b4[NS > 4 ? C::STAGE : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t b5[NS > 5 ? C::STAGE : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t b6[NS > 6 ? C::STAGE : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t b7[NS > 7 ? C::STAGE : 16];
    __shared__ __attribute__((aligned(16))) float e_sw[BN];
    __shared__ __attribute__((aligned(16))) uint16_t e_bias[BN];
    __shared__ __attribute__((aligned(16))) float e_sx[BM];
    auto buf = [&](auto I) -> uint8_t* {
        constexpr int i = decltype(I)::value % NS;
        if constexpr (i == 0)
            return b0;
        else if constexpr (i == 1)
            return b1;
        else if constexpr (i == 2)
            return b2;
        else if constexpr (i == 3)
            return b3;
        else if constexpr (i == 4)
            return b4;
        else if constexpr (i == 5)
            return b5;
        else if constexpr (i == 6)
            return b6;
        else
            return b7;
    };

    int64_t tn, tm;
    xcd_tile_of<GM>(tn, tm);
    P p;
    p.qw = qw;
    p.qx = qx;
    p.n = n;
    p.m = m;
    p.k = k;
    p.n0 = tn * BN;
    p.m0 = tm * BM;
    p.lane = threadIdx.x & (kWave - 1);
    p.wave = threadIdx.x / kWave;
    p.wn = p.wave % WN;
    p.wm = p.wave / WN;

    // epilogue operands, one per thread, fetched before the ring starts and
    // stored to LDS once the ring's first wait (which covers them: loads
    // complete in order) has passed
    const int tt = threadIdx.x;
    float r_sw = 0.0f, r_sx = 0.0f;
    uint16_t r_bias = 0;
    if (tt < BN) {
        const int64_t c = p.n0 + tt < n ? p.n0 + tt : n - 1;
        r_sw = sw[c];
        r_bias = bias_bits(bias, c);
    }
    if (tt < BM)
        r_sx = sx[p.m0 + tt < m ? p.m0 + tt : m - 1];
    auto store_epilogue_operands = [&]() {
        if (tt < BN) {
            e_sw[tt] = r_sw;
            e_bias[tt] = r_bias;
        }
        if (tt < BM)
            e_sx[tt] = r_sx;
    };

    f32x16 acc[C::FN * C::FM];
#pragma unroll
    for (int f = 0; f < C::FN * C::FM; ++f)
        acc[f] = f32x16{0.0f};
    const int64_t S = k / 64;
    // k stagger per XCD: the workgroups one XCD holds (linear id L, XCD L % 8)
    // walk k in step and share operand rows in its L2; the eight XCDs start
    // an eighth of k apart, so their weight reads spread over more of HBM.
    // Measured on MI355X: 5-11 % faster on the 4096-channel prefill layers at
    // M = 512 and 2048, within run-to-run noise elsewhere; a stagger per
    // workgroup was slower.
    p.S = S;
    p.rot = ((blockIdx.x + (int64_t)gridDim.x * blockIdx.y) % 8) * (S / 8);

    if constexpr (C::W == 8) {
        // two waves per SIMD: the plain ring (csrc/ring.hpp)
        store_epilogue_operands();
        run_ring<NS, L>(p, S, b0, b1, b2, b3, acc);
    } else {
        // The prefetching ring: stage s + NS - 1 is issued at step s into the
        // buffer of stage s - 1, whose fragments were read during step s - 2;
        // step s waits for stage s + 1 (NS - 3 later stages may still be in
        // flight), runs stage s's MFMAs and reads stage s + 1's fragments into
        // the other register set (even steps compute set 0, odd steps set 1).
        i32x8 a0[C::FN], x0[C::FM], a1[C::FN], x1[C::FM];
        static_for<NS - 1>([&](auto I) { p.issue(decltype(I)::value, buf(I)); });
        wait_loads_at_most<(NS - 2) * L>();
        stage_barrier();
        store_epilogue_operands();
        p.read(b0, a0, x0);
        auto step = [&](auto U) {
            constexpr int u = decltype(U)::value;
            if constexpr (u % 2 == 0)
                p.step(buf(std::integral_constant<int, u + 1>{}), a0, x0, a1, x1, acc);
            else
                p.step(buf(std::integral_constant<int, u + 1>{}), a1, x1, a0, x0, acc);
        };
        int64_t s = 0;
        for (; s < S - NS; s += NS) {
            static_for<NS>([&](auto U) {
                constexpr int u = decltype(U)::value;
                wait_loads_at_most<(NS - 3) * L>();
                stage_barrier();
                p.issue(s + u + NS - 1, buf(std::integral_constant<int, u + NS - 1>{}));
                step(U);
            });
        }
        // the last NS stages: S - 1 is issued at the first step, then the ring drains
        wait_loads_at_most<(NS - 3) * L>();
        stage_barrier();
        p.issue(s + NS - 1, buf(std::integral_constant<int, NS - 1>{}));
        step(std::integral_constant<int, 0>{});
        static_for<NS - 2>([&](auto J) {
            constexpr int j = decltype(J)::value + 1;
            wait_loads_at_most<(NS - 2 - j) * L>();
            stage_barrier();
            step(std::integral_constant<int, j>{});
        });
        p.mma(a1, x1, acc);  // NS is even: the last step computes set 1
    }
    __syncthreads();

    // lane (i, h) holds channels c0 + 8j + 4h + r (r = 0..3) of token t
    const int i = p.lane & 31, h = p.lane >> 5;
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm) {
        const int tl = p.wm * (BM / WM) + 32 * fm + i;
        const int64_t t = p.m0 + tl;
        if (t >= m)
            continue;
        const float st = e_sx[tl];
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn) {
            const f32x16 d = acc[fn * C::FM + fm];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int cl = p.wn * (BN / WN) + 32 * fn + 8 * j + 4 * h;
                const int64_t c0 = p.n0 + cl;
                const f32x4 s4 = *reinterpret_cast<const f32x4*>(&e_sw[cl]);
                const u32x2 b4 = *reinterpret_cast<const u32x2*>(&e_bias[cl]);
                const float bf[4] = {A::lo_f32(b4.x), A::hi_f32(b4.x), A::lo_f32(b4.y), A::hi_f32(b4.y)};
                uint16_t o[4];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    o[r] = A::from_f32((d[4 * j + r] * st) * s4[r] + bf[r]);
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

template <typename A, int BN, int BM, int NS, int WN, int WM>
hipError_t launch_w8(const uint8_t* qx, const float* sx, int64_t m, int64_t k, const uint8_t* qw, const float* sw,
                     const void* bias, int64_t n, void* y, hipStream_t stream)
{
    const dim3 grid((unsigned)((n + BN - 1) / BN), (unsigned)((m + BM - 1) / BM)), block(WN * WM * kWave);
    hipLaunchKernelGGL((w8a8_kernel<A, BN, BM, NS, WN, WM>), grid, block, 0, stream, qx, sx, qw, sw,
                       static_cast<const uint16_t*>(bias), static_cast<uint16_t*>(y), m, n, k);
    return hipGetLastError();
}

// Tile choice, from a sweep of four tile shapes on the prefill shapes
// (M = 512 / 2048 / 4096 on [4096, 4096], [14336, 4096], [4096, 14336]): the
// largest tile that still gives at least 224 workgroups (7/8 of the CUs, one
// workgroup per CU), in the order 256 x 256, 256 x 128, 128 x 128, 128 x 64
// (channels x tokens); the smallest below that. It picked the fastest or
// within 1 % of the fastest shape in all nine cases.
//
// Waves: eight (2 x 4, two per SIMD) on the three larger tiles, which measured
// 15-25 % faster than four at 256 x 256, 3-8 % at 256 x 128 and 128 x 128;
// four (2 x 2) at 128 x 64, whose 12 load instructions per stage do not split
// over eight waves.
//
// Ring depth (four-wave tile): with two MFMAs per wave per stage, four stages
// cover too little of the weights' trip from HBM. Where the tile gives at most
// 256 workgroups (one per CU either way) eight stages are used (k % 512 == 0):
// measured 12-14 % faster at M = 512 on the 4096-channel layers. With more
// workgroups, the four-stage ring's smaller LDS footprint lets two or three
// share a CU, which measured faster.
struct W8Tile {
    int bn, bm, ns, waves;
};

W8Tile w8a8_tile(int64_t m, int64_t n, int64_t k)
{
    auto tiles = [&](int64_t bn, int64_t bm) { return ((n + bn - 1) / bn) * ((m + bm - 1) / bm); };
    if (tiles(256, 256) >= 224)
        return {256, 256, 4, 8};
    if (tiles(256, 128) >= 224)
        return {256, 128, 4, 8};
    if (tiles(128, 128) >= 224)
        return {128, 128, 4, 8};
    return {128, 64, tiles(128, 64) <= 256 && k % 512 == 0 ? 8 : 4, 4};
}

template <typename A>
hipError_t launch_w8_typed(const uint8_t* qx, const float* sx, int64_t m, int64_t k, const uint8_t* qw,
                           const float* sw, const void* bias, int64_t n, void* y, hipStream_t stream)
{
    const W8Tile t = w8a8_tile(m, n, k);
    if (t.bn == 256 && t.bm == 256)
        return launch_w8<A, 256, 256, 4, 2, 4>(qx, sx, m, k, qw, sw, bias, n, y, stream);
    if (t.bn == 256)
        return launch_w8<A, 256, 128, 4, 2, 4>(qx, sx, m, k, qw, sw, bias, n, y, stream);
    if (t.bm == 128)
        return launch_w8<A, 128, 128, 4, 2, 4>(qx, sx, m, k, qw, sw, bias, n, y, stream);
    return t.ns == 8 ? launch_w8<A, 128, 64, 8, 2, 2>(qx, sx, m, k, qw, sw, bias, n, y, stream)
                     : launch_w8<A, 128, 64, 4, 2, 2>(qx, sx, m, k, qw, sw, bias, n, y, stream);
}

}  // namespace

hipError_t launch_w8a8(const uint8_t* qx, const float* sx, int64_t m, int64_t k, const uint8_t* qw, const float* sw,
                       const void* bias, int64_t n, void* y, Act out, hipStream_t stream)
{
    if (m == 0 || n == 0)
        return hipSuccess;
    if (out == Act::BF16)
        return launch_w8_typed<Bf16>(qx, sx, m, k, qw, sw, bias, n, y, stream);
    if (out == Act::FP16)
        return launch_w8_typed<F16>(qx, sx, m, k, qw, sw, bias, n, y, stream);
    return hipErrorInvalidValue;
}

const char* w8a8_kernel_name(int64_t m, int64_t n, int64_t k)
{
    const W8Tile t = w8a8_tile(m, n, k);
    if (t.bn == 256 && t.bm == 256)
        return "w8a8_kernel<BN=256,BM=256,NS=4,W=8>";
    if (t.bn == 256)
        return "w8a8_kernel<BN=256,BM=128,NS=4,W=8>";
    if (t.bm == 128)
        return "w8a8_kernel<BN=128,BM=128,NS=4,W=8>";
    return t.ns == 8 ? "w8a8_kernel<BN=128,BM=64,NS=8,W=4>" : "w8a8_kernel<BN=128,BM=64,NS=4,W=4>";
}

}  // namespace fp8w
