// The weight-only linear for batches above the skinny kernels' 32 tokens
// (batched decode): y[m, n] = scale[n] * sum_k x[m, k] * value(q[n, k]) + bias[n],
// the same contract as the other paths ("FP8 weight-only (precision:
// fp8_weights)", section "The contract": e4m3 weights, activations kept in
// bf16 / fp16, fp32 accumulation, the scale and bias in an fp32 epilogue, one
// rounding to the activation dtype). Unlike the fallback it never writes a
// dequantised weight: the codes are decoded in the GEMM itself, exactly, into
// the activation dtype ("Dequantise in registers": every e4m3 value is a bf16
// and an fp16 value), so the layer reads one byte per weight per tile row.
//
// A workgroup of WN x WM waves owns BN channels x BM tokens. Stages of 64 k of
// both tiles (BN rows of 64 codes, BM rows of 64 activations) go HBM/L2 -> LDS
// by direct global-to-LDS loads through the four-stage ring of csrc/ring.hpp.
// The matrix cores run v_mfma_f32_32x32x16_{bf16,f16}: channels are the A
// operand, tokens the B operand, so a lane's four consecutive accumulators are
// four consecutive channels of one token (one 8-byte store).
//
// Which k a lane feeds: in MFMA step j (0..3) of a stage, lane half h feeds k
// = 32h + 8j .. 32h + 8j + 7 of the stage to both operands. Each MFMA then
// sums 16 of the stage's products, every product exactly once over the four
// steps; only the summation order differs from a plain k loop, which the
// contract leaves open. A lane thus reads its 32 codes of a weight row as two
// 16-byte LDS reads and decodes them per step.
//
// Split k: with too few tiles to fill the chip (few tokens, or few channels),
// k is split over grid.z; each workgroup writes the fp32 sums of its k range to
// the caller's workspace and the skinny path's reduce kernel adds them in split
// order and applies the epilogue (deterministic). The plan (tile and split
// count) comes from a cost model fitted to measured plans (batch_plan).
//
// LDS layout: each 64-byte weight row keeps its four 16-byte chunks rotated by
// row / 4, each 128-byte activation row its eight chunks rotated by row / 2,
// so the 16 lanes of a ds_read_b128 phase (16 consecutive rows, one chunk)
// hit distinct bank groups. Tiles are dealt XCD-aware and each XCD starts an
// eighth of k later, as in the W8A8 kernel.
//
// Group scales along k (template G = 32 / 64 / 128; "FP8 weight-only
// (precision: fp8_weights)" and the per-group reading of the quantization
// pages: one scale per run of G weights of a row): each stage also stages its
// channels' group scales in LDS, the MFMA steps take the standard k order so a
// span of min(G, 64) k lies in one group, and every span's fp32 sum is scaled
// and added to the accumulator; the scale is never folded into the decoded
// weight. A k split writes partial sums that already hold the group scales.
#include <stdio.h>

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "ring.hpp"

namespace fp8w {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

template <typename A>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c)
{
    if constexpr (std::is_same<A, Bf16>::value)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                      0, 0, 0);
}

// G = 0: per-channel scales (applied in the epilogue). G = 32, 64, 128: group
// scales along k ([n, k / G] fp32), staged per stage next to the operands.
template <int BN, int BM, int WN, int WM, int G = 0>
struct BatchCfg {
    static constexpr int W = WN * WM;                  // waves
    static constexpr int FN = BN / WN / 32;            // 32-channel fragments per wave
    static constexpr int FM = BM / WM / 32;            // 32-token fragments per wave
    static constexpr int ABLK = BN / 16;               // 1 KB load blocks of weight rows (16 rows x 64 codes)
    static constexpr int BBLK = BM / 8;                // 1 KB load blocks of activation rows (8 rows x 64 values)
    static constexpr int BLOCKS = ABLK + BBLK;
    static constexpr int OPS = (BLOCKS + W - 1) / W;   // operand loads per wave; the last round repeats blocks
    static constexpr int SPANS = G == 0 ? 0 : (G >= 64 ? 1 : 64 / G);  // spans of one group in a 64-k stage
    static constexpr int SBLK = SPANS * (BN / 64);     // 256-byte scale loads per stage (64 channels each)
    static constexpr int SLW = (SBLK + W - 1) / W;     // per wave; repeats fill the last round
    static constexpr int LOADS = OPS + SLW;            // load instructions per wave and stage
    static constexpr int ABYTES = BN * 64;
    static constexpr int SOFF = ABYTES + BM * 128;     // the stage's group scales, [span][channel] fp32
    static constexpr int STAGE = SOFF + SPANS * BN * 4;
    static_assert(FN >= 1 && FM >= 1 && BN == FN * WN * 32 && BM == FM * WM * 32, "tile and wave layout");
    static_assert(G == 0 || ((G == 32 || G == 64 || G == 128) && BN % 64 == 0), "group size and tile");
    static_assert(LOADS * 2 < 64, "vmcnt range of the four-stage ring");
};

template <typename A, int BN, int BM, int WN, int WM, int G = 0>
struct BatchPipe {
    using C = BatchCfg<BN, BM, WN, WM, G>;
    const uint8_t* q;   // [n, k]
    const uint16_t* x;  // [m, k]
    const float* gs;    // G > 0: group scales [n, ng]
    int64_t n, m, k, n0, m0, ng, kz0;  // kz0: the k this workgroup's split slice starts at
    int64_t S, rot;  // stages; the k stage this workgroup starts at
    int lane, wave, wn, wm;

    // Stage s covers k stage (s + rot) mod S. Block b < ABLK holds weight rows
    // 16b .. 16b + 15 (lane l: row 16b + l / 4, slot l % 4, chunk (slot - row
    // / 4) mod 4); block ABLK + b holds activation rows 8b .. 8b + 7 (lane l:
    // row 8b + l / 8, slot l % 8, chunk (slot - row / 2) mod 8). Blocks are
    // dealt to the waves in turn; when they do not divide evenly, waves repeat
    // blocks of the first round (identical bytes to the same LDS address).
    // Rows past n or m read the last real row; their results are not stored.
    __device__ __forceinline__ void issue(int64_t s, uint8_t* buf) const
    {
        int64_t sr = s + rot;  // s < S and rot < S
        sr = sr < S ? sr : sr - S;
        const int64_t kb = sr * 64;
#pragma unroll
        for (int u = 0; u < C::OPS; ++u) {
            const int b = (wave * C::OPS + u) % C::BLOCKS;
            const void* src;
            if (b < C::ABLK) {
                const int r = 16 * b + (lane >> 2);
                const int chunk = ((lane & 3) - (r >> 2)) & 3;
                int64_t row = n0 + r;
                row = row < n ? row : n - 1;
                src = q + row * k + kb + 16 * chunk;
            } else {
                const int r = 8 * (b - C::ABLK) + (lane >> 3);
                const int chunk = ((lane & 7) - (r >> 1)) & 7;
                int64_t row = m0 + r;
                row = row < m ? row : m - 1;
                src = x + row * k + kb + 8 * chunk;
            }
            __builtin_amdgcn_global_load_lds(src, FP8W_LDS(buf + 1024 * b), 16, 0, 0);
        }
        if constexpr (G > 0) {
            // scale load u: span sp, channels 64c .. 64c + 63 (lane l: channel
            // 64c + l), the group that holds the span's k
#pragma unroll
            for (int u = 0; u < C::SLW; ++u) {
                const int idx = (wave * C::SLW + u) % C::SBLK;
                const int sp = idx / (BN / 64), c = idx % (BN / 64);
                int64_t row = n0 + 64 * c + lane;
                row = row < n ? row : n - 1;
                const int64_t gidx = (kz0 + kb) / G + (C::SPANS > 1 ? sp : 0);
                __builtin_amdgcn_global_load_lds(gs + row * ng + gidx,
                                                 FP8W_LDS(buf + C::SOFF + 4 * (sp * BN + 64 * c)), 4, 0, 0);
            }
        }
    }

    // one stage: FN weight and FM token fragments, four MFMA steps each pair
    __device__ __forceinline__ void compute(const uint8_t* buf, f32x16* acc) const
    {
        if constexpr (G > 0) {
            compute_grouped(buf, acc);
            return;
        }
        const int i = lane & 31, h = lane >> 5;
        u32x4 wc[C::FN][2];  // 32 codes of the lane's weight row: k 32h .. 32h + 31
#pragma unroll
        for (int f = 0; f < C::FN; ++f) {
            const int r = wn * (BN / WN) + 32 * f + i;
            const uint8_t* p = buf + 64 * r;
            wc[f][0] = *reinterpret_cast<const u32x4*>(p + 16 * ((2 * h + (r >> 2)) & 3));
            wc[f][1] = *reinterpret_cast<const u32x4*>(p + 16 * ((2 * h + 1 + (r >> 2)) & 3));
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            u32x4 a[C::FN], b[C::FM];
#pragma unroll
            for (int f = 0; f < C::FN; ++f) {
                const u32x4& c = wc[f][j >> 1];
                const u32x2 d0 = A::decode4((j & 1) ? c.z : c.x);
                const u32x2 d1 = A::decode4((j & 1) ? c.w : c.y);
                a[f] = u32x4{d0.x, d0.y, d1.x, d1.y};
            }
#pragma unroll
            for (int f = 0; f < C::FM; ++f) {
                const int r = wm * (BM / WM) + 32 * f + i;
                b[f] = *reinterpret_cast<const u32x4*>(buf + C::ABYTES + 128 * r + 16 * ((4 * h + j + (r >> 1)) & 7));
            }
#pragma unroll
            for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
                for (int fm = 0; fm < C::FM; ++fm)
                    acc[fn * C::FM + fm] = mfma32<A>(a[fn], b[fm], acc[fn * C::FM + fm]);
        }
    }

    // Group scales: MFMA step j sums the 16 consecutive k 16j .. 16j + 15 of
    // the stage (lane half h feeds 8h .. 8h + 7 of them), so a span of
    // min(G, 64) k lies in one group. Each span's exact fp32 sum is scaled by
    // its group's scale and added to the accumulator (one fmaf per output).
    __device__ __forceinline__ void compute_grouped(const uint8_t* buf, f32x16* acc) const
    {
        const int i = lane & 31, h = lane >> 5;
        constexpr int STEPS = 4 / C::SPANS;
#pragma unroll
        for (int sp = 0; sp < C::SPANS; ++sp) {
            u32x4 b[C::FM][STEPS];
#pragma unroll
            for (int f = 0; f < C::FM; ++f) {
                const int r = wm * (BM / WM) + 32 * f + i;
#pragma unroll
                for (int jj = 0; jj < STEPS; ++jj)
                    b[f][jj] = *reinterpret_cast<const u32x4*>(buf + C::ABYTES + 128 * r +
                                                               16 * ((2 * (sp * STEPS + jj) + h + (r >> 1)) & 7));
            }
            // one weight fragment at a time: a single span sum is live
#pragma unroll
            for (int fn = 0; fn < C::FN; ++fn) {
                const int r = wn * (BN / WN) + 32 * fn + i;
                u32x4 a[STEPS];
#pragma unroll
                for (int jj = 0; jj < STEPS; ++jj) {
                    const int j = sp * STEPS + jj;
                    const u32x2 c8 = *reinterpret_cast<const u32x2*>(buf + 64 * r + 16 * ((j + (r >> 2)) & 3) + 8 * h);
                    const u32x2 d0 = A::decode4(c8.x), d1 = A::decode4(c8.y);
                    a[jj] = u32x4{d0.x, d0.y, d1.x, d1.y};
                }
                // accumulator 4q + e of the fragment is channel 32 fn + 8q + 4h + e
                const float* sc =
                    reinterpret_cast<const float*>(buf + C::SOFF) + sp * BN + wn * (BN / WN) + 32 * fn + 4 * h;
                f32x4 s4[4];
#pragma unroll
                for (int qq = 0; qq < 4; ++qq)
                    s4[qq] = *reinterpret_cast<const f32x4*>(sc + 8 * qq);
#pragma unroll
                for (int fm = 0; fm < C::FM; ++fm) {
                    f32x16 part = f32x16{0.0f};
#pragma unroll
                    for (int jj = 0; jj < STEPS; ++jj)
                        part = mfma32<A>(a[jj], b[fm][jj], part);
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        acc[fn * C::FM + fm][e] = __builtin_fmaf(s4[e >> 2][e & 3], part[e], acc[fn * C::FM + fm][e]);
                }
            }
        }
    }
};

// Requires k % 256 == 0 (k / 64 stages, a multiple of the four-stage ring); x
// and q 16-byte aligned.
// grid.z > 1 splits k: workgroup row z owns k range [z * kc, (z + 1) * kc),
// kc = k / gridDim.z (a multiple of 256), and writes fp32 sums to part
// ([gridDim.z, m, n]) instead of y.
// G > 0: scale holds the group scales [n, k / G] and the epilogue adds only the
// bias (no split).
template <typename A, int BN, int BM, int WN, int WM, int G = 0, int GM = 4>
__global__ __launch_bounds__(WN* WM * kWave) __attribute__((amdgpu_waves_per_eu(G > 0 && WN * WM < 8 ? 2 : 1)))
void batch_kernel(const uint16_t* __restrict__ x,
                                                              const uint8_t* __restrict__ q,
                                                              const float* __restrict__ scale,
                                                              const uint16_t* __restrict__ bias,
                                                              uint16_t* __restrict__ y, int64_t m, int64_t n,
                                                              int64_t k, float* __restrict__ part)
{
    using P = BatchPipe<A, BN, BM, WN, WM, G>;
    using C = typename P::C;
    static_assert(BN <= C::W * kWave, "one epilogue operand per thread");
    __shared__ __attribute__((aligned(1024))) uint8_t b0[C::STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t b1[C::STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t b2[C::STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t b3[C::STAGE];
    __shared__ __attribute__((aligned(16))) float e_scale[BN];
    __shared__ __attribute__((aligned(16))) uint16_t e_bias[BN];

    int64_t tn, tm;
    xcd_tile_of<GM>(tn, tm);
    const int64_t kc = k / gridDim.z;
    P p;
    p.q = q + (int64_t)blockIdx.z * kc;
    p.x = x + (int64_t)blockIdx.z * kc;
    p.n = n;
    p.m = m;
    p.k = k;  // row stride
    p.n0 = tn * BN;
    p.m0 = tm * BM;
    p.lane = threadIdx.x & (kWave - 1);
    p.wave = threadIdx.x / kWave;
    p.wn = p.wave % WN;
    p.wm = p.wave / WN;
    p.S = kc / 64;
    p.gs = scale;
    p.ng = G > 0 ? k / G : 0;
    p.kz0 = (int64_t)blockIdx.z * kc;
    // the workgroups one XCD holds walk k in step; the XCDs start an eighth of k
    // apart (with a k split the XCD is taken within each slice of grid.z: the
    // tile order and the stagger are placement heuristics, the results do not
    // depend on them)
    p.rot = ((blockIdx.x + (int64_t)gridDim.x * blockIdx.y) % 8) * (p.S / 8);

    // epilogue operands of the tile's channels, one per thread: loaded before
    // the ring, held in registers through it (their latency overlaps the
    // ring's), then passed through LDS
    const int tt = threadIdx.x;
    float r_scale = 0.0f;
    uint16_t r_bias = 0;
    if (tt < BN) {
        const int64_t c = p.n0 + tt < n ? p.n0 + tt : n - 1;
        r_scale = G > 0 ? 1.0f : scale[c];  // group scales were applied in the k loop
        r_bias = bias_bits(bias, c);
    }

    f32x16 acc[C::FN * C::FM];
#pragma unroll
    for (int f = 0; f < C::FN * C::FM; ++f)
        acc[f] = f32x16{0.0f};
    run_ring<4, C::LOADS>(p, p.S, b0, b1, b2, b3, acc);
    if (tt < BN) {
        e_scale[tt] = r_scale;
        e_bias[tt] = r_bias;
    }
    __syncthreads();

    // lane (i, h) holds channels 8j + 4h + r (r = 0..3) of token i in
    // accumulators 4j + r of each fragment
    const int i = p.lane & 31, h = p.lane >> 5;
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm) {
        const int64_t t = p.m0 + p.wm * (BM / WM) + 32 * fm + i;
        if (t >= m)
            continue;
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn) {
            const f32x16 d = acc[fn * C::FM + fm];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int cl = p.wn * (BN / WN) + 32 * fn + 8 * j + 4 * h;
                const int64_t c0 = p.n0 + cl;
                if (part) {  // split k: fp32 sums of this k range
                    float* dst = part + ((int64_t)blockIdx.z * m + t) * n + c0;
                    if (c0 + 3 < n && ((reinterpret_cast<uintptr_t>(dst) & 15) == 0)) {
                        *reinterpret_cast<f32x4*>(dst) = f32x4{d[4 * j], d[4 * j + 1], d[4 * j + 2], d[4 * j + 3]};
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (c0 + r < n)
                                dst[r] = d[4 * j + r];
                    }
                    continue;
                }
                const f32x4 s4 = *reinterpret_cast<const f32x4*>(&e_scale[cl]);
                const u32x2 b4 = *reinterpret_cast<const u32x2*>(&e_bias[cl]);
                const uint16_t bb[4] = {(uint16_t)(b4.x & 0xffffu), (uint16_t)(b4.x >> 16), (uint16_t)(b4.y & 0xffffu),
                                        (uint16_t)(b4.y >> 16)};
                uint16_t o[4];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    o[r] = epilogue<A>(d[4 * j + r], s4[r], bb[r]);
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

template <typename A, int BN, int BM, int WN, int WM, int G = 0>
hipError_t launch_b(const void* x, int64_t m, int64_t k, const uint8_t* q, const float* scale, const void* bias,
                    int64_t n, void* y, int splits, float* part, hipStream_t stream)
{
    const dim3 grid((unsigned)((n + BN - 1) / BN), (unsigned)((m + BM - 1) / BM), (unsigned)splits);
    const dim3 block(WN * WM * kWave);
    hipLaunchKernelGGL((batch_kernel<A, BN, BM, WN, WM, G>), grid, block, 0, stream, static_cast<const uint16_t*>(x), q,
                       scale, static_cast<const uint16_t*>(bias), static_cast<uint16_t*>(y), m, n, k,
                       splits > 1 ? part : nullptr);
    return hipGetLastError();
}

struct BatchTile {
    int bn, bm, wn, wm;
};

constexpr BatchTile kBatchTiles[] = {{256, 128, 2, 4}, {256, 64, 4, 2}, {128, 128, 2, 4}, {128, 64, 4, 2},
                                     {64, 64, 2, 2},   {64, 32, 2, 1},  {32, 32, 1, 1}};

struct BatchPlan {
    BatchTile tile;
    int splits;
};

// Plan choice: the plan with the lowest modelled time, a model fitted to a
// sweep of every tile and split count over 40 shapes on MI355X (n = 4096,
// 14336, 28672; k = 4096, 14336; m = 48..512), where it picked a plan within
// 4 % of the fastest measured one on every shape (0.3 % on average):
//   - the operand stream (weight tiles read once per token tile, activation
//     tiles once per channel tile, padded to whole tiles) at 8 bytes per ns,
//     80 % of that for the 256-channel tiles, scaled by the share of the CUs
//     the grid fills (224 workgroups count as full; an eight-wave tile takes a
//     whole CU, so a grid past 256 of them pays for a partly empty round);
//   - or, when larger, the padded MFMA work at 1 PFLOP/s;
//   - plus, for a split, the fp32 partial sums written and read back at 2
//     bytes per ns.
// Split counts divide k / 256 and leave at least 512 k per workgroup; without
// workspace (allow_split false) every plan is single-pass. Ties go to the
// larger tile. With group scales (group > 0) only the tiles whose grouped
// kernel fits its registers without spills are planned: 64 x 64 and 64 x 32,
// and 128 x 64 for groups of 64 and 128 (the span sums of groups of 32 push
// it past the 256 registers an eight-wave tile has per lane; the larger tiles
// spill at every group size).
double batch_cost_us(const BatchTile& t, int64_t s, int64_t m, int64_t n, int64_t k)
{
    const int64_t tn = (n + t.bn - 1) / t.bn, tm = (m + t.bm - 1) / t.bm, wgs = tn * tm * s;
    const double mbytes = ((double)(tm * tn * t.bn) * (double)k + (double)(tn * tm * t.bm) * (double)k * 2.0) * 1e-6;
    const double gflop = 2.0 * (double)(tm * t.bm) * (double)(tn * t.bn) * (double)k * 1e-9;
    double fill = wgs < 224 ? (double)wgs / 224.0 : 1.0;
    if (t.wn * t.wm == 8 && wgs > 256)
        fill = (double)wgs / (256.0 * (double)((wgs + 255) / 256));
    const double t_mem = mbytes / (8.0 * (t.bn == 256 ? 0.8 : 1.0) * fill);
    const double t_mfma = gflop / (wgs < 256 ? (double)wgs / 256.0 : 1.0);
    const double t_split = s > 1 ? 8.0 * (double)s * (double)m * (double)n * 1e-6 / 2.0 : 0.0;
    return (t_mem > t_mfma ? t_mem : t_mfma) + t_split;
}

bool grouped_tile(const BatchTile& t, int64_t group)
{
    return t.bn == 64 || (t.bn == 128 && t.bm == 64 && group >= 64);
}

BatchPlan batch_plan(int64_t m, int64_t n, int64_t k, bool allow_split, int64_t group = 0)
{
    BatchPlan best{kBatchTiles[0], 1};
    double best_cost = -1.0;
    const int64_t k256 = k / 256;
    for (const BatchTile& t : kBatchTiles) {
        if (group > 0 && !grouped_tile(t, group))
            continue;
        for (int64_t s = 1; s <= (allow_split ? k256 : 1); ++s) {
            if (k256 % s != 0 || (s > 1 && k / s < 512))
                continue;
            const double c = batch_cost_us(t, s, m, n, k);
            if (best_cost < 0.0 || c < best_cost) {  // tiles are listed largest first: ties keep the larger
                best_cost = c;
                best = BatchPlan{t, (int)s};
            }
        }
    }
    return best;
}

template <typename A>
hipError_t launch_typed(const BatchPlan& p, const void* x, int64_t m, int64_t k, const uint8_t* q,
                        const float* scale, const void* bias, int64_t n, void* y, float* part, hipStream_t stream)
{
    const BatchTile& t = p.tile;
    const int s = p.splits;
    if (t.bn == 256 && t.bm == 128)
        return launch_b<A, 256, 128, 2, 4>(x, m, k, q, scale, bias, n, y, s, part, stream);
    if (t.bn == 256)
        return launch_b<A, 256, 64, 4, 2>(x, m, k, q, scale, bias, n, y, s, part, stream);
    if (t.bn == 128 && t.bm == 128)
        return launch_b<A, 128, 128, 2, 4>(x, m, k, q, scale, bias, n, y, s, part, stream);
    if (t.bn == 128)
        return launch_b<A, 128, 64, 4, 2>(x, m, k, q, scale, bias, n, y, s, part, stream);
    if (t.bm == 64)
        return launch_b<A, 64, 64, 2, 2>(x, m, k, q, scale, bias, n, y, s, part, stream);
    if (t.bn == 64)
        return launch_b<A, 64, 32, 2, 1>(x, m, k, q, scale, bias, n, y, s, part, stream);
    return launch_b<A, 32, 32, 1, 1>(x, m, k, q, scale, bias, n, y, s, part, stream);
}

template <typename A, int G>
hipError_t launch_grouped_tile(const BatchTile& t, int splits, const void* x, int64_t m, int64_t k, const uint8_t* q,
                               const float* gs, const void* bias, int64_t n, void* y, float* part,
                               hipStream_t stream)
{
    if constexpr (G >= 64) {
        if (t.bn == 128)
            return launch_b<A, 128, 64, 4, 2, G>(x, m, k, q, gs, bias, n, y, splits, part, stream);
    }
    if (t.bn != 64)
        return hipErrorInvalidValue;  // not a grouped tile (batch_plan never picks one)
    if (t.bm == 64)
        return launch_b<A, 64, 64, 2, 2, G>(x, m, k, q, gs, bias, n, y, splits, part, stream);
    return launch_b<A, 64, 32, 2, 1, G>(x, m, k, q, gs, bias, n, y, splits, part, stream);
}

template <typename A>
hipError_t launch_grouped_typed(const BatchPlan& p, int64_t group, const void* x, int64_t m, int64_t k,
                                const uint8_t* q, const float* gs, const void* bias, int64_t n, void* y,
                                float* part, hipStream_t stream)
{
    if (group == 32)
        return launch_grouped_tile<A, 32>(p.tile, p.splits, x, m, k, q, gs, bias, n, y, part, stream);
    if (group == 64)
        return launch_grouped_tile<A, 64>(p.tile, p.splits, x, m, k, q, gs, bias, n, y, part, stream);
    if (group == 128)
        return launch_grouped_tile<A, 128>(p.tile, p.splits, x, m, k, q, gs, bias, n, y, part, stream);
    return hipErrorInvalidValue;
}

}  // namespace

size_t batch_grouped_workspace_bytes(int64_t m, int64_t n, int64_t k, int64_t group)
{
    if (m < 1 || n < 1 || k < 256 || k % 256 != 0)
        return 0;
    const BatchPlan p = batch_plan(m, n, k, true, group);
    return p.splits > 1 ? (size_t)p.splits * (size_t)m * (size_t)n * sizeof(float) : 0;
}

// A k split writes partial sums that already hold the group scales; the reduce
// adds them in split order and applies only the bias (unit scale).
hipError_t launch_batch_grouped(const void* x, Act act, int64_t m, int64_t k, const uint8_t* q, const float* gs,
                                int64_t group, const void* bias, int64_t n, void* y, void* ws, size_t ws_bytes,
                                hipStream_t stream)
{
    if (m == 0 || n == 0)
        return hipSuccess;
    if (k % 256 != 0 || k == 0)
        return hipErrorInvalidValue;
    const size_t need = batch_grouped_workspace_bytes(m, n, k, group);
    const BatchPlan p = batch_plan(m, n, k, ws != nullptr && need > 0 && ws_bytes >= need, group);
    float* part = static_cast<float*>(ws);
    hipError_t e = hipErrorInvalidValue;
    if (act == Act::BF16)
        e = launch_grouped_typed<Bf16>(p, group, x, m, k, q, gs, bias, n, y, part, stream);
    else if (act == Act::FP16)
        e = launch_grouped_typed<F16>(p, group, x, m, k, q, gs, bias, n, y, part, stream);
    if (e != hipSuccess || p.splits <= 1)
        return e;
    return launch_splitk_reduce(part, p.splits, m, n, nullptr, bias, y, act, stream);
}

const char* batch_grouped_kernel_name(int64_t m, int64_t n, int64_t k, int64_t group, bool with_workspace)
{
    thread_local char name[96];
    const BatchPlan p = batch_plan(m, n, k, with_workspace, group);
    const BatchTile& t = p.tile;
    if (p.splits > 1)
        snprintf(name, sizeof name, "batch_grouped_kernel<BN=%d,BM=%d,W=%d>x%d+splitk_reduce_kernel", t.bn, t.bm,
                 t.wn * t.wm, p.splits);
    else
        snprintf(name, sizeof name, "batch_grouped_kernel<BN=%d,BM=%d,W=%d>", t.bn, t.bm, t.wn * t.wm);
    return name;
}

size_t batch_workspace_bytes(int64_t m, int64_t n, int64_t k)
{
    if (m < 1 || n < 1 || k < 256 || k % 256 != 0)
        return 0;
    const BatchPlan p = batch_plan(m, n, k, true);
    return p.splits > 1 ? (size_t)p.splits * (size_t)m * (size_t)n * sizeof(float) : 0;
}

hipError_t launch_batch(const void* x, Act act, int64_t m, int64_t k, const uint8_t* q, const float* scale,
                        const void* bias, int64_t n, void* y, void* ws, size_t ws_bytes, hipStream_t stream)
{
    if (m == 0 || n == 0)
        return hipSuccess;
    if (k % 256 != 0 || k == 0)
        return hipErrorInvalidValue;
    const size_t need = batch_workspace_bytes(m, n, k);
    const BatchPlan p = batch_plan(m, n, k, ws != nullptr && need > 0 && ws_bytes >= need);
    float* part = static_cast<float*>(ws);
    hipError_t e = hipErrorInvalidValue;
    if (act == Act::BF16)
        e = launch_typed<Bf16>(p, x, m, k, q, scale, bias, n, y, part, stream);
    else if (act == Act::FP16)
        e = launch_typed<F16>(p, x, m, k, q, scale, bias, n, y, part, stream);
    if (e != hipSuccess || p.splits <= 1)
        return e;
    return launch_splitk_reduce(part, p.splits, m, n, scale, bias, y, act, stream);
}

const char* batch_kernel_name(int64_t m, int64_t n, int64_t k, bool with_workspace)
{
    thread_local char name[96];
    const BatchPlan p = batch_plan(m, n, k, with_workspace);
    const BatchTile& t = p.tile;
    if (p.splits > 1)
        snprintf(name, sizeof name, "batch_kernel<BN=%d,BM=%d,W=%d>x%d+splitk_reduce_kernel", t.bn, t.bm, t.wn * t.wm,
                 p.splits);
    else
        snprintf(name, sizeof name, "batch_kernel<BN=%d,BM=%d,W=%d>", t.bn, t.bm, t.wn * t.wm);
    return name;
}

}  // namespace fp8w
