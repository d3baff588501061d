// The linear layer with group-wise weight scales along k: one fp32 scale per
// run of G weights of a row (G = 32, 64 or 128), scale [n, k / G] row-major.
//
//   y[m,n] = sum_j scale[n,j] * (sum_{i<G} x[m, jG+i] * value(q[n, jG+i])) + bias[n]
//
// "B04 - Precision & Quantization", sections "Post-training quantization
// versus quantization-aware training" (one scale per run of g weights of a
// row) and "The one that matters: quantization is a quality decision"
// (per-channel -> per-group when an outlier inside a row costs accuracy); the
// Day-98 lab page's "one scale per 32" census. Everything else is the
// per-channel contract of "FP8 weight-only (precision: fp8_weights)": exact
// decode, fp32 accumulation, bias in fp32, one rounding to the activation type.
//
// The scale now changes inside the k loop, so it cannot wait for the epilogue.
// It is not folded into the decoded weight either (a bf16/fp16 rounding of
// value * scale would round every weight a second time). Each kernel sums
// exact products over a span of k that lies inside one group, in fp32, and
// adds scale * that partial sum to the fp32 accumulator:
// * gemv_grouped_kernel: the 16-code chunk of the per-channel GEMV;
// * pipe_grouped_kernel: one v_mfma_f32_16x16x32 whose 32 k are one run of 32
//   consecutive k (a k order different from the per-channel ring's), with the
//   four scales a lane needs (its four D rows) read from LDS, where the ring
//   stages them next to the codes;
// * grouped_generic_kernel: the same MFMA step with guarded scalar loads, for
//   the shapes and alignments the other two do not take.
#include <math.h>
#include <stdio.h>

#include "common.hpp"
#include "kernels.hpp"
#include "ring.hpp"

namespace fp8w {
namespace {

// ---------------------------------------------------------------- M = 1
// The per-channel GEMV's layout (R rows per NT-thread workgroup, thread t reads
// chunk t of each row, groups of U passes in flight, double-buffered with DB),
// with a per-chunk partial sum and the chunk's group scale loaded beside its
// codes.
template <typename A, int R>
__device__ __forceinline__ void grouped_chunk(const u32x4* code, const float* sc, u32x4 x0, u32x4 x1, float* acc)
{
    float xf[16];
    const uint32_t xw[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        xf[2 * e + 0] = A::lo_f32(xw[e]);
        xf[2 * e + 1] = A::hi_f32(xw[e]);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const uint32_t cw[4] = {code[r].x, code[r].y, code[r].z, code[r].w};
        float dot = 0.0f;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            float w0, w1, w2, w3;
            decode4_f32(cw[d], w0, w1, w2, w3);
            dot = __builtin_fmaf(xf[4 * d + 0], w0, dot);
            dot = __builtin_fmaf(xf[4 * d + 1], w1, dot);
            dot = __builtin_fmaf(xf[4 * d + 2], w2, dot);
            dot = __builtin_fmaf(xf[4 * d + 3], w3, dot);
        }
        acc[r] = __builtin_fmaf(sc[r], dot, acc[r]);
    }
}

// U passes of a thread's chunks for R rows, their group scales and the
// activation chunks they share; load() issues all of it back to back.
template <int R, int U>
struct GGroup {
    u32x4 code[U][R];
    u32x4 xv[U][2];
    float sc[U][R];
    __device__ __forceinline__ void load(const uint8_t* const* qr, const float* const* sr, const uint16_t* xp,
                                         int64_t c0, int t, int nt, int lg_chunks)
    {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t c = c0 + (int64_t)nt * u;
            const int64_t off = c * 16;
            const int64_t gi = (c + t) >> lg_chunks;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                code[u][r] = load_stream16(qr[r] + off);
                sc[u][r] = sr[r][gi];
            }
            xv[u][0] = load16(xp + off);
            xv[u][1] = load16(xp + off + 8);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    template <typename A>
    __device__ __forceinline__ void use(float* acc) const
    {
#pragma unroll
        for (int u = 0; u < U; ++u)
            grouped_chunk<A, R>(code[u], sc[u], xv[u][0], xv[u][1], acc);
    }
};

// The output pointer comes last, so that the sizes lie in the 56 bytes of
// arguments the wave finds preloaded in SGPRs.
template <typename A, int R, int U, int NT, bool DB>
__global__ __launch_bounds__(NT) void gemv_grouped_kernel(const uint16_t* __restrict__ x,
                                                          const uint8_t* __restrict__ q,
                                                          const float* __restrict__ scale,
                                                          const uint16_t* __restrict__ bias, int64_t n, int64_t k,
                                                          int lg_chunks,  // log2(G / 16)
                                                          uint16_t* __restrict__ y)
{
    constexpr int NW = NT / kWave;
    __shared__ float red[NW][R];
    const int t = threadIdx.x;
    const int lane = t & (kWave - 1);
    const int wave = t >> 6;
    const int64_t row0 = (int64_t)blockIdx.x * R;
    const int64_t nch = k >> 4;
    const int64_t ng = nch >> lg_chunks;

    const uint8_t* qr[R];
    const float* sr[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t row = row0 + r < n ? row0 + r : n - 1;
        qr[r] = q + row * k + (int64_t)t * 16;
        sr[r] = scale + row * ng;
    }
    const uint16_t* xp = x + (int64_t)t * 16;
    const int64_t er = row0 + (t % R) < n ? row0 + (t % R) : n - 1;
    const uint16_t bi = bias_bits(bias, er);

    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
        acc[r] = 0.0f;

    constexpr int64_t GS = (int64_t)NT * U;
    const int64_t G = nch / GS;
    GGroup<R, U> ga, gb;
    if constexpr (DB) {
        int64_t g = 0;
        if (G > 0) {
            ga.load(qr, sr, xp, 0, t, NT, lg_chunks);
            for (; g + 2 < G; g += 2) {
                gb.load(qr, sr, xp, (g + 1) * GS, t, NT, lg_chunks);
                ga.template use<A>(acc);
                ga.load(qr, sr, xp, (g + 2) * GS, t, NT, lg_chunks);
                gb.template use<A>(acc);
            }
            if (g + 1 < G) {
                gb.load(qr, sr, xp, (g + 1) * GS, t, NT, lg_chunks);
                ga.template use<A>(acc);
                gb.template use<A>(acc);
            } else {
                ga.template use<A>(acc);
            }
        }
    } else {
        for (int64_t g = 0; g < G; ++g) {
            ga.load(qr, sr, xp, g * GS, t, NT, lg_chunks);
            ga.template use<A>(acc);
        }
    }
    for (int64_t c0 = G * GS; c0 < nch; c0 += NT) {  // tail passes
        if (c0 + t < nch) {
            const int64_t off = c0 * 16;
            const int64_t gi = (c0 + t) >> lg_chunks;
            u32x4 code[R];
            float sc[R];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                code[r] = load_stream16(qr[r] + off);
                sc[r] = sr[r][gi];
            }
            grouped_chunk<A, R>(code, sc, load16(xp + off), load16(xp + off + 8), acc);
        }
    }

    if constexpr (NW == 1) {
        // one wave: every lane holds every row's sum after the butterfly
        float tot = 0.0f;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float s = wave_sum(acc[r]);
            if (t == r)
                tot = s;
        }
        if (t < R && row0 + t < n)
            y[row0 + t] = epilogue<A>(tot, 1.0f, bi);
        return;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const float s = wave_sum(acc[r]);
        if (lane == 0)
            red[wave][r] = s;
    }
    __syncthreads();
    if (t < R && row0 + t < n) {
        float s = red[0][t];
#pragma unroll
        for (int w = 1; w < NW; ++w)
            s += red[w][t];
        y[row0 + t] = epilogue<A>(s, 1.0f, bi);
    }
}

// ---------------------------------------------------------------- M = 2..32
// The direct-to-LDS ring of the per-channel skinny kernel (same code and
// activation staging: rotated 16-byte chunks, XR activation rows, KP k-parts,
// NS stages, k-staggered start), plus each wave's group scales for the stage:
// 16 channels x (256 / G) groups, 4 bytes per lane (lane l of instruction p
// brings scale[channel (64p + l) % 16][group ((64p + l) / 16) mod (256 / G)],
// landing at 4 (64p + l), so the LDS holds them as [group][channel]; for
// G = 128 the surplus lanes write copies that are never read).
template <int XR, int CT, int KP, int NS, int G>
struct PipeGCfg {
    static_assert(XR % 2 == 0 && XR >= 2 && XR <= 32, "activation rows");
    static_assert(G == 32 || G == 64 || G == 128, "group size");
    static constexpr int MT = XR > 16 ? 2 : 1;
    static constexpr int W = CT * KP;
    static constexpr int CODE = 16 * 256;
    static constexpr int XPART = XR * 512;
    static constexpr int NGS = 256 / G;                  // groups per wave and stage
    static constexpr int SLW = NGS * 16 * 4 > 256 ? 2 : 1;  // scale load instructions per wave
    static constexpr int SCB = 256 * SLW;                // scale bytes per wave and stage
    static constexpr int STAGE = W * CODE + KP * XPART + W * SCB;
    static constexpr int XLOADS = (XR / 2) * KP;
    static constexpr int XPW = (XLOADS + W - 1) / W;
    static constexpr int LOADS = 4 + XPW + SLW;
    static_assert(LOADS * (NS - 2) < 64, "vmcnt range");
};

template <typename A, int XR, int CT, int KP, int NS, int G>
struct PipeG {
    using C = PipeGCfg<XR, CT, KP, NS, G>;
    static constexpr int MT = C::MT;
    static constexpr int NGS = C::NGS;
    static constexpr int TPG = G / 32;  // MFMAs per group

    const uint16_t* x;
    const uint8_t* q;
    const float* scale;
    int m;
    int64_t n, k, n0, ng;
    int64_t S, rot;
    int lane, wave, ct, kp;

    __device__ __forceinline__ void issue(int64_t s, uint8_t* buf) const
    {
        int64_t sr = s + rot;
        sr = sr < S ? sr : sr - S;
        const int64_t kb = sr * (KP * 256);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 4 * j + (lane >> 4);
            const int chunk = ((lane & 15) - r) & 15;
            int64_t row = n0 + 16 * ct + r;
            row = row < n ? row : n - 1;
            const uint8_t* src = q + row * k + kb + kp * 256 + chunk * 16;
            __builtin_amdgcn_global_load_lds((const void*)src, FP8W_LDS(buf + wave * C::CODE + j * 1024), 16, 0,
                                             2 /* non-temporal */);
        }
#pragma unroll
        for (int u = 0; u < C::XPW; ++u) {
            const int p = (wave * C::XPW + u) % C::XLOADS;
            const int kpx = p / (XR / 2);
            const int pair = p % (XR / 2);
            const int t = 2 * pair + (lane >> 5);
            const int chunk = ((lane & 31) - t) & 31;
            const int tc = t < m ? t : m - 1;
            const uint16_t* src = x + (int64_t)tc * k + kb + kpx * 256 + chunk * 8;
            __builtin_amdgcn_global_load_lds((const void*)src,
                                             FP8W_LDS(buf + C::W * C::CODE + kpx * C::XPART + pair * 1024), 16, 0, 0);
        }
        const int64_t g0 = (kb + kp * 256) / G;
#pragma unroll
        for (int p = 0; p < C::SLW; ++p) {
            const int idx = 64 * p + lane;
            int64_t row = n0 + 16 * ct + (idx & 15);
            row = row < n ? row : n - 1;
            const float* src = scale + row * ng + g0 + ((idx >> 4) % NGS);
            __builtin_amdgcn_global_load_lds((const void*)src,
                                             FP8W_LDS(buf + C::W * C::CODE + KP * C::XPART + wave * C::SCB + 256 * p),
                                             4, 0, 0);
        }
    }

    // MFMA t of this wave's 256 k covers k = 32t .. 32t + 31: lane (i, g)
    // takes codes 32t + 8g .. +7 of channel i and the same k of token i. The
    // G / 32 MFMAs of one group chain into one partial sum, which is scaled and
    // added once. The stage runs in three phases, fenced so the scheduler
    // cannot interleave them back into a chain: every LDS read; every decode
    // and MFMA; then the scaled adds, by which time the products are done.
    // Interleaved, each step waited for its own LDS read and MFMA result.
    __device__ __forceinline__ void compute(const uint8_t* buf, f32x4* acc) const
    {
        const int i = lane & 15, g = lane >> 4;
        const uint8_t* cb = buf + wave * C::CODE;
        const uint8_t* xb = buf + C::W * C::CODE + kp * C::XPART;
        const uint8_t* sb = buf + C::W * C::CODE + KP * C::XPART + wave * C::SCB;
        const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
        u32x2 c8[8];
        u32x4 b[8][MT];
        f32x4 s4[NGS];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int c = 2 * t + (g >> 1);
            c8[t] = *reinterpret_cast<const u32x2*>(cb + 16 * (16 * i + ((c + i) & 15)) + 8 * (g & 1));
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int tok = (i + 16 * mt) < XR ? (i + 16 * mt) : XR - 1;
                b[t][mt] = *reinterpret_cast<const u32x4*>(xb + 16 * (32 * tok + ((4 * t + g + tok) & 31)));
            }
        }
#pragma unroll
        for (int j = 0; j < NGS; ++j)
            s4[j] = *reinterpret_cast<const f32x4*>(sb + 4 * (16 * j + 4 * g));
        __builtin_amdgcn_sched_barrier(0);
        f32x4 part[NGS][MT];
#pragma unroll
        for (int j = 0; j < NGS; ++j)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                part[j][mt] = zero;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const u32x2 d0 = A::decode4(c8[t].x), d1 = A::decode4(c8[t].y);
            const u32x4 a = {d0.x, d0.y, d1.x, d1.y};
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                part[t / TPG][mt] = A::mfma(a, b[t][mt], part[t / TPG][mt]);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < NGS; ++j)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                acc[mt].x = __builtin_fmaf(s4[j].x, part[j][mt].x, acc[mt].x);
                acc[mt].y = __builtin_fmaf(s4[j].y, part[j][mt].y, acc[mt].y);
                acc[mt].z = __builtin_fmaf(s4[j].z, part[j][mt].z, acc[mt].z);
                acc[mt].w = __builtin_fmaf(s4[j].w, part[j][mt].w, acc[mt].w);
            }
    }
};

// Requires k % (KP * 256 * NS) == 0 and scale 4-byte aligned.
template <typename A, int XR, int CT, int KP, int NS, int G>
__global__ __launch_bounds__(CT* KP * kWave) void pipe_grouped_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ q, const float* __restrict__ scale,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ y, int m, int64_t n, int64_t k)
{
    using P = PipeG<A, XR, CT, KP, NS, G>;
    using C = typename P::C;
    constexpr int MT = C::MT;
    __shared__ __attribute__((aligned(1024))) uint8_t b0[C::STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t b1[C::STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t b2[NS > 2 ? C::STAGE : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t b3[NS > 3 ? C::STAGE : 16];

    P p;
    p.x = x;
    p.q = q;
    p.scale = scale;
    p.m = m;
    p.n = n;
    p.k = k;
    p.ng = k / G;
    p.lane = threadIdx.x & (kWave - 1);
    p.wave = threadIdx.x / kWave;
    p.ct = p.wave % CT;
    p.kp = p.wave / CT;
    p.n0 = (int64_t)blockIdx.x * (16 * CT);

    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
        acc[mt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    uint16_t bi[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        int64_t ch = p.n0 + 16 * p.ct + 4 * (p.lane >> 4) + r;
        ch = ch < n ? ch : n - 1;
        bi[r] = bias_bits(bias, ch);
    }

    const int64_t S = k / (KP * 256);
    p.S = S;
    p.rot = (int64_t)(blockIdx.x / 8) % S;
    run_ring<NS, C::LOADS>(p, S, b0, b1, b2, b3, acc);

    static_assert(C::STAGE >= C::W * MT * kWave * 16, "reduction fits in a stage buffer");
    f32x4(*part)[MT][kWave] = reinterpret_cast<f32x4(*)[MT][kWave]>(b0);
    __syncthreads();
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
        part[p.wave][mt][p.lane] = acc[mt];
    __syncthreads();
    if (p.kp != 0)
        return;
    const int i = p.lane & 15, g = p.lane >> 4;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        f32x4 sum = part[p.ct][mt][p.lane];
#pragma unroll
        for (int kp = 1; kp < KP; ++kp)
            sum += part[kp * CT + p.ct][mt][p.lane];
        const int tok = i + 16 * mt;
        if (tok >= m)
            continue;
        const float v[4] = {sum.x, sum.y, sum.z, sum.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t ch = p.n0 + 16 * p.ct + 4 * g + r;
            if (ch < n)
                y[(int64_t)tok * n + ch] = epilogue<A>(v[r], 1.0f, bi[r]);
        }
    }
}

// ---------------------------------------------------------------- any shape
// One wave per 16-channel x 16-token tile, four waves per workgroup along n.
// Each step of 32 k is one MFMA on guarded scalar loads (any m, n, any 2-byte
// alignment of x, any alignment of q), then the scaled add.
template <typename A>
__global__ __launch_bounds__(256) void grouped_generic_kernel(const uint16_t* __restrict__ x,
                                                             const uint8_t* __restrict__ q,
                                                             const float* __restrict__ scale,
                                                             const uint16_t* __restrict__ bias,
                                                             uint16_t* __restrict__ y, int64_t m, int64_t n,
                                                             int64_t k, int lg)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t n0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 16;
    const int64_t m0 = (int64_t)blockIdx.y * 16;
    if (n0 >= n)
        return;
    const int i = lane & 15, g = lane >> 4;
    const int64_t ch = n0 + i, tok = m0 + i;
    const bool chok = ch < n, tokok = tok < m;
    const uint8_t* qp = q + (chok ? ch : 0) * k + 8 * g;
    const uint16_t* xp = x + (tokok ? tok : 0) * k + 8 * g;
    const int64_t ng = k >> lg;
    const float* sp[4];
    bool sok[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int64_t c = n0 + 4 * g + r;
        sok[r] = c < n;
        sp[r] = scale + (sok[r] ? c : 0) * ng;
    }
    const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
    f32x4 acc = zero;
    for (int64_t k0 = 0; k0 < k; k0 += 32) {
        uint32_t cw[2] = {0u, 0u};
        uint32_t xw[4] = {0u, 0u, 0u, 0u};
        if (chok) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                cw[e >> 2] |= (uint32_t)qp[k0 + e] << (8 * (e & 3));
        }
        if (tokok) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                xw[e >> 1] |= (uint32_t)xp[k0 + e] << (16 * (e & 1));
        }
        const u32x2 d0 = A::decode4(cw[0]), d1 = A::decode4(cw[1]);
        const u32x4 a = {d0.x, d0.y, d1.x, d1.y};
        const u32x4 b = {xw[0], xw[1], xw[2], xw[3]};
        const f32x4 part = A::mfma(a, b, zero);
        const int64_t gi = k0 >> lg;
        acc.x = __builtin_fmaf(sok[0] ? sp[0][gi] : 0.0f, part.x, acc.x);
        acc.y = __builtin_fmaf(sok[1] ? sp[1][gi] : 0.0f, part.y, acc.y);
        acc.z = __builtin_fmaf(sok[2] ? sp[2][gi] : 0.0f, part.z, acc.z);
        acc.w = __builtin_fmaf(sok[3] ? sp[3][gi] : 0.0f, part.w, acc.w);
    }
    if (!tokok)
        return;
    const float v[4] = {acc.x, acc.y, acc.z, acc.w};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int64_t c = n0 + 4 * g + r;
        if (c < n)
            y[tok * n + c] = epilogue<A>(v[r], 1.0f, bias, c);
    }
}

// ---------------------------------------------------------------- dequantize
// out[r, j] = out_type(fl32(value(q[r, j]) * scale[r, j / G])), grid-stride.
template <typename Out>
__global__ __launch_bounds__(256) void dequantize_grouped_kernel(const uint8_t* __restrict__ q,
                                                                 const float* __restrict__ scale, int64_t n,
                                                                 int64_t k, int lg, Out out)
{
    const int64_t total = n * k;
    const int64_t ng = k >> lg;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
        const int64_t r = e / k, j = e - r * k;
        float v, unused0, unused1, unused2;
        decode4_f32((uint32_t)q[e], v, unused0, unused1, unused2);
        out.store(e, v * scale[r * ng + (j >> lg)]);
    }
}

struct OutF32 {
    float* p;
    __device__ __forceinline__ void store(int64_t e, float v) const { p[e] = v; }
};

template <typename A>
struct OutA16 {
    uint16_t* p;
    __device__ __forceinline__ void store(int64_t e, float v) const { p[e] = A::from_f32(v); }
};

// ---------------------------------------------------------------- dispatch
struct GroupedPlan {
    bool pipe;
    int xr, ct, kp, ns;
};

// The per-channel skinny plan's choices, on the instances compiled here: 64
// channels per workgroup on layers of 8192 channels and more (the ring at
// NS = 2 on the widest), 16 channels with two k-parts below; NS falls to 2
// where k or the LDS (32 activation rows with two k-parts) needs it; shapes
// whose k the ring cannot tile take the generic kernel.
GroupedPlan plan_grouped(int64_t m, int64_t n, int64_t k)
{
    GroupedPlan p{};
    p.xr = m <= 4 ? 4 : m <= 8 ? 8 : m <= 16 ? 16 : 32;
    if (n >= 8192) {
        p.ct = 4;
        p.kp = 1;
        p.ns = n >= 16384 ? 2 : 4;
    } else {
        p.ct = 1;
        p.kp = 2;
        p.ns = p.xr == 32 ? 2 : 4;
    }
    if (k % (p.kp * 256 * p.ns) != 0)
        p.ns = 2;
    p.pipe = k % (p.kp * 256 * p.ns) == 0;
    return p;
}

template <typename A, int XR, int CT, int KP, int NS, int G>
hipError_t launch_pipe_g(const void* x, int m, int64_t k, const uint8_t* q, const float* scale, const void* bias,
                         int64_t n, void* y, hipStream_t stream)
{
    const dim3 grid((unsigned)((n + 16 * CT - 1) / (16 * CT))), block(CT * KP * kWave);
    hipLaunchKernelGGL((pipe_grouped_kernel<A, XR, CT, KP, NS, G>), grid, block, 0, stream,
                       static_cast<const uint16_t*>(x), q, scale, static_cast<const uint16_t*>(bias),
                       static_cast<uint16_t*>(y), m, n, k);
    return hipGetLastError();
}

template <typename A, int XR, int G>
hipError_t launch_pipe_g_xr(const GroupedPlan& p, const void* x, int m, int64_t k, const uint8_t* q,
                            const float* scale, const void* bias, int64_t n, void* y, hipStream_t stream)
{
    const int key = p.ct * 100 + p.kp * 10 + p.ns;
    switch (key) {
    case 412: return launch_pipe_g<A, XR, 4, 1, 2, G>(x, m, k, q, scale, bias, n, y, stream);
    case 414: return launch_pipe_g<A, XR, 4, 1, 4, G>(x, m, k, q, scale, bias, n, y, stream);
    case 122: return launch_pipe_g<A, XR, 1, 2, 2, G>(x, m, k, q, scale, bias, n, y, stream);
    case 124:
        if constexpr (XR <= 16)
            return launch_pipe_g<A, XR, 1, 2, 4, G>(x, m, k, q, scale, bias, n, y, stream);
        return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
    }
}

template <typename A, int G>
hipError_t launch_pipe_g_plan(const GroupedPlan& p, const void* x, int m, int64_t k, const uint8_t* q,
                              const float* scale, const void* bias, int64_t n, void* y, hipStream_t stream)
{
    switch (p.xr) {
    case 4: return launch_pipe_g_xr<A, 4, G>(p, x, m, k, q, scale, bias, n, y, stream);
    case 8: return launch_pipe_g_xr<A, 8, G>(p, x, m, k, q, scale, bias, n, y, stream);
    case 16: return launch_pipe_g_xr<A, 16, G>(p, x, m, k, q, scale, bias, n, y, stream);
    default: return launch_pipe_g_xr<A, 32, G>(p, x, m, k, q, scale, bias, n, y, stream);
    }
}

template <typename A>
hipError_t launch_grouped_typed(int path, const void* x, int64_t m, int64_t k, const uint8_t* q,
                                const float* scale, int lg, const void* bias, int64_t n, void* y,
                                hipStream_t stream)
{
    if (path == 0) {  // the per-channel GEMV's tiles (one-wave double-buffered below 96 MB)
        if (n * k >= ((int64_t)96 << 20)) {
            hipLaunchKernelGGL((gemv_grouped_kernel<A, 4, 2, 128, false>), dim3((unsigned)((n + 3) / 4)), dim3(128), 0,
                               stream, static_cast<const uint16_t*>(x), q, scale,
                               static_cast<const uint16_t*>(bias), n, k, lg - 4, static_cast<uint16_t*>(y));
        } else {
            hipLaunchKernelGGL((gemv_grouped_kernel<A, 2, 2, 64, true>), dim3((unsigned)((n + 1) / 2)), dim3(64), 0,
                               stream, static_cast<const uint16_t*>(x), q, scale,
                               static_cast<const uint16_t*>(bias), n, k, lg - 4, static_cast<uint16_t*>(y));
        }
        return hipGetLastError();
    }
    if (path == 1) {
        const GroupedPlan p = plan_grouped(m, n, k);
        if (p.pipe) {
            const int mi = (int)m;
            if (lg == 5)
                return launch_pipe_g_plan<A, 32>(p, x, mi, k, q, scale, bias, n, y, stream);
            if (lg == 6)
                return launch_pipe_g_plan<A, 64>(p, x, mi, k, q, scale, bias, n, y, stream);
            return launch_pipe_g_plan<A, 128>(p, x, mi, k, q, scale, bias, n, y, stream);
        }
    }
    const dim3 grid((unsigned)((n + 63) / 64), (unsigned)((m + 15) / 16)), block(256);
    hipLaunchKernelGGL((grouped_generic_kernel<A>), grid, block, 0, stream, static_cast<const uint16_t*>(x), q,
                       scale, static_cast<const uint16_t*>(bias), static_cast<uint16_t*>(y), m, n, k, lg);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_linear_grouped(int path, const void* x, Act act, int64_t m, int64_t k, const uint8_t* q,
                                 const float* scale, int64_t group, const void* bias, int64_t n, void* y, void* ws,
                                 size_t ws_bytes, hipStream_t stream)
{
    if (m == 0 || n == 0)
        return hipSuccess;
    if (k == 0)
        path = 2;  // y = bias: the generic kernel's k loop is empty
    if (path == 3)
        return launch_batch_grouped(x, act, m, k, q, scale, group, bias, n, y, ws, ws_bytes, stream);
    const int lg = 63 - __builtin_clzll((unsigned long long)group);
    if (act == Act::BF16)
        return launch_grouped_typed<Bf16>(path, x, m, k, q, scale, lg, bias, n, y, stream);
    if (act == Act::FP16)
        return launch_grouped_typed<F16>(path, x, m, k, q, scale, lg, bias, n, y, stream);
    return hipErrorInvalidValue;
}

const char* grouped_kernel_name(int path, int64_t m, int64_t n, int64_t k, int64_t group, bool with_workspace)
{
    static thread_local char name[96];
    if (path == 0)
        return n * k >= ((int64_t)96 << 20) ? "gemv_grouped_kernel<R=4,U=2,NT=128>"
                                            : "gemv_grouped_kernel<R=2,U=2,NT=64,DB>";
    if (path == 3)
        return batch_grouped_kernel_name(m, n, k, group, with_workspace);
    if (path == 1) {
        const GroupedPlan p = plan_grouped(m, n, k);
        if (p.pipe) {
            snprintf(name, sizeof name, "pipe_grouped_kernel<XR=%d,CT=%d,KP=%d,NS=%d>", p.xr, p.ct, p.kp, p.ns);
            return name;
        }
    }
    return "grouped_generic_kernel";
}

hipError_t launch_dequantize_grouped(const uint8_t* q, const float* scale, int64_t group, int64_t n, int64_t k,
                                     void* out, Act out_type, hipStream_t stream)
{
    if (n == 0 || k == 0)
        return hipSuccess;
    const int lg = 63 - __builtin_clzll((unsigned long long)group);
    const int64_t total = n * k;
    const int64_t blocks64 = (total + 255) / 256;
    const unsigned blocks = (unsigned)(blocks64 < 65536 ? blocks64 : 65536);
    switch (out_type) {
    case Act::FP32:
        hipLaunchKernelGGL((dequantize_grouped_kernel<OutF32>), dim3(blocks), dim3(256), 0, stream, q, scale, n, k,
                           lg, OutF32{static_cast<float*>(out)});
        break;
    case Act::BF16:
        hipLaunchKernelGGL((dequantize_grouped_kernel<OutA16<Bf16>>), dim3(blocks), dim3(256), 0, stream, q, scale,
                           n, k, lg, OutA16<Bf16>{static_cast<uint16_t*>(out)});
        break;
    case Act::FP16:
        hipLaunchKernelGGL((dequantize_grouped_kernel<OutA16<F16>>), dim3(blocks), dim3(256), 0, stream, q, scale,
                           n, k, lg, OutA16<F16>{static_cast<uint16_t*>(out)});
        break;
    }
    return hipGetLastError();
}

}  // namespace fp8w
