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
// * seg_kernel (M <= 8 on layers under 8192 channels, and shapes the pipe
//   ring cannot tile): one MFMA covers MP = 16/SEG
//   channels x MP tokens x SEG k-segments. A row i = MP*s + c and B column
//   j = MP*s + t; only the D blocks with matching segment (s == s') are kept and
//   summed over s at the end. Lane (i, g) reads the 16 codes of channel c at
//   kb + 16*SEG*g + 16*s, so a quarter-wave reads 16*SEG contiguous bytes per
//   channel (64 B for M <= 4). T channel groups per wave share the activation
//   fragments; W waves split k.
// * pipe_kernel (M = 2..32 on layers of 4096 channels and more): codes and
//   activations travel from HBM/L2 straight into LDS with gfx950's direct
//   global-to-LDS loads (no register staging), through a ring of NS stage
//   buffers, so NS - 1 stages of every workgroup are in flight while the
//   matrix cores work on the oldest one. Each load instruction moves 1 KB: a
//   quarter-wave fetches 256 contiguous bytes of one code row (or half a row of
//   activations), and the lane-to-address mapping rotates every row's 16-byte
//   chunks so that the MFMA-layout reads from LDS hit 16 distinct banks.
//
// One workgroup owns a block of output channels over the whole of k (no
// cross-workgroup reduction: on MI355X the eight XCDs have separate L2s and a
// device-scope handoff between workgroups costs more than it saves).
#include <stdio.h>

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "ring.hpp"

namespace fp8w {
namespace {

// ---------------------------------------------------------------- seg_kernel
// The output pointer comes last, so that the sizes lie in the 56 bytes of
// arguments the wave finds preloaded in SGPRs.
template <typename A, int SEG, int T, int W, int U, int MT>
__global__ __launch_bounds__(W* kWave) void seg_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ q, const float* __restrict__ scale,
    const uint16_t* __restrict__ bias, int m, int64_t n, int64_t k, uint16_t* __restrict__ y)
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

// ---------------------------------------------------------------- pipe_kernel
// XR activation rows are fetched (m <= XR; MFMA columns past XR read row XR - 1
// and are discarded); CT channel tiles of 16 and KP k-parts make the
// workgroup's CT * KP waves; NS stage buffers; one stage is 256 k per wave.
// CB is the alignment of the code rows the kernel is built for: 16 (16-byte
// loads), 8 (rows 8-byte aligned: 16-byte loads from each row's first 16-byte
// boundary, a workgroup's rows all of one parity) or 4 (4-byte loads).
template <int XR, int CT, int KP, int NS, int CB = 16>
struct PipeCfg {
    static_assert(CB == 16 || CB == 8 || CB == 4, "code row alignment");
    static_assert(XR % 2 == 0 && XR >= 2 && XR <= 32, "activation rows");
    static_assert(NS >= 2 && NS <= 4, "stages");
    static constexpr int MT = XR > 16 ? 2 : 1;      // 16-token MFMA tiles
    static constexpr int W = CT * KP;               // waves
    static constexpr int CODE = 16 * 256;           // code bytes per wave and stage
    static constexpr int XPART = XR * 512;          // activation bytes per k-part and stage
    static constexpr int STAGE = W * CODE + KP * XPART;
    static constexpr int XLOADS = (XR / 2) * KP;    // 1 KB activation loads per stage
    static constexpr int XPW = (XLOADS + W - 1) / W;  // per wave; duplicates fill the last round
    static constexpr int CLOADS = CODE / (kWave * (CB == 4 ? 4 : 16));  // code loads per wave and stage
    static constexpr int LOADS = CLOADS + XPW;      // load instructions per wave and stage
    static_assert(LOADS * (NS - 2) < 64, "vmcnt range");
};

// Eight codes as two 4-byte loads (the rows these blocks read may be only 4-byte aligned).
__device__ __forceinline__ u32x2 load_codes8(const uint8_t* p)
{
    const uint32_t* w = reinterpret_cast<const uint32_t*>(p);
    return u32x2{w[0], w[1]};
}

template <typename A, int XR, int CT, int KP, int NS, int CB = 16>
struct Pipe {
    using C = PipeCfg<XR, CT, KP, NS, CB>;
    static constexpr int MT = C::MT;
    // CB == 8: the workgroup's channels are n0, n0 + 2, .. (one parity), which
    // share their alignment mod 16 (2k % 16 == 0)
    static constexpr int RS = CB == 8 ? 2 : 1;

    const uint16_t* x;  // CB == 8: both advanced by the workgroup's shift sh
    const uint8_t* q;
    int m;
    int64_t n, k, n0;
    int64_t S, rot;  // stages; this workgroup's first stage
    int64_t T, sh;   // columns outside the ring (k - kr); columns before the ring (0, or 8 for CB == 8)
    int lane, wave, ct, kp;

    // channel c of the workgroup (16 ct + r), clamped to a real row of the
    // same alignment; results of clamped rows are never stored
    __device__ __forceinline__ int64_t chan(int c) const
    {
        const int64_t ch = n0 + (int64_t)RS * c;
        return ch < n ? ch : (CB == 8 ? n0 : n - 1);
    }

    // Stage s into buf. Workgroups start at different stages (rot) and wrap
    // around, so that the workgroups resident on one XCD at a time read all
    // the k offsets of their rows rather than the same one: measured on MI355X,
    // the unstaggered order ran 10-30 % slower on the large layers, by an amount
    // that depended on where the weight happened to be allocated. Wave (ct, kp) loads
    // its 16 code rows of k-part kp: instruction j puts rows 4j..4j+3 at
    // buf + wave * CODE + 1024 j, lane l landing at 16 l, i.e. row r = 4j + l / 16
    // at slot l % 16 holds chunk (slot - r) mod 16 of that row. Activation
    // instruction p puts rows 2p', 2p'+1 of k-part p / (XR / 2) (p' = p mod XR / 2)
    // in the same rotated way, 32 chunks per row. Rows past n or m are clamped
    // to real rows; their results are never stored.
    __device__ __forceinline__ void issue(int64_t s, uint8_t* buf) const
    {
        int64_t sr = s + rot;  // s < S and rot < S
        sr = sr < S ? sr : sr - S;
        const int64_t kb = sr * (KP * 256);
        if constexpr (CB != 4) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 4 * j + (lane >> 4);
                const int chunk = ((lane & 15) - r) & 15;
                const int64_t row = chan(16 * ct + r);
                const uint8_t* src = q + row * k + kb + kp * 256 + chunk * 16;
                __builtin_amdgcn_global_load_lds((const void*)src, FP8W_LDS(buf + wave * C::CODE + j * 1024), 16,
                                                 0, 2 /* non-temporal */);
            }
        } else {
            // 4-byte loads, the same LDS image: instruction r fills row r, lane
            // l the word l % 4 of slot l / 4, which holds chunk (slot - r) mod 16
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int chunk = ((lane >> 2) - r) & 15;
                const int64_t row = chan(16 * ct + r);
                const uint8_t* src = q + row * k + kb + kp * 256 + chunk * 16 + 4 * (lane & 3);
                __builtin_amdgcn_global_load_lds((const void*)src, FP8W_LDS(buf + wave * C::CODE + r * 256), 4, 0,
                                                 2 /* non-temporal */);
            }
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
    }

    // Which k each wave multiplies. Sliced (CT dividing 4, a ring of more than
    // two stages): the 256 k of a k-part are four groups of 64, and wave (ct,
    // kp) takes groups ct, ct + CT, .. of every channel tile of the k-part, so
    // each activation fragment is read from LDS once and serves all CT tiles.
    // At 32 tokens this cuts the LDS reads per stage from 80 to 32 KB; measured
    // on MI355X, [14336 x 4096] went from 14.8 to 13.5 us at 22 tokens and from
    // 15.5 to 14.7 at 32. With two stages it measured slower (18.9 against 20.6
    // us on [4096 x 14336] at 22 tokens, split four ways), so there, as for
    // CT = 3, wave (ct, kp) takes all of k-part kp for its own tile.
    static constexpr bool kSliced = 4 % CT == 0 && NS > 2;
    static constexpr int NACC = kSliced ? CT : 1;  // channel tiles a wave accumulates

    // 16 contiguous codes of row i (two MFMAs' A fragments) and the matching
    // activations of token i (+ 16 mt): lane (i, g) of group j takes chunk
    // 4 j + g (sliced) or 4 g + j; rows sit rotated in LDS as issue() put them.
    __device__ __forceinline__ void mfma_pair(const uint8_t* cb, const u32x4* b0, const u32x4* b1, int c,
                                              f32x4* acc) const
    {
        const int i = lane & 15;
        const u32x4 c16 = *reinterpret_cast<const u32x4*>(cb + 16 * (16 * i + ((c + i) & 15)));
        const u32x2 d0 = A::decode4(c16.x), d1 = A::decode4(c16.y);
        const u32x2 d2 = A::decode4(c16.z), d3 = A::decode4(c16.w);
        const u32x4 a0 = {d0.x, d0.y, d1.x, d1.y};
        const u32x4 a1 = {d2.x, d2.y, d3.x, d3.y};
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            acc[mt] = A::mfma(a0, b0[mt], acc[mt]);
            acc[mt] = A::mfma(a1, b1[mt], acc[mt]);
        }
    }

    __device__ __forceinline__ void x_frag(const uint8_t* xb, int c, u32x4* b0, u32x4* b1) const
    {
        const int i = lane & 15;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int t = (i + 16 * mt) < XR ? (i + 16 * mt) : XR - 1;
            const uint8_t* xr = xb + 16 * (32 * t);
            b0[mt] = *reinterpret_cast<const u32x4*>(xr + 16 * ((2 * c + t) & 31));
            b1[mt] = *reinterpret_cast<const u32x4*>(xr + 16 * ((2 * c + 1 + t) & 31));
        }
    }

    // Block b of the columns outside the ring (the T = k - kr columns before
    // and after it, in that order: the sh before, then kr + sh .. k - 1): 32
    // of them; lane (i, g) takes the eight at 32 b + 8 g, as the A (codes of
    // row i of each tile it holds) and B (token i) operands of one MFMA.
    // Groups at or past T load nothing and stay zero in both operands. (These
    // columns exist only without a k split; q and x point at column sh of the
    // rows, so column c sits at offset c - sh.)
    template <int NT>
    __device__ __forceinline__ void tail_load(int64_t kr, int b, u32x2 (&code)[NT], u32x4 (&xv)[MT]) const
    {
        const int i = lane & 15, g = lane >> 4;
        const int64_t v = 32 * b + 8 * g;
        const int64_t c = (v < sh ? v : kr + v) - sh;
#pragma unroll
        for (int t = 0; t < NT; ++t)
            code[t] = u32x2{0u, 0u};
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            xv[mt] = u32x4{0u, 0u, 0u, 0u};
        if (v < T) {
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const int64_t ch = chan(16 * (NT == 1 ? ct : t) + i);
                code[t] = load_codes8(q + ch * k + c);
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int tok = i + 16 * mt < m ? i + 16 * mt : m - 1;
                xv[mt] = load16(x + (int64_t)tok * k + c);
            }
        }
    }

    template <int NT>
    __device__ __forceinline__ void tail_use(const u32x2 (&code)[NT], const u32x4 (&xv)[MT], f32x4 (*acc)[MT]) const
    {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const u32x2 d0 = A::decode4(code[t].x), d1 = A::decode4(code[t].y);
            const u32x4 a = {d0.x, d0.y, d1.x, d1.y};
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                acc[t][mt] = A::mfma(a, xv[mt], acc[t][mt]);
        }
    }

    __device__ __forceinline__ void compute(const uint8_t* buf, f32x4 (*acc)[MT]) const
    {
        const int g = lane >> 4;
        const uint8_t* xb = buf + C::W * C::CODE + kp * C::XPART;
        u32x4 b0[MT], b1[MT];
        if constexpr (kSliced) {
#pragma unroll
            for (int jj = 0; jj < 4 / CT; ++jj) {
                const int c = 4 * (ct + CT * jj) + g;
                x_frag(xb, c, b0, b1);
#pragma unroll
                for (int t = 0; t < CT; ++t)
                    mfma_pair(buf + (t + CT * kp) * C::CODE, b0, b1, c, acc[t]);
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                x_frag(xb, 4 * g + j, b0, b1);
                mfma_pair(buf + wave * C::CODE, b0, b1, 4 * g + j, acc[0]);
            }
        }
    }
};

// Sum for tile ct of the partial sums in part[w][t][lane], over the waves in
// index order: with NACC == CT (sliced) every wave w contributes part[w][ct];
// with NACC == 1 the waves of tile ct are ct, ct + CT, .. (one per k-part).
template <int NACC, int W, int CT>
__device__ __forceinline__ f32x4 kSlicedSum(f32x4 (*part)[NACC][kWave], int ct, int lane)
{
    if constexpr (NACC == CT && CT > 1) {
        f32x4 sum = part[0][ct][lane];
#pragma unroll
        for (int w = 1; w < W; ++w)
            sum += part[w][ct][lane];
        return sum;
    } else {
        f32x4 sum = part[ct][0][lane];
#pragma unroll
        for (int w = ct + CT; w < W; w += CT)
            sum += part[w][0][lane];
        return sum;
    }
}

// The ring covers kr columns (kr / splits a multiple of KP * 256 * NS) from
// column sh: 0, or for CB == 8 the columns to the first 16-byte boundary of
// the workgroup's rows (0 or 8); k is the row stride. The other k - kr columns
// (CB 8 and 4 only, a multiple of 8 below 512, no split) are further MFMAs on
// operands loaded straight into registers (Pipe::tail_load), 32 columns each,
// dealt to the waves in turn; each wave fetches its first before the ring
// starts. CB == 8: workgroups 2j and 2j + 1 own the even and the odd channels
// of 32 CT.
//
// Arguments: what the ring needs from its first instruction (the operands,
// the sizes, kc = kr / splits and the stages per split S, each under 2^31)
// lie in the first 56 bytes, which the wave finds preloaded in SGPRs (the
// build preloads 14); the output pointers, needed only at the end, follow.
// Measured on MI355X: 0.2-0.3 us per launch against sizes fetched with a
// scalar load (and a 64-bit division by the grid's height) before the ring.
template <typename A, int XR, int CT, int KP, int NS, int CB, bool ANY>
__global__ __launch_bounds__(CT* KP * kWave) void pipe_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ q, const float* __restrict__ scale,
    const uint16_t* __restrict__ bias, int n, int k, int kr, int kc, int m, int S, uint16_t* __restrict__ y,
    float* __restrict__ part_out)
{
    using P = Pipe<A, XR, CT, KP, NS, CB>;
    using C = typename P::C;
    constexpr int MT = C::MT;
    __shared__ __attribute__((aligned(1024))) uint8_t b0[C::STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t b1[C::STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t b2[NS > 2 ? C::STAGE : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t b3[NS > 3 ? C::STAGE : 16];

    // split k: workgroup row blockIdx.y owns k range [y * kc, (y + 1) * kc);
    // ANY rings with a split: S is the stage count of all splits together, and
    // row y owns stages [y S / splits, (y + 1) S / splits) (splits may differ
    // by one stage)
    int Sy = S;
    int64_t k0 = (int64_t)blockIdx.y * kc;
    if constexpr (ANY) {
        if (gridDim.y > 1) {
            const unsigned sp = gridDim.y, y0 = blockIdx.y;
            const int sb = (int)((y0 * (unsigned)S) / sp), se = (int)(((y0 + 1) * (unsigned)S) / sp);
            Sy = se - sb;
            k0 = (int64_t)sb * (KP * 256);
        }
    }
    P p;
    p.x = x + k0;
    p.q = q + k0;
    p.m = m;
    p.n = n;
    p.k = k;
    p.lane = threadIdx.x & (kWave - 1);
    p.wave = threadIdx.x / kWave;
    p.ct = p.wave % CT;
    p.kp = p.wave / CT;
    p.n0 = CB == 8 ? (int64_t)(blockIdx.x >> 1) * (32 * CT) + (blockIdx.x & 1) : (int64_t)blockIdx.x * (16 * CT);
    p.T = k - kr;
    p.sh = 0;
    if constexpr (CB == 8) {
        if (p.n0 >= n)  // the odd workgroup of the last pair when n is short
            return;
        // columns to the first 16-byte boundary of the workgroup's rows
        p.sh = (int64_t)((16 - (reinterpret_cast<uintptr_t>(q + p.n0 * k) & 15)) & 15);
        p.x += p.sh;
        p.q += p.sh;
    }

    constexpr int NACC = P::NACC;
    f32x4 acc[NACC][MT];
#pragma unroll
    for (int t = 0; t < NACC; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            acc[t][mt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // epilogue operands of this lane's four channels, fetched before the ring
    // starts (extra loads ahead of the ring only make its waits stricter)
    float sc[4];
    uint16_t bi[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int64_t ch = p.chan(16 * p.ct + 4 * (p.lane >> 4) + r);
        sc[r] = scale[ch];
        bi[r] = bias_bits(bias, ch);
    }
    // the k tail's blocks this wave multiplies (sliced: all its tiles, blocks
    // wave, wave + W, ..; else its own tile, blocks kp, kp + KP, ..), the first
    // fetched now
    constexpr int NT = P::NACC;
    const int bstep = P::kSliced ? C::W : KP;
    const int tb0 = P::kSliced ? p.wave : p.kp;
    const int nblk = CB != 16 ? (int)((p.T + 31) / 32) : 0;
    u32x2 tcode[NT];
    u32x4 txv[MT];
    if constexpr (CB != 16) {
        if (tb0 < nblk)
            p.tail_load(kr, tb0, tcode, txv);
    }

    p.S = Sy;
    // workgroups are dealt to the eight XCDs in turn: consecutive workgroups of
    // one XCD get consecutive start stages
    p.rot = (int64_t)((blockIdx.x / 8) % (unsigned)Sy);
    // with the sliced compute, the loads pinned ahead of each step's compute
    // measured 0.2-0.4 us faster at 16-22 tokens on [14336 x 4096]; for CT = 3
    // they were 0.2-0.6 us slower
    if constexpr (ANY)  // any S >= NS, not only multiples of NS
        run_ring_any<NS, C::LOADS, P::kSliced>(p, Sy, b0, b1, b2, b3, acc);
    else
        run_ring<NS, C::LOADS, P::kSliced>(p, Sy, b0, b1, b2, b3, acc);
    if constexpr (CB != 16) {
        if (tb0 < nblk) {
            p.tail_use(tcode, txv, acc);
            for (int b = tb0 + bstep; b < nblk; b += 2 * bstep) {  // two blocks' loads in flight at a time
                u32x2 c1[NT], c2[NT];
                u32x4 x1[MT], x2[MT];
                const bool two = b + bstep < nblk;
                p.tail_load(kr, b, c1, x1);
                if (two)
                    p.tail_load(kr, b + bstep, c2, x2);
                p.tail_use(c1, x1, acc);
                if (two)
                    p.tail_use(c2, x2, acc);
            }
        }
    }

    // The waves' partial sums meet in stage buffer 0, one token tile at a
    // time: wave w's sums for tile t at part[w][t]. Wave (ct, 0) adds those of
    // tile ct over the waves in index order and applies the epilogue;
    // D[4g + r][i] is channel 4g + r, token i.
    static_assert(C::STAGE >= C::W * NACC * kWave * 16, "reduction fits in a stage buffer");
    f32x4(*part)[NACC][kWave] = reinterpret_cast<f32x4(*)[NACC][kWave]>(b0);
    const int i = p.lane & 15, g = p.lane >> 4;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        __syncthreads();
#pragma unroll
        for (int t = 0; t < NACC; ++t)
            part[p.wave][t][p.lane] = acc[t][mt];
        __syncthreads();
        const int tok = i + 16 * mt;
        if (p.kp != 0 || tok >= m)
            continue;
        // sliced: every wave holds a share of every tile; else wave (ct, kp) holds tile ct of k-part kp
        f32x4 sum = kSlicedSum<NACC, C::W, CT>(part, p.ct, p.lane);
        const float v[4] = {sum.x, sum.y, sum.z, sum.w};
        if (part_out) {  // split k: fp32 partial sums, reduced by splitk_reduce_kernel
            float* o = part_out + ((int64_t)blockIdx.y * m + tok) * n;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t ch = p.n0 + 16 * p.ct + 4 * g + r;  // a split runs only with CB == 16
                if (ch < n)
                    o[ch] = v[r];
            }
            continue;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t ch = p.n0 + (int64_t)P::RS * (16 * p.ct + 4 * g + r);
            if (ch < n)
                y[(int64_t)tok * n + ch] = epilogue<A>(v[r], sc[r], bi[r]);
        }
    }
}

// Sum of the split-k partial sums in split order, then the epilogue: one
// output per thread. scale == nullptr: unit scale (the partial sums of the
// grouped batch GEMM already hold their group scales).
template <typename A>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part, int splits, int m,
                                                            int64_t n, const float* __restrict__ scale,
                                                            const uint16_t* __restrict__ bias,
                                                            uint16_t* __restrict__ y)
{
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= (int64_t)m * n)
        return;
    const int64_t ch = e % n;
    float sum = part[e];
    for (int s = 1; s < splits; ++s)
        sum += part[(int64_t)s * m * n + e];
    y[e] = epilogue<A>(sum, scale ? scale[ch] : 1.0f, bias_bits(bias, ch));
}

// ---------------------------------------------------------------- dispatch
template <typename A, int SEG, int T, int W, int U, int MT>
hipError_t launch_seg(const void* x, int m, int64_t k, const uint8_t* q, const float* scale, const void* bias,
                      int64_t n, void* y, hipStream_t stream)
{
    constexpr int C = (16 / SEG) * T;  // channels per workgroup
    const dim3 grid((unsigned)((n + C - 1) / C)), block(W * kWave);
    hipLaunchKernelGGL((seg_kernel<A, SEG, T, W, U, MT>), grid, block, 0, stream,
                       static_cast<const uint16_t*>(x), q, scale, static_cast<const uint16_t*>(bias), m, n, k,
                       static_cast<uint16_t*>(y));
    return hipGetLastError();
}

// splits > 1: k is split over `splits` workgroup rows whose fp32 partial sums
// go to part (splits * m * n floats), then a second kernel reduces them.
// kr (default k): the columns the ring covers; the rest is the k tail.
// ANY (always with NS = 3): the ring takes any whole number of stages >= NS.
template <typename A, int XR, int CT, int KP, int NS, int CB = 16, bool ANY = (NS == 3)>
hipError_t launch_pipe(const void* x, int m, int64_t k, const uint8_t* q, const float* scale, const void* bias,
                       int64_t n, void* y, hipStream_t stream, int splits = 1, float* part = nullptr,
                       int64_t kr = -1)
{
    if (kr < 0)
        kr = k;
    // the ring issues only stages that exist when each split's k is a whole,
    // positive number of NS-stage groups (three-stage rings: any whole number
    // of stages, at least three)
    if (splits < 1 || kr <= 0 || kr > k)
        return hipErrorInvalidValue;
    static_assert(ANY || NS != 3, "three-stage rings take any stage count");
    // ANY: whole stages, at least NS in the smallest split (splits may differ by one stage)
    if (ANY ? (kr % ((int64_t)KP * 256) != 0 || kr / ((int64_t)KP * 256) / splits < NS)
            : kr % ((int64_t)splits * KP * 256 * NS) != 0)
        return hipErrorInvalidValue;
    // a tail only without a split, in whole 8-column blocks; rows as wide as the
    // loads; CB == 8: room for a shift of 8 columns before the ring
    if ((kr != k && (splits != 1 || (k - kr) % 8 != 0)) || k % 8 != 0 || (CB == 16 && k % 16 != 0) ||
        (CB == 8 && (splits != 1 || kr > k - 8 || reinterpret_cast<uintptr_t>(q) % 8 != 0)))
        return hipErrorInvalidValue;
    if (n > INT32_MAX || k > INT32_MAX)  // the kernel takes its sizes as 32-bit values
        return hipErrorInvalidValue;
    const unsigned gx = CB == 8 ? (unsigned)(2 * ((n + 32 * CT - 1) / (32 * CT))) : (unsigned)((n + 16 * CT - 1) / (16 * CT));
    const dim3 grid(gx, (unsigned)splits), block(CT * KP * kWave);
    // each split's columns (equal splits; an ANY ring with a split gets the
    // stage count of all splits and divides it itself)
    const int64_t kc = kr / splits;
    const int64_t stages = ANY && splits > 1 ? kr / (KP * 256) : kc / (KP * 256);
    hipLaunchKernelGGL((pipe_kernel<A, XR, CT, KP, NS, CB, ANY>), grid, block, 0, stream,
                       static_cast<const uint16_t*>(x), q, scale, static_cast<const uint16_t*>(bias), (int)n, (int)k,
                       (int)kr, (int)kc, m, (int)stages, static_cast<uint16_t*>(y), splits > 1 ? part : nullptr);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || splits <= 1)
        return e;
    return launch_splitk_reduce(part, splits, m, n, scale, bias, y, std::is_same<A, Bf16>::value ? Act::BF16 : Act::FP16,
                                stream);
}

// Kernel choice per shape, from sweeps on MI355X (k % 256 == 0 here).
// pipe_kernel: a workgroup owns 16 * CT channels, so CT is the largest that
// still gives about one workgroup per CU (224-448 workgroups on the decode and
// sweep layers), KP > 1 adds waves on narrower layers, and NS is the deepest
// ring whose LDS lets every workgroup be resident at once. Every workgroup
// streams all XR activation rows of its k range, so on narrow layers above 16
// tokens the activations outweigh the codes; there k is split over workgroup
// rows instead (four on layers of 4096-8191 channels, two on 8192-channel
// layers), each with 64 channels, and a second kernel reduces the fp32
// partial sums from the caller's workspace. Measured on MI355X this pays only
// above 16 tokens, where it cut [4096 x 14336] at 32 tokens from 28.8 to
// 19.7 us; without workspace these shapes take the single-pass plan.
// Activation rows are fetched in steps of four up to 16 (then 24, 32): 12 rows
// for 9-12 tokens measured 3-6 % faster than 16 on the 4096- and 8192-channel
// layers, where the activations are most of what the ring carries.
// A layer of exactly 256 * 48 = 12288 channels (merged q/k/v) takes three
// channel tiles: 256 workgroups, one per CU, where four tiles leave a quarter of
// the CUs idle (10.9 against 11.7 us at 16 tokens on [12288 x 4096], 14.7
// against 15.3 at 32). seg_kernel covers small batches on narrow layers, where
// it measured faster, and the shapes the ring cannot tile.
// Layers of 16384+ channels with k >= 8192 take eight channel tiles and a
// three-stage ring from 13 tokens on (224 workgroups of eight waves on 28672
// channels, 144 KB of LDS at 32 tokens): half the activation bytes per code
// byte of the four-tile plan. [28672 x 8192] at 16 / 22 / 32 tokens 37.5 /
// 41.1 / 45.8 -> 36.8 / 40.0 / 41.4 us, [28672 x 12288] 57.9 / 62.8 / 69.7 ->
// 54.4 / 59.0 / 60.7; at k = 4096, and below 13 tokens, the ring is too short
// or the activations too few for it to pay (up to 2.7 us slower).
// Splits whose stages are not a multiple of four take three-stage rings (any
// stage count) instead of two: [4096 x 14336] split four ways at 17 / 22 / 32
// tokens 18.2 / 18.4 / 19.1 -> 15.0 / 15.6 / 16.6 us; [4096 x 10240] at 16 /
// 32 tokens 14.1 / 15.4 -> 13.2 / 14.8. On 4096-8191-channel layers with
// k % 7168 == 0 and k % 4096 != 0 (the 14336-wide down projection) that split
// also runs from 12 tokens when the caller gives workspace, ahead of
// narrow_kernel: 14.6 / 16.2 -> 13.9 / 14.3 us at 12 / 16 tokens.
// On 8192-channel layers the k split starts at 12 tokens where k >= 20480:
// [8192 x 28672] at 12 / 14 / 16 tokens 39.7 / 41.3 / 42.4 -> 38.2 / 38.6 /
// 39.0 us; with k = 14336 the two plans are within 0.5 us, with k = 8192 the
// split is 2-3 us slower.
struct SkinnyPlan {
    bool pipe;
    int xr, ct, kp, ns, splits;  // pipe_kernel
    int seg, t, w, u, mt;        // seg_kernel
};

SkinnyPlan plan_skinny(int64_t m, int64_t n, int64_t k, bool allow_split)
{
    SkinnyPlan p{};
    int ct = 0, kp = 1, ns = 4, splits = 1;
    // an odd number of 256-column stages on a 2048-8191-channel layer: no
    // single-pass ring shape divides it; splits of whole stages (uneven by at
    // most one) on three-stage rings, as many as keep the grid near one
    // workgroup per CU ([4096, 11008] at 12 / 16 / 32 tokens 32.2 / 32.8 /
    // 36.8 -> 13.0 / 13.5 / 15.0 us; [5120, 13824] at 2 / 16 / 32 tokens 19.7 /
    // 40.9 / 45.4 -> 15.7 / 17.6 / 19.8; [2048, 5632] at 16 / 32 tokens 17.1 /
    // 19.7 -> 8.7 / 10.1; below 9 tokens seg_kernel stays unless each split
    // has 16+ stages on 4096+ channels: [4096, 11008] split four ways 12.7 us
    // at 2 tokens against 12.4; short rows stay on the single pass)
    const int oct = n >= 4096 ? 4 : 2;
    const int64_t otiles = (n + 16 * oct - 1) / (16 * oct);
    const int64_t osp = 256 / otiles < 2 ? 2 : 256 / otiles > 4 ? 4 : 256 / otiles;
    const bool odd_split = n >= 2048 && n < 8192 && k % 2048 != 0 && k % 256 == 0 && k >= 5120 &&
                           k / 256 / osp >= 3 && (m >= 9 || (n >= 4096 && k / 256 / osp >= 16)) && allow_split;
    if (m >= 2) {
        if (n >= 16384 && m >= 13 && k >= 8192) {
            ct = 8;  // eight tiles, three stages (the stage count need not divide by three)
            ns = 3;
        } else if (n >= 16384) {
            ct = 4;
            ns = 2;
        } else if (n >= 12288) {
            ct = n <= 256 * 48 ? 3 : 4;
        } else if (n >= 8192) {
            if ((m > 16 || (m >= 12 && k >= 20480)) && allow_split && k % (2 * 1024) == 0) {
                ct = 4;
                splits = 2;
            } else if (m <= 16 && k % 2048 == 0) {
                ct = 2;
                kp = 2;
            } else {
                ct = 2;
            }
        } else if ((m > 16 || (m >= 12 && k % 7168 == 0 && k % 4096 != 0)) && n >= 4096 && allow_split &&
                   k % (4 * 512) == 0) {
            ct = 4;
            splits = 4;
        } else if (odd_split) {
            ct = oct;
            splits = (int)osp;
            ns = 3;
        } else if (m > 8) {
            ct = 1;
            kp = 2;
        }
    }
    if (ct != 0) {
        const int64_t kc = k / splits;
        if (ns == 3 && splits == 1 && (kc % 256 != 0 || kc / 256 < 3))
            ct = 4, ns = 2;
        if (ns != 3 && kc % (kp * 256 * ns) != 0)  // a split's stages not a multiple of four: three
            ns = splits > 1 && kp == 1 && kc % 256 == 0 && kc / 256 >= 3 ? 3 : 2;
        if (ns == 3 || kc % (kp * 256 * ns) == 0) {
            p.pipe = true;
            p.xr = m <= 4 ? 4 : m <= 8 ? 8 : m <= 12 ? 12 : m <= 16 ? 16 : m <= 24 ? 24 : 32;
            p.ct = ct;
            p.kp = kp;
            p.ns = ns;
            p.splits = splits;
            return p;
        }
    }
    p.splits = 1;
    if (m <= 4)
        p.seg = 4, p.t = 4, p.w = 4, p.u = 2, p.mt = 1;
    else if (m <= 8 && n >= 8192)
        p.seg = 2, p.t = 4, p.w = 4, p.u = 1, p.mt = 1;
    else if (m <= 8)
        p.seg = 2, p.t = 2, p.w = 8, p.u = 2, p.mt = 1;
    else
        p.seg = 1, p.t = 2, p.w = 4, p.u = 1, p.mt = 2;
    return p;
}

template <typename A, int XR>
hipError_t launch_pipe_xr(const SkinnyPlan& p, const void* x, int m, int64_t k, const uint8_t* q,
                          const float* scale, const void* bias, int64_t n, void* y, float* part,
                          hipStream_t stream)
{
    const int key = p.ct * 100 + p.kp * 10 + p.ns;
    const int sp = p.splits;
    switch (key) {
    case 813:
        if constexpr (XR >= 16)  // the plan takes eight tiles from 13 tokens on
            return launch_pipe<A, XR, 8, 1, 3>(x, m, k, q, scale, bias, n, y, stream, sp, part);
        return hipErrorInvalidValue;
    case 413: return launch_pipe<A, XR, 4, 1, 3>(x, m, k, q, scale, bias, n, y, stream, sp, part);
    case 213:
        if constexpr (XR >= 12)  // splits of 2048-4095-channel layers, from 9 tokens on
            return launch_pipe<A, XR, 2, 1, 3>(x, m, k, q, scale, bias, n, y, stream, sp, part);
        return hipErrorInvalidValue;
    case 412: return launch_pipe<A, XR, 4, 1, 2>(x, m, k, q, scale, bias, n, y, stream, sp, part);
    case 414: return launch_pipe<A, XR, 4, 1, 4>(x, m, k, q, scale, bias, n, y, stream, sp, part);
    case 312: return launch_pipe<A, XR, 3, 1, 2>(x, m, k, q, scale, bias, n, y, stream, sp, part);
    case 314: return launch_pipe<A, XR, 3, 1, 4>(x, m, k, q, scale, bias, n, y, stream, sp, part);
    case 212: return launch_pipe<A, XR, 2, 1, 2>(x, m, k, q, scale, bias, n, y, stream, sp, part);
    case 214: return launch_pipe<A, XR, 2, 1, 4>(x, m, k, q, scale, bias, n, y, stream, sp, part);
    case 122: return launch_pipe<A, XR, 1, 2, 2>(x, m, k, q, scale, bias, n, y, stream, sp, part);
    case 124: return launch_pipe<A, XR, 1, 2, 4>(x, m, k, q, scale, bias, n, y, stream, sp, part);
    case 222:
    case 224:
        if constexpr (XR <= 16) {  // the plan uses two k-parts of 32 channels only up to 16 tokens
            if (key == 222)
                return launch_pipe<A, XR, 2, 2, 2>(x, m, k, q, scale, bias, n, y, stream, sp, part);
            return launch_pipe<A, XR, 2, 2, 4>(x, m, k, q, scale, bias, n, y, stream, sp, part);
        }
        return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
    }
}

template <typename A, int XR, int CB>
hipError_t launch_ring4_xr(const Ring4Plan& p, const void* x, int m, int64_t k, const uint8_t* q,
                           const float* scale, const void* bias, int64_t n, void* y, hipStream_t stream)
{
    const int key = p.ct * 100 + p.kp * 10 + p.ns;
    const int64_t kr = p.kr;
    switch (key) {
    case 412: return launch_pipe<A, XR, 4, 1, 2, CB>(x, m, k, q, scale, bias, n, y, stream, 1, nullptr, kr);
    case 414: return launch_pipe<A, XR, 4, 1, 4, CB>(x, m, k, q, scale, bias, n, y, stream, 1, nullptr, kr);
    case 212: return launch_pipe<A, XR, 2, 1, 2, CB>(x, m, k, q, scale, bias, n, y, stream, 1, nullptr, kr);
    case 214: return launch_pipe<A, XR, 2, 1, 4, CB>(x, m, k, q, scale, bias, n, y, stream, 1, nullptr, kr);
    case 122: return launch_pipe<A, XR, 1, 2, 2, CB>(x, m, k, q, scale, bias, n, y, stream, 1, nullptr, kr);
    case 124:
        if constexpr (XR <= 16)  // 32 rows: 16 activation loads per wave, too many for four stages
            return launch_pipe<A, XR, 1, 2, 4, CB>(x, m, k, q, scale, bias, n, y, stream, 1, nullptr, kr);
        return hipErrorInvalidValue;
    case 222:
    case 224:
        if constexpr (XR <= 16) {
            if (key == 222)
                return launch_pipe<A, XR, 2, 2, 2, CB>(x, m, k, q, scale, bias, n, y, stream, 1, nullptr, kr);
            return launch_pipe<A, XR, 2, 2, 4, CB>(x, m, k, q, scale, bias, n, y, stream, 1, nullptr, kr);
        }
        return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
    }
}

template <typename A, int CB>
hipError_t launch_ring4_cb(const Ring4Plan& p, const void* x, int m, int64_t k, const uint8_t* q,
                           const float* scale, const void* bias, int64_t n, void* y, hipStream_t stream)
{
    switch (p.xr) {
    case 4: return launch_ring4_xr<A, 4, CB>(p, x, m, k, q, scale, bias, n, y, stream);
    case 8: return launch_ring4_xr<A, 8, CB>(p, x, m, k, q, scale, bias, n, y, stream);
    case 16: return launch_ring4_xr<A, 16, CB>(p, x, m, k, q, scale, bias, n, y, stream);
    default: return launch_ring4_xr<A, 32, CB>(p, x, m, k, q, scale, bias, n, y, stream);
    }
}

template <typename A>
hipError_t launch_ring4(const void* x, int64_t m, int64_t k, const uint8_t* q, const float* scale, const void* bias,
                        int64_t n, void* y, hipStream_t stream)
{
    const Ring4Plan p = plan_ring4(m, n, k, q);
    if (!p.ok)
        return hipErrorInvalidValue;
    if (p.cb == 8)
        return launch_ring4_cb<A, 8>(p, x, (int)m, k, q, scale, bias, n, y, stream);
    return launch_ring4_cb<A, 4>(p, x, (int)m, k, q, scale, bias, n, y, stream);
}

template <typename A>
hipError_t launch_typed(const void* x, int64_t m, int64_t k, const uint8_t* q, const float* scale,
                        const void* bias, int64_t n, void* y, float* part, size_t part_bytes, hipStream_t stream)
{
    const int mi = (int)m;
    const size_t need = skinny_workspace_bytes(m, n, k);
    const bool ws_ok = part != nullptr && need > 0 && part_bytes >= need;
    const NarrowPlan np = plan_narrow(m, n, k, ws_ok);
    if (np.ok)
        return launch_narrow(np, x, std::is_same<A, Bf16>::value ? Act::BF16 : Act::FP16, m, k, q, scale, bias, n, y,
                             stream);
    const SkinnyPlan p = plan_skinny(m, n, k, ws_ok);
    if (p.pipe) {
        switch (p.xr) {
        case 4: return launch_pipe_xr<A, 4>(p, x, mi, k, q, scale, bias, n, y, part, stream);
        case 8: return launch_pipe_xr<A, 8>(p, x, mi, k, q, scale, bias, n, y, part, stream);
        case 12: return launch_pipe_xr<A, 12>(p, x, mi, k, q, scale, bias, n, y, part, stream);
        case 16: return launch_pipe_xr<A, 16>(p, x, mi, k, q, scale, bias, n, y, part, stream);
        case 24: return launch_pipe_xr<A, 24>(p, x, mi, k, q, scale, bias, n, y, part, stream);
        default: return launch_pipe_xr<A, 32>(p, x, mi, k, q, scale, bias, n, y, part, stream);
        }
    }
    if (p.seg == 4)
        return launch_seg<A, 4, 4, 4, 2, 1>(x, mi, k, q, scale, bias, n, y, stream);
    if (p.seg == 2 && p.t == 4)
        return launch_seg<A, 2, 4, 4, 1, 1>(x, mi, k, q, scale, bias, n, y, stream);
    if (p.seg == 2)
        return launch_seg<A, 2, 2, 8, 2, 1>(x, mi, k, q, scale, bias, n, y, stream);
    return launch_seg<A, 1, 2, 4, 1, 2>(x, mi, k, q, scale, bias, n, y, stream);
}

}  // namespace

namespace {

// The ring's columns and tile for 1..32 tokens when the ring may cover at most
// `room` columns of each row (k, or k - 8 to leave room for a shift).
Ring4Plan plan_ring4_within(int64_t m, int64_t n, int64_t k, int64_t room)
{
    Ring4Plan r{};
    if (m < 1 || m > 32 || n < 1 || k < 512 || k % 8 != 0)
        return r;
    int64_t kr = room - room % 256;
    if ((kr / 256) % 2 != 0)
        kr -= 256;
    if (kr <= 0)
        return r;
    SkinnyPlan p = plan_skinny(m < 2 ? 2 : m, n, kr, false);
    if (p.pipe && p.ct == 8) {  // this ring keeps the widest layers' four tiles and two stages
        p.ct = 4;
        p.ns = 2;
    }
    // where plan_skinny picks seg_kernel (under 8192 channels, up to 8 tokens):
    // one tile and two k-parts, so that a 4096-channel layer still has 256
    // workgroups (two tiles left half the CUs idle: [4096, 14344] at one
    // token 36.7 us); where it picks three tiles, two
    int ct = p.pipe ? (p.ct != 3 ? p.ct : 2) : 1, kp = p.pipe ? (p.ct != 3 ? p.kp : 1) : 2;
    if (ct == 2 && kp == 2 && m > 16)
        kp = 1;
    const int xr = m <= 4 ? 4 : m <= 8 ? 8 : m <= 16 ? 16 : 32;
    // four stages unless plan_skinny runs two (the widest layers, for two
    // workgroups per CU), the k-parts do not divide them, or the wait counter
    // cannot hold them (one tile, two k-parts, 32 rows: 16 activation loads
    // per wave)
    const bool deep = !(p.pipe && p.ns == 2);
    const bool four = deep && !(ct == 1 && kp == 2 && xr == 32);
    int ns = four && kr % ((int64_t)kp * 256 * 4) == 0 ? 4 : kr % ((int64_t)kp * 256 * 2) == 0 ? 2 : 0;
    if (ns == 0) {  // one k-part: kr / 256 is even, so two stages always fit
        if (ct == 1)
            ct = 2;
        kp = 1;
        ns = deep && kr % 1024 == 0 ? 4 : 2;
    }
    r.ok = true;
    r.xr = xr;
    r.ct = ct;
    r.kp = kp;
    r.ns = ns;
    r.kr = kr;
    return r;
}

}  // namespace

// The skinny path for codes the 16-byte kernels cannot load (k a multiple of
// 8 but not of 256, or q not 16-byte aligned; k >= 512), 1..32 tokens:
// pipe_kernel over kr columns, an even number of 256-column stages; the other
// columns (at most 512, a multiple of 8) are further MFMAs on register
// operands. cb = 8 (rows 16-byte aligned, or k % 16 == 8 with q 8-byte
// aligned, so that neighbouring rows alternate between two alignments):
// 16-byte loads from the first 16-byte boundary of each workgroup's rows (with
// k % 16 == 8 the ring leaves room for a shift of 8 columns). Measured on
// MI355X against 4-byte loads: [28672, 8200] at 4 / 8 / 32 tokens 46.4 / 47.2
// / 54.4 us against 50.3 / 49.3 / 79.2, [4096, 14344] at 4 tokens 13.3 against
// 22.3, [12288, 2056] at 24 tokens 15.3 against 21.2. Otherwise (cb = 4)
// 4-byte loads: with every row 8 bytes off a 16-byte boundary the shift would
// leave up to 512 columns to the register operands ([4096, 4096] with q 8
// bytes off at 8 tokens: 15.7 us shifted, 9.7 with 4-byte loads). 4-byte loads
// measured as fast as 16-byte ones on aligned rows (9.98 against 9.84 us over
// [14336, 4096]) but touch three 128-byte lines per 256-byte segment of a row
// that is not 16-byte aligned instead of two. Channel tiles and k-parts follow
// plan_skinny for kr without a split (with the exceptions in
// plan_ring4_within). Activation rows 4, 8, 16 or 32. One token with 8-byte
// aligned codes takes the GEMV instead (fp8w_linear's dispatch).
Ring4Plan plan_ring4(int64_t m, int64_t n, int64_t k, const uint8_t* q)
{
    const uintptr_t a = reinterpret_cast<uintptr_t>(q);
    if (a % 8 == 0 && (k % 16 == 8 || a % 16 == 0)) {
        Ring4Plan r = plan_ring4_within(m, n, k, k % 16 == 8 ? k - 8 : k);
        r.cb = 8;
        if (r.ok)
            return r;
    }
    Ring4Plan r = plan_ring4_within(m, n, k, k);
    r.cb = 4;
    return r;
}

size_t skinny_workspace_bytes(int64_t m, int64_t n, int64_t k)
{
    if (m < 1 || m > 32 || n < 1 || k < 256 || k % 256 != 0 || plan_narrow(m, n, k, true).ok)
        return 0;
    const SkinnyPlan p = plan_skinny(m, n, k, true);
    return p.pipe && p.splits > 1 ? (size_t)p.splits * (size_t)m * (size_t)n * sizeof(float) : 0;
}

hipError_t launch_splitk_reduce(const float* part, int splits, int64_t m, int64_t n, const float* scale,
                                const void* bias, void* y, Act act, hipStream_t stream)
{
    const int64_t total = m * n;
    if (total == 0)
        return hipSuccess;
    if ((total + 255) / 256 > INT32_MAX || m > INT32_MAX)
        return hipErrorInvalidValue;
    const dim3 grid((unsigned)((total + 255) / 256)), block(256);
    const uint16_t* b = static_cast<const uint16_t*>(bias);
    uint16_t* yy = static_cast<uint16_t*>(y);
    if (act == Act::BF16)
        hipLaunchKernelGGL((splitk_reduce_kernel<Bf16>), grid, block, 0, stream, part, splits, (int)m, n, scale, b, yy);
    else if (act == Act::FP16)
        hipLaunchKernelGGL((splitk_reduce_kernel<F16>), grid, block, 0, stream, part, splits, (int)m, n, scale, b, yy);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_skinny(const void* x, Act act, int64_t m, int64_t k, const uint8_t* q, const float* scale,
                         const void* bias, int64_t n, void* y, void* ws, size_t ws_bytes, hipStream_t stream)
{
    if (n == 0 || m == 0)
        return hipSuccess;
    if (m > 32)
        return hipErrorInvalidValue;
    if (k % 256 != 0 || reinterpret_cast<uintptr_t>(q) % 16 != 0) {  // codes the 16-byte kernels cannot load
        if (reinterpret_cast<uintptr_t>(q) % 4 != 0 || reinterpret_cast<uintptr_t>(x) % 16 != 0)
            return hipErrorInvalidValue;
        if (act == Act::BF16)
            return launch_ring4<Bf16>(x, m, k, q, scale, bias, n, y, stream);
        if (act == Act::FP16)
            return launch_ring4<F16>(x, m, k, q, scale, bias, n, y, stream);
        return hipErrorInvalidValue;
    }
    float* part = static_cast<float*>(ws);
    if (act == Act::BF16)
        return launch_typed<Bf16>(x, m, k, q, scale, bias, n, y, part, ws_bytes, stream);
    if (act == Act::FP16)
        return launch_typed<F16>(x, m, k, q, scale, bias, n, y, part, ws_bytes, stream);
    return hipErrorInvalidValue;
}

const char* skinny_kernel_name(int64_t m, int64_t n, int64_t k, bool with_workspace, bool ring4, const uint8_t* q)
{
    thread_local char name[96];
    if (ring4) {
        const Ring4Plan p = plan_ring4(m, n, k, q);
        if (!p.ok)
            return nullptr;
        snprintf(name, sizeof name, "pipe_kernel<XR=%d,CT=%d,KP=%d,NS=%d,CB=%d>", p.xr, p.ct, p.kp, p.ns, p.cb);
        return name;
    }
    const NarrowPlan np = plan_narrow(m, n, k, with_workspace);
    if (np.ok)
        return narrow_kernel_name(np);
    const SkinnyPlan p = plan_skinny(m, n, k, with_workspace);
    if (p.pipe && p.splits > 1)
        snprintf(name, sizeof name, "pipe_kernel<XR=%d,CT=%d,KP=%d,NS=%d>x%d+splitk_reduce_kernel", p.xr, p.ct,
                 p.kp, p.ns, p.splits);
    else if (p.pipe)
        snprintf(name, sizeof name, "pipe_kernel<XR=%d,CT=%d,KP=%d,NS=%d>", p.xr, p.ct, p.kp, p.ns);
    else
        snprintf(name, sizeof name, "seg_kernel<SEG=%d,T=%d,W=%d,U=%d,MT=%d>", p.seg, p.t, p.w, p.u, p.mt);
    return name;
}

}  // namespace fp8w
