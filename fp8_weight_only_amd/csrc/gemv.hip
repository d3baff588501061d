// M = 1 fp8-weight GEMV: y[n] = scale[n] * sum_k x[k] * value(q[n,k]) + bias[n].
//
// "FP8 weight-only (precision: fp8_weights)", section "Dequantise in
// registers": 128-bit streaming loads of 16 codes, exact hardware conversion of
// each code to fp32, fp32 FMA, a cross-lane reduction and the scale in the
// epilogue ("The contract": fp32 accumulation, scale and bias in fp32, one
// rounding). Batch-1 decode is bound by the bytes of the weight stream ("B04 -
// Precision & Quantization", "Worked example: batch-1 decode is a bandwidth
// problem"), so the layout is chosen for the memory system, not the ALUs.
//
// Layout (gfx950): a workgroup of NT threads owns R consecutive output rows and
// splits k among all its threads: in each pass thread t reads the 16-code chunk
// t of every one of its rows, so a quarter-wave reads 256 contiguous bytes of
// one row and each load instruction touches the fewest cache lines. The
// activation chunk a thread needs is the same for its R rows and is read once
// per pass. U passes are issued back to back before any is consumed (one
// group); the decode-sized instance keeps the next group in flight while it
// consumes the current one (double buffering in registers); a predicated tail
// pass handles k that is not a multiple of 16*NT*U. Per-thread
// sums are reduced with cross-lane shuffles, then (workgroups of several
// waves) across the waves through LDS in a fixed order (deterministic).
//
// Many small workgroups (R rows each) keep every CU streaming until the end
// of the matrix; measured on MI355X, this shape runs within a few percent of a
// plain streaming-read kernel of the same bytes for matrices of 58 MB and up.
//
// Rows that are not all 16-byte aligned (k % 8 == 0, q 8-byte aligned):
// - k % 16 == 8: consecutive rows alternate between two alignments mod 16,
//   and rows two apart always share one (2k % 16 == 0). gemv_shift_kernel
//   gives each workgroup R rows of one parity and starts its 16-code chunks at
//   the first 16-byte boundary of those rows (a shift of 0 or 8 columns, the
//   same for the activation chunks); the columns before the shift and after
//   the last whole chunk (fewer than 16 each) are one lane's work each.
// - k % 16 == 0 with q 8 bytes off a 16-byte boundary: every row is off by 8;
//   gemv_kernel runs on 8-code chunks (8-byte loads), which measured faster
//   here than the shifted 16-code chunks.
#include "common.hpp"
#include "kernels.hpp"

namespace fp8w {
namespace {

// A chunk is CH consecutive codes of a row (one load: 16 bytes, or 8 where
// rows are only 8-byte aligned) and the CH activations they multiply.
template <int CH>
struct Chunk {
    static_assert(CH == 16 || CH == 8, "chunk width");
    static constexpr int CW = CH / 4;  // code words
    static constexpr int XV = CH / 8;  // 16-byte activation loads
    typedef uint32_t Words[CW];
    __device__ __forceinline__ static void load_codes(const uint8_t* p, uint32_t* w)
    {
        if constexpr (CH == 16) {
            const u32x4 v = load_stream16(p);
            w[0] = v.x, w[1] = v.y, w[2] = v.z, w[3] = v.w;
        } else {
            const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
            w[0] = v.x, w[1] = v.y;
        }
    }
};

template <typename A, int R, int CH>
__device__ __forceinline__ void accum_chunk(const uint32_t (*code)[CH / 4], const u32x4* xv, float* acc)
{
    float xf[CH];
#pragma unroll
    for (int v = 0; v < CH / 8; ++v) {
        const uint32_t xw[4] = {xv[v].x, xv[v].y, xv[v].z, xv[v].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            xf[8 * v + 2 * e + 0] = A::lo_f32(xw[e]);
            xf[8 * v + 2 * e + 1] = A::hi_f32(xw[e]);
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
        for (int d = 0; d < CH / 4; ++d) {
            float w0, w1, w2, w3;
            decode4_f32(code[r][d], w0, w1, w2, w3);
            acc[r] = __builtin_fmaf(xf[4 * d + 0], w0, acc[r]);
            acc[r] = __builtin_fmaf(xf[4 * d + 1], w1, acc[r]);
            acc[r] = __builtin_fmaf(xf[4 * d + 2], w2, acc[r]);
            acc[r] = __builtin_fmaf(xf[4 * d + 3], w3, acc[r]);
        }
    }
}

// U passes of a thread's chunks for R rows, and the activation chunks they
// share. load() issues every load of the group back to back (the scheduling
// barrier keeps the compiler from trading loads in flight for registers).
template <int R, int U, int CH>
struct Group {
    uint32_t code[U][R][CH / 4];
    u32x4 xv[U][CH / 8];
    __device__ __forceinline__ void load(const uint8_t* const* qr, const uint16_t* xp, int64_t c0, int nt)
    {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t off = (c0 + (int64_t)nt * u) * CH;
#pragma unroll
            for (int r = 0; r < R; ++r)
                Chunk<CH>::load_codes(qr[r] + off, code[u][r]);
#pragma unroll
            for (int v = 0; v < CH / 8; ++v)
                xv[u][v] = load16(xp + off + 8 * v);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    template <typename A>
    __device__ __forceinline__ void use(float* acc) const
    {
#pragma unroll
        for (int u = 0; u < U; ++u)
            accum_chunk<A, R, CH>(code[u], xv[u], acc);
    }
};

// The same group of U passes for the shifted kernel, whose last group may be
// partial: a chunk index past `last` loads chunk `last` (in bounds) and its
// codes and activations are then zeroed, so that it adds exactly 0.
template <int R, int U>
struct ClampedGroup {
    uint32_t code[U][R][4];
    u32x4 xv[U][2];
    // c0: this lane's chunk index in the group's first pass
    __device__ __forceinline__ void load(const uint8_t* const* qr, const uint16_t* xp, int64_t c0, int nt,
                                         int64_t last)
    {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t c = c0 + (int64_t)nt * u;
            const int64_t off = (c < last ? c : last) * 16;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const u32x4 v = load_stream16(qr[r] + off);
                code[u][r][0] = v.x, code[u][r][1] = v.y, code[u][r][2] = v.z, code[u][r][3] = v.w;
            }
            xv[u][0] = load16(xp + off);
            xv[u][1] = load16(xp + off + 8);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (c0 + (int64_t)nt * u > last) {
#pragma unroll
                for (int r = 0; r < R; ++r)
                    code[u][r][0] = code[u][r][1] = code[u][r][2] = code[u][r][3] = 0u;
                xv[u][0] = xv[u][1] = u32x4{0u, 0u, 0u, 0u};
            }
        }
    }
    template <typename A>
    __device__ __forceinline__ void use(float* acc) const
    {
#pragma unroll
        for (int u = 0; u < U; ++u)
            accum_chunk<A, R, 16>(code[u], xv[u], acc);
    }
};

// Groups 0..G-1, loaded by load(group, g) and consumed in order by
// group.use(acc). With DB the next group's loads are issued before the current
// group is consumed, so each wave keeps a continuous stream of requests in
// flight instead of draining it at every group.
template <typename A, bool DB, typename Grp, typename Load>
__device__ __forceinline__ void stream_groups(int64_t G, Grp& ga, Grp& gb, Load load, float* acc)
{
    if constexpr (DB) {
        if (G <= 0)
            return;
        int64_t g = 0;
        load(ga, 0);
        for (; g + 2 < G; g += 2) {
            load(gb, g + 1);
            ga.template use<A>(acc);
            load(ga, g + 2);
            gb.template use<A>(acc);
        }
        if (g + 1 < G) {
            load(gb, g + 1);
            ga.template use<A>(acc);
            gb.template use<A>(acc);
        } else {
            ga.template use<A>(acc);
        }
    } else {
        for (int64_t g = 0; g < G; ++g) {
            load(ga, g);
            ga.template use<A>(acc);
        }
    }
}

// Per-thread sums of R rows to the R outputs: one wave reduces in registers
// and lane r stores output r; several waves meet in LDS in wave order. row(r)
// is output r's channel; rows at or past n are not stored.
template <typename A, int R, int NT, typename Row>
__device__ __forceinline__ void finish_rows(const float* acc, float (*red)[R], float sc, uint16_t bi, Row row,
                                            int64_t n, uint16_t* __restrict__ y)
{
    constexpr int NW = NT / kWave;
    const int t = threadIdx.x;
    if constexpr (NW == 1) {
        // after the butterfly every lane holds every row's sum (no LDS, no barrier)
        float tot = 0.0f;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float s = wave_sum(acc[r]);
            if (t == r)
                tot = s;
        }
        if (t < R && row(t) < n)
            y[row(t)] = epilogue<A>(tot, sc, bi);
        return;
    }
    const int lane = t & (kWave - 1), wave = t >> 6;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const float s = wave_sum(acc[r]);
        if (lane == 0)
            red[wave][r] = s;
    }
    __syncthreads();
    if (t < R && row(t) < n) {
        float s = red[0][t];
#pragma unroll
        for (int w = 1; w < NW; ++w)
            s += red[w][t];
        y[row(t)] = epilogue<A>(s, sc, bi);
    }
}

template <typename A, int R, int U, int NT, bool DB, int CH>
__global__ __launch_bounds__(NT) void gemv_kernel(const uint16_t* __restrict__ x, const uint8_t* __restrict__ q,
                                                  const float* __restrict__ scale,
                                                  const uint16_t* __restrict__ bias, uint16_t* __restrict__ y,
                                                  int64_t n, int64_t k)
{
    __shared__ float red[NT / kWave][R];
    const int t = threadIdx.x;
    const int64_t row0 = (int64_t)blockIdx.x * R;
    const int64_t nch = k / CH;  // chunks per row

    const uint8_t* qr[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
        qr[r] = q + (row0 + r < n ? row0 + r : n - 1) * k + (int64_t)t * CH;
    const uint16_t* xp = x + (int64_t)t * CH;

    // epilogue operands of this workgroup's rows, fetched up front (threads
    // t < R use them; the others read a valid row and discard it)
    const int64_t er = row0 + (t % R) < n ? row0 + (t % R) : n - 1;
    const float sc = scale[er];
    const uint16_t bi = bias_bits(bias, er);

    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
        acc[r] = 0.0f;

    // whole groups of U passes, then predicated tail passes: only threads whose chunk exists
    constexpr int64_t GS = (int64_t)NT * U;
    Group<R, U, CH> ga, gb;
    stream_groups<A, DB>(
        nch / GS, ga, gb, [&](Group<R, U, CH>& grp, int64_t g) { grp.load(qr, xp, g * GS, NT); }, acc);
    for (int64_t c0 = nch / GS * GS; c0 < nch; c0 += NT) {
        if (c0 + t < nch) {
            const int64_t off = c0 * CH;
            uint32_t code[R][CH / 4];
            u32x4 xv[CH / 8];
#pragma unroll
            for (int r = 0; r < R; ++r)
                Chunk<CH>::load_codes(qr[r] + off, code[r]);
#pragma unroll
            for (int v = 0; v < CH / 8; ++v)
                xv[v] = load16(xp + off + 8 * v);
            accum_chunk<A, R, CH>(code, xv, acc);
        }
    }
    finish_rows<A, R, NT>(acc, red, sc, bi, [&](int r) { return row0 + r; }, n, y);
}

// Rows only 8-byte aligned with k % 16 == 8 (see the top of this file).
// Workgroups 2j and 2j + 1 take rows 2Rj .. 2Rj + 2R - 1, the even ones and
// the odd ones: R rows two apart, which share their alignment mod 16.
template <typename A, int R, int U, int NT, bool DB>
__global__ __launch_bounds__(NT) void gemv_shift_kernel(const uint16_t* __restrict__ x,
                                                        const uint8_t* __restrict__ q,
                                                        const float* __restrict__ scale,
                                                        const uint16_t* __restrict__ bias,
                                                        uint16_t* __restrict__ y, int64_t n, int64_t k)
{
    constexpr int CH = 16;
    __shared__ float red[NT / kWave][R];
    const int t = threadIdx.x;
    const int64_t base = (int64_t)(blockIdx.x >> 1) * 2 * R + (blockIdx.x & 1);
    if (base >= n)
        return;
    int64_t row[R];  // rows past n: row `base`, read and discarded
#pragma unroll
    for (int r = 0; r < R; ++r)
        row[r] = base + 2 * r < n ? base + 2 * r : base;
    // columns to the first 16-byte boundary of these rows: 0 or 8
    const int s = (int)((16 - (reinterpret_cast<uintptr_t>(q + base * k) & 15)) & 15);
    const int64_t nch = (k - s) / CH;  // whole chunks from column s
    const uint8_t* qr[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
        qr[r] = q + row[r] * k + s;
    const uint16_t* xp = x + s;

    const int64_t er = row[t % R];
    const float sc = scale[er];
    const uint16_t bi = bias_bits(bias, er);
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
        acc[r] = 0.0f;

    // groups of U passes, the last one possibly partial
    constexpr int64_t GS = (int64_t)NT * U;
    ClampedGroup<R, U> ga, gb;
    stream_groups<A, DB>(
        (nch + GS - 1) / GS, ga, gb,
        [&](ClampedGroup<R, U>& grp, int64_t g) { grp.load(qr, xp, g * GS + t, NT, nch - 1); }, acc);

    // columns before s and after the last whole chunk: one lane per column
    const int64_t tail0 = s + CH * nch;
    const int64_t c = t < s ? t : tail0 + (t - s);
    if (t < s || c < k) {
        const float xf = A::to_f32(x[c]);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float w0, w1, w2, w3;
            decode4_f32((uint32_t)q[row[r] * k + c], w0, w1, w2, w3);
            acc[r] = __builtin_fmaf(xf, w0, acc[r]);
        }
    }
    finish_rows<A, R, NT>(acc, red, sc, bi, [&](int r) { return base + 2 * (int64_t)r; }, n, y);
}

template <typename A, int R, int U, int NT, bool DB, int CH = 16>
hipError_t launch_cfg(const void* x, int64_t k, const uint8_t* q, const float* scale, const void* bias, int64_t n,
                      void* y, hipStream_t stream)
{
    const dim3 grid((unsigned)((n + R - 1) / R)), block(NT);
    hipLaunchKernelGGL((gemv_kernel<A, R, U, NT, DB, CH>), grid, block, 0, stream, static_cast<const uint16_t*>(x),
                       q, scale, static_cast<const uint16_t*>(bias), static_cast<uint16_t*>(y), n, k);
    return hipGetLastError();
}

// Tile choice, from sweeps on MI355X (kernel durations, weights rotated
// through 1 GiB). Weights under 96 MB: one-wave workgroups of two rows,
// double-buffered groups of two passes; four-row, 128-thread workgroups with
// single-buffered two-pass groups above. On the long rows of the
// [4096, 14336] down projection the double-buffered one-wave tile took 11.1-11.5
// us against 12.3 for the single-buffered 128-thread one (a plain read of the
// same bytes: 10.1-10.3); on [4096, 4096] and [14336, 4096] the two were
// within 0.3 us of each other. Double buffering did not help the large
// weights' four-row tile.
constexpr int64_t kLargeWeight = (int64_t)96 << 20;

// Groups of one pass (each wave two passes ahead instead of its whole share at
// once) on long rows of 4096-8191-channel layers: [4096, 14336] 11.10 -> 10.73
// us, [5120, 13824] 14.50 -> 13.97, [4096, 8192] 7.42 -> 7.24, [4096, 6144]
// 6.03 -> 5.85; not on [2048, 8192] (+0.5 us), [1024, 16384] (+1.5), [8192,
// 10240] (+0.15) or k % 512 != 0 ([4096, 11008]: +0.6). In the decode step
// the down projection's second kernel binary cost no measurable time beside
// the other layers' (the GEMV family's mean launch 9.07 -> 8.82 us).
bool one_pass_groups(int64_t n, int64_t k)
{
    return n >= 4096 && n < 8192 && k >= 6144 && k % 512 == 0;
}

template <typename A, int R, int U, int NT, bool DB>
hipError_t launch_shift(const void* x, int64_t k, const uint8_t* q, const float* scale, const void* bias, int64_t n,
                        void* y, hipStream_t stream)
{
    const dim3 grid((unsigned)(2 * ((n + 2 * R - 1) / (2 * R)))), block(NT);
    hipLaunchKernelGGL((gemv_shift_kernel<A, R, U, NT, DB>), grid, block, 0, stream,
                       static_cast<const uint16_t*>(x), q, scale, static_cast<const uint16_t*>(bias),
                       static_cast<uint16_t*>(y), n, k);
    return hipGetLastError();
}

// Which chunking the rows allow (x is 16-byte aligned, k % 8 == 0 and q
// 8-byte aligned on every path here).
enum class Rows { ALIGNED, ALTERNATE, OFF8 };

Rows rows_of(int64_t k, const uint8_t* q)
{
    if (k % 16 != 0)
        return Rows::ALTERNATE;  // rows 2 apart share an alignment, neighbours differ by 8
    return reinterpret_cast<uintptr_t>(q) % 16 == 0 ? Rows::ALIGNED : Rows::OFF8;
}

template <typename A>
hipError_t launch_typed(const void* x, int64_t k, const uint8_t* q, const float* scale, const void* bias,
                        int64_t n, void* y, hipStream_t stream)
{
    const bool large = n * k >= kLargeWeight;
    switch (rows_of(k, q)) {
    case Rows::ALTERNATE:  // [28672, 8200]: 43.6 us on 8-code chunks, 39.7 shifted; [4096, 14344]: 12.7 -> 12.1
        return large ? launch_shift<A, 4, 2, 128, false>(x, k, q, scale, bias, n, y, stream)
                     : launch_shift<A, 2, 2, 64, true>(x, k, q, scale, bias, n, y, stream);
    case Rows::OFF8:  // [4096, 4096] with q 8 bytes off: 5.3 us on 8-code chunks, 5.8 shifted
        return large ? launch_cfg<A, 4, 2, 128, false, 8>(x, k, q, scale, bias, n, y, stream)
                     : launch_cfg<A, 2, 2, 64, true, 8>(x, k, q, scale, bias, n, y, stream);
    default:
        if (large)
            return launch_cfg<A, 4, 2, 128, false>(x, k, q, scale, bias, n, y, stream);
        return one_pass_groups(n, k) ? launch_cfg<A, 2, 1, 64, true>(x, k, q, scale, bias, n, y, stream)
                                     : launch_cfg<A, 2, 2, 64, true>(x, k, q, scale, bias, n, y, stream);
    }
}

}  // namespace

const char* gemv_kernel_name(int64_t n, int64_t k, const uint8_t* q)
{
    const bool large = n * k >= kLargeWeight;
    switch (rows_of(k, q)) {
    case Rows::ALTERNATE:
        return large ? "gemv_shift_kernel<R=4,U=2,NT=128>" : "gemv_shift_kernel<R=2,U=2,NT=64,DB>";
    case Rows::OFF8:
        return large ? "gemv_kernel<R=4,U=2,NT=128,CH=8>" : "gemv_kernel<R=2,U=2,NT=64,DB,CH=8>";
    default:
        return large                     ? "gemv_kernel<R=4,U=2,NT=128>"
               : one_pass_groups(n, k) ? "gemv_kernel<R=2,U=1,NT=64,DB>"
                                       : "gemv_kernel<R=2,U=2,NT=64,DB>";
    }
}

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
