// Direct-to-LDS load ring shared by the streaming MFMA kernels (gfx950).
//
// A workgroup keeps NS stage buffers in LDS. Stage s is loaded with
// global_load_lds_dwordx4 (each lane's 16 bytes land at the instruction's LDS
// base + 16 * lane; no registers hold data in flight), NS - 1 stages are in
// flight while the matrix cores consume the oldest one.
//
// How the waits stay exact: every stage issues the same number of load
// instructions per wave (LOADS), all unconditionally, and the stage buffers
// are distinct __shared__ arrays addressed only through statically unrolled
// steps. The compiler's own wait-count pass can then tell the buffers apart
// and inserts no drain of its own inside the loop, and the explicit
// s_waitcnt vmcnt(LOADS * (NS - 2)) before each step's barrier is exactly
// "this stage has landed" (loads complete in order). The barrier is a bare
// s_barrier: __syncthreads() would add release/acquire fences that drain
// every outstanding load, the prefetched stages included.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "common.hpp"

#define FP8W_LDS(p) ((__attribute__((address_space(3))) void*)(p))

namespace fp8w {

// s_waitcnt vmcnt(N) lgkmcnt(0): at most N of this wave's vector-memory loads
// (the direct-to-LDS ones included) still outstanding, all LDS reads returned.
template <int N>
__device__ __forceinline__ void wait_loads_at_most()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// Workgroup barrier without the release/acquire fences of __syncthreads();
// LDS visibility comes from the explicit wait before it, and the empty asm
// keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void stage_barrier()
{
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Runs stages 0 .. S-1 through the ring (S % NS == 0, S >= NS). P provides
// issue(s, buf) (exactly LOADS load instructions per wave) and compute(buf, acc).
// The last group of NS stages issues only its first load, then drains.
// PIN keeps the compiler from moving any of a step's compute ahead of that
// step's loads, so the next stage is requested as soon as the barrier opens.
template <int NS, int LOADS, bool PIN = false, typename P, typename Acc>
__device__ __forceinline__ void run_ring(const P& p, int64_t S, uint8_t* b0, uint8_t* b1, uint8_t* b2, uint8_t* b3,
                                         Acc* acc)
{
    static_assert(NS >= 2 && NS <= 4, "stages");
    static_assert(LOADS * (NS - 2) < 64, "vmcnt range");
    auto step = [&](int64_t s, const uint8_t* cur, uint8_t* nxt) {
        wait_loads_at_most<LOADS*(NS - 2)>();
        stage_barrier();
        p.issue(s + NS - 1, nxt);
        if constexpr (PIN)
            __builtin_amdgcn_sched_barrier(0);
        p.compute(cur, acc);
    };
    p.issue(0, b0);
    if constexpr (NS > 2)
        p.issue(1, b1);
    if constexpr (NS > 3)
        p.issue(2, b2);
    int64_t s = 0;
    for (; s < S - NS; s += NS) {
        if constexpr (NS == 2) {
            step(s, b0, b1);
            step(s + 1, b1, b0);
        } else if constexpr (NS == 3) {
            step(s, b0, b2);
            step(s + 1, b1, b0);
            step(s + 2, b2, b1);
        } else {
            step(s, b0, b3);
            step(s + 1, b1, b0);
            step(s + 2, b2, b1);
            step(s + 3, b3, b2);
        }
    }
    if constexpr (NS == 2) {
        step(s, b0, b1);
        wait_loads_at_most<0>();
        stage_barrier();
        p.compute(b1, acc);
    } else if constexpr (NS == 3) {
        step(s, b0, b2);
        wait_loads_at_most<LOADS>();
        stage_barrier();
        p.compute(b1, acc);
        wait_loads_at_most<0>();
        stage_barrier();
        p.compute(b2, acc);
    } else {
        step(s, b0, b3);
        wait_loads_at_most<2 * LOADS>();
        stage_barrier();
        p.compute(b1, acc);
        wait_loads_at_most<LOADS>();
        stage_barrier();
        p.compute(b2, acc);
        wait_loads_at_most<0>();
        stage_barrier();
        p.compute(b3, acc);
    }
}

// f(std::integral_constant<int, I>) for I = B .. E-1, unrolled at compile time.
template <int B, int E, typename F>
__device__ __forceinline__ void ring_for(F&& f)
{
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        ring_for<B + 1, E>(f);
    }
}

// Stage buffer I of four, chosen at compile time (no array of pointers, so
// every LDS access keeps its own __shared__ object).
template <int I>
__device__ __forceinline__ uint8_t* ring_buf(uint8_t* b0, uint8_t* b1, uint8_t* b2, uint8_t* b3)
{
    if constexpr (I == 0)
        return b0;
    else if constexpr (I == 1)
        return b1;
    else if constexpr (I == 2)
        return b2;
    else
        return b3;
}

// The last R steps of run_ring_any (NS - 1 <= R <= 2 NS - 2), from stage s0
// (a multiple of NS) on, all known at compile time: step u issues stage
// s0 + u + NS - 1 while it exists and waits with the stages issued after its
// own, min(NS - 2, R - 1 - u), still allowed in flight (loads complete in
// order). Straight-line code, so the compiler's wait-count pass still tells
// the stage buffers apart; a run-time test around each issue made it drain
// every outstanding load before each step's compute.
template <int NS, int LOADS, bool PIN, int R, typename P, typename Acc>
__device__ __forceinline__ void ring_tail(const P& p, int64_t s0, uint8_t* b0, uint8_t* b1, uint8_t* b2, uint8_t* b3,
                                          Acc* acc)
{
    ring_for<0, R>([&](auto uc) {
        constexpr int u = decltype(uc)::value;
        constexpr int after = R - 1 - u < NS - 2 ? R - 1 - u : NS - 2;
        wait_loads_at_most<LOADS * after>();
        stage_barrier();
        if constexpr (u + NS - 1 < R) {
            p.issue(s0 + u + NS - 1, ring_buf<(u + NS - 1) % NS>(b0, b1, b2, b3));
            if constexpr (PIN)
                __builtin_amdgcn_sched_barrier(0);
        }
        p.compute(ring_buf<u % NS>(b0, b1, b2, b3), acc);
    });
}

// run_ring for any number of stages S >= NS (S need not be a multiple of NS).
// Step s waits for stage s, opens the barrier, issues stage s + NS - 1 into
// the buffer stage s - 1 used (while that stage exists) and computes stage s
// from buffer s mod NS. Whole groups of NS steps run as in run_ring while at
// least 2 NS - 1 steps remain; the last R steps (NS - 1 <= R <= 2 NS - 2) run
// as one of NS straight-line tails, chosen by R.
template <int NS, int LOADS, bool PIN = false, typename P, typename Acc>
__device__ __forceinline__ void run_ring_any(const P& p, int64_t S, uint8_t* b0, uint8_t* b1, uint8_t* b2,
                                             uint8_t* b3, Acc* acc)
{
    static_assert(NS >= 2 && NS <= 4, "stages");
    static_assert(LOADS * (NS - 2) < 64, "vmcnt range");
    p.issue(0, b0);
    if constexpr (NS > 2)
        p.issue(1, b1);
    if constexpr (NS > 3)
        p.issue(2, b2);
    int64_t s0 = 0;
    for (; s0 + 2 * NS - 2 < S; s0 += NS) {
        ring_for<0, NS>([&](auto uc) {
            constexpr int u = decltype(uc)::value;
            wait_loads_at_most<LOADS*(NS - 2)>();
            stage_barrier();
            p.issue(s0 + u + NS - 1, ring_buf<(u + NS - 1) % NS>(b0, b1, b2, b3));
            if constexpr (PIN)
                __builtin_amdgcn_sched_barrier(0);
            p.compute(ring_buf<u>(b0, b1, b2, b3), acc);
        });
    }
    const int64_t rest = S - s0;
    ring_for<NS - 1, 2 * NS - 1>([&](auto rc) {
        constexpr int R = decltype(rc)::value;
        if (rest == R)
            ring_tail<NS, LOADS, PIN, R>(p, s0, b0, b1, b2, b3, acc);
    });
}

// Tile (tn, tm) of workgroup (blockIdx.x, blockIdx.y). Workgroups are dealt
// to the 8 XCDs in turn by linear id L: XCD x = L % 8 is given the contiguous
// range of tile ids that starts at x * (T / 8) + min(x, T % 8), walked in the
// order that fills groups of GM tile rows (GM token tiles x all channel
// tiles) column by column, so the tiles one XCD holds at a time form a
// GM x (32 / GM) block. A bijection of [0, T).
template <int GM>
__device__ __forceinline__ void xcd_tile_of(int64_t& tn, int64_t& tm)
{
    const int64_t TN = gridDim.x, TM = gridDim.y, T = TN * TM;
    const int64_t L = blockIdx.x + TN * blockIdx.y;
    const int64_t xcd = L % 8, loc = L / 8, q = T / 8, r = T % 8;
    const int64_t id = xcd * q + (xcd < r ? xcd : r) + loc;
    const int64_t grp = id / (GM * TN), first = grp * GM;
    const int64_t gs = TM - first < GM ? TM - first : GM;
    const int64_t w = id - grp * GM * TN;
    tm = first + w % gs;
    tn = w / gs;
}

}  // namespace fp8w
