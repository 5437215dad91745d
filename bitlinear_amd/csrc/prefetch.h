// prefetch.h -- pulling weight lines toward the CUs ahead of the loads that use them.
//
// At one token (or a few) a BitLinear step is a short weight stream whose time
// is mostly load latency. A wave's vector loads complete in issue order, so
// loading a later step's rows into registers early would hold every wait in
// between. Instead a line is touched with one dword loaded straight into a
// scratch area of LDS (global_load_lds_dword): no register is held, and the
// compiler, which does not see the load, inserts no wait for it. The line
// lands in L2 of the issuing CU's XCD and in the memory-side cache. Inside one
// launch a later load of the same XCD hits L2; across a launch boundary only
// the memory-side cache keeps it (the L2 traffic counters of the next launch
// do not drop). The instruction still counts in the wave's vmcnt, so the
// wave's next wait for a vector load also waits for it, and a wave must wait
// for it (wait_loads) before it ends while the LDS target is still its own.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bl {

// One dword of the line at p into LDS at lds_off + 4 lane. m0 holds the LDS
// address for the instruction and is restored afterwards.
__device__ __forceinline__ void prefetch_line(const void* p, uint32_t lds_off)
{
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\t"
                 "s_mov_b32 m0, %2\n\t"
                 "global_load_lds_dword %1, off\n\t"
                 "s_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "v"(p), "s"(lds_off));
}

// Waits until every vector load of the wave, prefetches included, has landed.
__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Weights for a launch to pull toward the CUs on behalf of the launch that
// follows it: up to two byte spans (4-byte aligned, sizes multiples of 4) of
// which workgroup b of the next launch reads bytes [b chunk, (b + 1) chunk) of
// each (chunk a multiple of 4). Workgroup i of a launch runs on XCD i mod 8
// (the round-robin dispatch of an MI355X, measured at every launch); chunks
// are handed out so that a line is prefetched on the XCD that will read it,
// which costs nothing, although the gain measured comes from the memory-side
// cache (see above).
struct Prefetch {
    const uint8_t* p[2];
    uint32_t bytes[2];
    uint32_t chunk;
};

// Prefetch workgroup pb of nb (nb a multiple of 8), launch index g: it takes
// the chunks b = g mod 8 + 8 (pb / 8 + (nb / 8) i) -- those read on its XCD --
// with nt threads over their 128-byte lines, then waits for its loads.
__device__ __forceinline__ void prefetch_chunks(const Prefetch& pf, int g, int pb, int nb, int nt, uint32_t lds_off)
{
    const uint32_t chunk = pf.chunk;
    const uint32_t top = pf.bytes[0] > pf.bytes[1] ? pf.bytes[0] : pf.bytes[1];
    const uint32_t lpc = (chunk + 127) / 128;  // lines per chunk and span
    for (uint32_t b = (uint32_t)(g & 7) + 8u * (uint32_t)(pb >> 3); (uint64_t)b * chunk < top; b += (uint32_t)nb) {
        for (uint32_t u = threadIdx.x; u < 2 * lpc; u += (uint32_t)nt) {
            const int sp = u < lpc ? 0 : 1;
            const uint64_t off = (uint64_t)b * chunk + 128ull * (u - (uint32_t)sp * lpc);
            if (pf.p[sp] && off < (uint64_t)pf.bytes[sp] && off < (uint64_t)(b + 1) * chunk)
                prefetch_line(pf.p[sp] + off, lds_off);
        }
    }
    wait_loads();
}

}  // namespace bl
