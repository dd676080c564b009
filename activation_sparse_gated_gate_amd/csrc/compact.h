// Ordered compaction of flag rows into ascending index lists (the optional
// active-list outputs of both regimes).
#pragma once

#include "device_common.h"

namespace sffn {

// Ordered compaction of one row of flags, for a block of 256 threads: calls
// emit(pos, i) for the channels i < F whose flag is set, pos = 0, 1, ... in
// ascending channel order, and returns the count to every thread. Chunks of
// 2048 channels, 8 consecutive ones per thread (coalesced reads); a block
// scan of the per-thread counts places them. on8(i0, f) sets f[e] for channel
// i0 + e (false from F on). scratch holds 5 ints. Contains barriers.
template <typename On8, typename Emit>
__device__ __forceinline__ int emit_ordered_fn(int F, On8 on8, Emit emit, int *scratch)
{
    int base = 0;
    for (int c0 = 0; c0 < F; c0 += 2048) {
        const int i0 = c0 + 8 * (int)threadIdx.x;
        bool f[8];
        on8(i0, f);
        int local = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) local += f[e];
        const int incl = block_incl_scan(local, scratch);
        int pos = base + incl - local;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (f[e]) emit(pos++, i0 + e);
        if (threadIdx.x == blockDim.x - 1) scratch[4] = incl;
        __syncthreads();
        base += scratch[4];
        __syncthreads();
    }
    return base;
}

// The same, writing the channels to out[0 .. count) (out may be null).
template <typename On8>
__device__ __forceinline__ int emit_ordered(int F, On8 on8, int32_t *out, int *scratch)
{
    return emit_ordered_fn(
        F, on8,
        [&](int pos, int i) {
            if (out) out[pos] = i;
        },
        scratch);
}

}  // namespace sffn
