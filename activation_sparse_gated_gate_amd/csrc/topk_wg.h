// Top-K boundary of one token by a 256-thread workgroup (wg_topk_boundary):
// the select that the decode up kernel runs in its select workgroups and the
// batched select kernel runs once per token.
#pragma once

#include "device_common.h"

namespace sffn {

// ---------------------------------------------------------------------------
// Top-K boundary of one token's keys s[0 .. F) by a workgroup of 256 threads:
// {f2key of the K-th largest key, the last channel kept among the keys equal
// to it}, the pair topk_on applies (1 <= K <= F).
//
// Pass 1 counts the keys into kKeyBins equal value bins over
// [kKeyLo, kKeyLo + 8) (SiLU keys are >= -0.2785; keys past either end go to
// the end bins, a NaN to bin 0). The bin is non-decreasing in the key, so
// every key of a higher bin ranks at least as high as every key of a lower
// one (equal keys share a bin) and the K-th largest lies in the bin b* where
// the count from the top reaches K; need of b*'s keys are kept. Pass 2
// gathers b*'s keys (up to kCandMax) in LDS and ranks each by (f2key
// descending, channel ascending): the one of rank need - 1 is the boundary.
// A fuller bin (ties, or keys far outside the range) goes through an MSD
// radix select on f2key restricted to b*, 8 bits per pass, then a block scan
// of the keys equal to the K-th gives the cutoff.
//
// The passes are written without branches per key: the four wavefronts of
// the workgroup share one scalar unit, and an exec-mask branch per key (a
// bounds test, a NaN test) also serializes the LDS reads behind it. So the
// positions past F hold -inf keys: they count in bin 0 below every channel,
// rank after every channel there (same or larger key, lower index), and the
// boundary, at rank need - 1 < the channels in b*, is never one of them.
// ---------------------------------------------------------------------------
constexpr int kKeyBins = 2048, kCandMax = 512;

// Max (MAX) or min over the 64 lanes, the result in every lane: within each
// row of 16 lanes by DPP moves (pairs, quads, half-row and row mirrors), then
// two lane shuffles across the rows. Every lane must be active.
template <bool MAX>
__device__ __forceinline__ float wave_minmax(float v)
{
    auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : fminf(a, b); };
#define SFFN_DPP_MV(x, ctrl) __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), ctrl, 0xf, 0xf, false))
    v = op(v, SFFN_DPP_MV(v, 0xb1));   // quad_perm [1,0,3,2]
    v = op(v, SFFN_DPP_MV(v, 0x4e));   // quad_perm [2,3,0,1]
    v = op(v, SFFN_DPP_MV(v, 0x141));  // row_half_mirror
    v = op(v, SFFN_DPP_MV(v, 0x140));  // row_mirror
#undef SFFN_DPP_MV
    v = op(v, __shfl_xor(v, 16, 64));
    return op(v, __shfl_xor(v, 32, 64));
}
constexpr float kKeyLo = -0.3f, kKeyScale = kKeyBins / 8.0f;

__device__ __forceinline__ int key_bin(float v)
{
    // fmaxf takes the number when the other operand is NaN; the clamp and the
    // truncation keep the order of (v - kKeyLo) * kKeyScale
    return (int)fminf(fmaxf((v - kKeyLo) * kKeyScale, 0.f), (float)(kKeyBins - 1));
}

struct __align__(16) TopkLds {
    int hist[kKeyBins];  // value bins, then 256 radix digits
    int hist64[64];      // the sample's coarse bins (32 value bins each)
    uint64_t cand[kCandMax];  // b*'s keys: f2key << 32 | ~channel (larger: earlier in the Top-K order)
    int cand_rank[64];
    int sh[6];  // b*, keys of it kept, keys in it, gathered; then the result
    int scan_scratch[4];
};

// Keys of one token kept in LDS by a select workgroup, for d_ff up to
// kTopkLdsKeys; larger layers stream them from global memory in each pass.
constexpr int kTopkLdsKeys = 24 * 256;

// The key of the positions past F.
static __device__ const float g_key_pad = -INFINITY;

// Keys j = tid + 256 u, u < U, of s[0 .. F) into kl[j], loaded straight
// into LDS (no registers; -inf past F). The caller waits (wait_vm_lgkm<0>)
// and syncs before reading kl.
template <int U>
__device__ __forceinline__ void topk_stage_keys(const float *__restrict__ s, int F, float *__restrict__ kl)
{
    const int tid = threadIdx.x, wave = tid >> 6;
#pragma unroll
    for (int u = 0; u < U; ++u)
        __builtin_amdgcn_global_load_lds((gmem_t *)(u * 256 + tid < F ? s + u * 256 + tid : &g_key_pad),
                                         (lmem_t *)(kl + u * 256 + wave * 64), 4, 0, 0);
}

// kl: the keys staged by topk_stage_keys<U> and a barrier since (U > 0), or
// null (U == 0: streamed from s). eslot, cslot: if not null, thread 0
// publishes there, tagged with epoch, a prefetch estimate (a coarse bin from
// a sample; 64: none) before the count, and the boundary bin b* as soon as
// it is known.
template <int U>
__device__ __forceinline__ int2 wg_topk_boundary(const float *__restrict__ s, int F, int K, TopkLds &L,
                                                 const float *__restrict__ kl, uint64_t *eslot, uint64_t *cslot,
                                                 uint32_t epoch)
{
    constexpr int V = U > 0 ? U : 16;  // keys per thread and round
    const int tid = threadIdx.x;
    int *hist = L.hist, *sh = L.sh;
    // fn(u, j, v) over this thread's positions j = tid + 256 u, the keys
    // past F being -inf; T positions in all
    const int T = U > 0 ? U * 256 : (F + 256 * V - 1) / (256 * V) * (256 * V);
    auto for_keys = [&](auto &&fn) {
        if constexpr (U > 0) {
            static_assert(U % 8 == 0, "keys in rounds of 8 per thread");
#pragma unroll 1
            for (int u0 = 0; u0 < U; u0 += 8) {  // rounds of 8 LDS reads keep the registers few
                float o[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) o[e] = kl[(u0 + e) * 256 + tid];
#pragma unroll
                for (int e = 0; e < 8; ++e) fn(u0 + e, (u0 + e) * 256 + tid, o[e]);
            }
        } else {
            for (int j0 = 0; j0 < F; j0 += 256 * V) {
                float o[V];
#pragma unroll
                for (int u = 0; u < V; ++u) o[u] = s[min(j0 + u * 256 + tid, F - 1)];
#pragma unroll
                for (int u = 0; u < V; ++u) fn(u, j0 + u * 256 + tid, j0 + u * 256 + tid < F ? o[u] : -INFINITY);
            }
        }
    };
    if (eslot) {
        // a prefetch estimate first: the coarse bin (32 value bins) where the
        // count from the top of every 8th position, times 8, passes 1.25 K
        int cb = 64;  // none: nothing to prefetch (keys not in LDS)
        if constexpr (U > 0) {
            static_assert(U % 8 == 0, "whole sample rounds");
            if (tid < 64) L.hist64[tid] = 0;
            __syncthreads();
#pragma unroll
            for (int v = 0; v < U / 8; ++v) atomicAdd(&L.hist64[key_bin(kl[8 * (v * 256 + tid)]) >> 5], 1);
            __syncthreads();
            if (tid < 64) {
                const int c = L.hist64[63 - tid];  // lane l: coarse bin 63 - l, from the top
                const int ks = min(U * 32, (K + 7) / 8 + (K + 7) / 32 + 2);
                const uint64_t hit = __ballot(wave_incl_scan(c) >= ks);
                cb = hit ? 63 - (__ffsll((long long)hit) - 1) : 0;
            }
        }
        if (tid == 0)
            __hip_atomic_store(eslot, ((uint64_t)epoch << 32) | (uint32_t)cb, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    reinterpret_cast<int4 *>(hist)[2 * tid] = make_int4(0, 0, 0, 0);
    reinterpret_cast<int4 *>(hist)[2 * tid + 1] = make_int4(0, 0, 0, 0);
    __syncthreads();
    // keys in LDS: the bins of this thread's keys stay in registers, two per
    // word, for the gather after b* (no second pass over the keys)
    uint32_t kb2[U > 0 ? U / 2 : 1];
    if constexpr (U > 0) {
#pragma unroll
        for (int u0 = 0; u0 < U; u0 += 8) {
            float o[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = kl[(u0 + e) * 256 + tid];
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                const int b0 = key_bin(o[e]), b1 = key_bin(o[e + 1]);
                atomicAdd(&hist[b0], 1);
                atomicAdd(&hist[b1], 1);
                kb2[(u0 + e) >> 1] = (uint32_t)b0 | (uint32_t)b1 << 16;
            }
        }
    } else {
        kb2[0] = 0;
        for_keys([&](int, int, float v) { atomicAdd(&hist[key_bin(v)], 1); });
    }
    __syncthreads();
    {
        // thread tid owns bins 8 tid .. 8 tid + 7
        const int4 h0 = reinterpret_cast<const int4 *>(hist)[2 * tid];
        const int4 h1 = reinterpret_cast<const int4 *>(hist)[2 * tid + 1];
        const int c[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
        int local = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) local += c[e];
        int run = T - block_incl_scan(local, L.scan_scratch);  // keys in the bins above this thread's
        if (run < K && K <= run + local) {
#pragma unroll
            for (int e = 7; e >= 0; --e) {
                if (run < K && K <= run + c[e]) {
                    sh[0] = 8 * tid + e;
                    sh[1] = K - run;
                    sh[2] = c[e];
                    sh[3] = 0;
                }
                run += c[e];
            }
        }
    }
    __syncthreads();
    const int bs = sh[0], cnt = sh[2];
    int need = sh[1];
    if (cslot && tid == 0)
        __hip_atomic_store(cslot, ((uint64_t)epoch << 32) | (uint32_t)bs, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (cnt <= kCandMax) {
        // gather b*'s keys: match bits in a register, one slot claim per
        // thread that has any, then the writes
        if constexpr (U > 0) {
            static_assert(U <= 32, "one match bit per key");
            uint32_t mb = 0;
#pragma unroll
            for (int u = 0; u < U; ++u) mb |= (uint32_t)((int)((kb2[u >> 1] >> (16 * (u & 1))) & 0xffffu) == bs) << u;
            if (mb) {
                int slot = atomicAdd(&sh[3], __popc(mb));  // < cnt: the same keys as the count
                for (uint32_t m = mb; m; m &= m - 1) {
                    const int j = (__ffs(m) - 1) * 256 + tid;
                    if (slot < kCandMax) L.cand[slot] = (uint64_t)f2key(kl[j]) << 32 | (uint32_t)~j;
                    ++slot;
                }
            }
        } else {
            for_keys([&](int, int j, float v) {  // the same positions as the count, -inf ones included
                if (key_bin(v) == bs) {
                    const int slot = atomicAdd(&sh[3], 1);
                    if (slot < kCandMax) L.cand[slot] = (uint64_t)f2key(v) << 32 | (uint32_t)~j;
                }
            });
        }
        if (tid < 64) L.cand_rank[tid] = 0;
        __syncthreads();
        // rank of each candidate = candidates with a larger composite (the
        // channels are distinct, so the composites are); up to 64 candidates:
        // wavefront w counts over its quarter of them
        if (cnt <= 64) {
            const int c = tid & 63, w = tid >> 6;
            if (c < cnt) {
                const uint64_t me = L.cand[c];
                int rank = 0;
                for (int m = w * 16; m < min(cnt, w * 16 + 16); ++m) rank += L.cand[m] > me;
                if (rank) atomicAdd(&L.cand_rank[c], rank);
            }
            __syncthreads();
            if (tid < cnt && L.cand_rank[tid] == need - 1) {
                const uint64_t me = L.cand[tid];
                sh[4] = (int)(uint32_t)(me >> 32);
                sh[5] = (int)~(uint32_t)me;
            }
        } else {
            for (int c = tid; c < cnt; c += 256) {
                const uint64_t me = L.cand[c];
                int rank = 0;
                for (int m = 0; m < cnt; ++m) rank += L.cand[m] > me;
                if (rank == need - 1) {
                    sh[4] = (int)(uint32_t)(me >> 32);
                    sh[5] = (int)~(uint32_t)me;
                }
            }
        }
        __syncthreads();
        const int2 r = make_int2(sh[4], sh[5]);
        __syncthreads();  // sh and the candidates are reused by the next select
        return r;
    }
    // ---- a full bin: radix select on f2key within b* ----
    uint32_t prefix = 0, pmask = 0;
#pragma unroll 1
    for (int p = 0; p < 4; ++p) {
        const int shift = 24 - 8 * p;
        hist[tid] = 0;
        __syncthreads();
        for (int j = tid; j < F; j += 256) {
            const float v = s[j];
            const uint32_t key = f2key(v);
            if (key_bin(v) == bs && (key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
        }
        __syncthreads();
        const int c = hist[255 - tid];  // thread tid owns digit 255 - tid: the scan runs from the top
        const int incl = block_incl_scan(c, L.scan_scratch);
        if (incl - c < need && need <= incl) {
            sh[0] = 255 - tid;
            sh[1] = need - (incl - c);
        }
        __syncthreads();
        prefix |= (uint32_t)sh[0] << shift;
        pmask |= 0xffu << shift;
        need = sh[1];
        __syncthreads();  // hist and sh are rewritten by the next pass
    }
    // the first `need` keys equal to the K-th, in channel order: contiguous
    // segments per thread make "equal keys before mine" an exclusive scan
    const int seg = (F + 255) / 256;
    const int i0 = min(F, tid * seg), i1 = min(F, i0 + seg);
    int eq = 0;
    for (int i = i0; i < i1; ++i) eq += f2key(s[i]) == prefix;
    const int before = block_incl_scan(eq, L.scan_scratch) - eq;
    if (before < need && need <= before + eq) {
        int left = need - before, cut = i0;
        for (int i = i0; i < i1 && left > 0; ++i)
            if (f2key(s[i]) == prefix) {
                cut = i;
                --left;
            }
        sh[4] = (int)prefix;
        sh[5] = cut;
    }
    __syncthreads();
    const int2 r = make_int2(sh[4], sh[5]);
    __syncthreads();
    return r;
}

// ---------------------------------------------------------------------------
// Top-p boundary of one token's keys by a workgroup of 256 threads: the
// first channel, in the Top-K order (key descending, channel ascending), at
// which the prefix of fixed-point masses (topp_mass against the token's
// largest key) reaches T = topp_target(p, Z), Z the total mass; returned as
// the pair topk_on applies. That channel is unique, so this is the result of
// select_mass exactly.
//
// The passes follow wg_topk_boundary with a 64-bit mass per value bin in
// place of the count: the largest key first; a prefetch estimate from every
// 8th key (the coarse bin where the sample's mass from the top reaches the
// target of min(1, 1.25 p)); the bin b* where the mass from the top reaches
// T (published), need = T minus the mass above it; b*'s keys (up to
// kToppCand) ranked by the mass ahead of each in the Top-K order, the
// boundary being the one whose mass ahead is below need and reaches it with
// its own. A fuller bin goes through an MSD radix select on f2key restricted
// to b* with a mass per digit, and the ties at the boundary key are taken in
// channel order: ceil(need left / their mass) of them.
// ---------------------------------------------------------------------------
constexpr int kToppCand = 256;

struct __align__(16) ToppLds {
    unsigned long long mass[kKeyBins];  // value bins, then 256 radix digits
    unsigned long long hist64m[64];     // the sample's coarse bins
    unsigned long long cand[kToppCand];  // f2key << 32 | ~channel
    unsigned long long cand_w[kToppCand];
    unsigned long long cand_ahead[64];
    unsigned long long scan64[4];
    unsigned long long shm[2];  // need at b*; need within the radix digit
    float red[4];
    int sh[6];  // b*, -, -, gathered; then the result
    int scan_scratch[4];
};

// Inclusive prefix sum of a 64-bit value over the 256 threads; *total gets
// the sum of all (every thread). Contains a barrier.
__device__ __forceinline__ unsigned long long block_incl_scan_u64(unsigned long long v, ToppLds &L,
                                                                  unsigned long long *total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    v = wave_incl_scan_u64(v);
    if (lane == 63) L.scan64[wave] = v;
    __syncthreads();
    unsigned long long add = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) add += w < wave ? L.scan64[w] : 0ull;
    *total = L.scan64[0] + L.scan64[1] + L.scan64[2] + L.scan64[3];
    return v + add;
}

template <int U>
__device__ __forceinline__ int2 wg_topp_boundary(const float *__restrict__ s, int F, float p, ToppLds &L,
                                                 const float *__restrict__ kl, uint64_t *eslot, uint64_t *cslot,
                                                 uint32_t epoch)
{
    constexpr int V = U > 0 ? U : 16;  // keys per thread and round
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    unsigned long long *mass = L.mass;
    int *sh = L.sh;
    // fn(u, j, v) over this thread's positions j = tid + 256 u, the keys past
    // F being -inf (mass 0)
    auto for_keys = [&](auto &&fn) {
        if constexpr (U > 0) {
            static_assert(U % 8 == 0, "keys in rounds of 8 per thread");
#pragma unroll 1
            for (int u0 = 0; u0 < U; u0 += 8) {
                float o[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) o[e] = kl[(u0 + e) * 256 + tid];
#pragma unroll
                for (int e = 0; e < 8; ++e) fn(u0 + e, (u0 + e) * 256 + tid, o[e]);
            }
        } else {
            for (int j0 = 0; j0 < F; j0 += 256 * V) {
                float o[V];
#pragma unroll
                for (int u = 0; u < V; ++u) o[u] = s[min(j0 + u * 256 + tid, F - 1)];
#pragma unroll
                for (int u = 0; u < V; ++u) fn(u, j0 + u * 256 + tid, j0 + u * 256 + tid < F ? o[u] : -INFINITY);
            }
        }
    };

    // ---- the largest key ----
    float mx = -INFINITY;
    for_keys([&](int, int, float v) { mx = fmaxf(mx, v); });
    mx = wave_minmax<true>(mx);
    if (lane == 0) L.red[wave] = mx;
#pragma unroll
    for (int e = 0; e < 8; ++e) mass[8 * tid + e] = 0ull;
    if (tid < 64) L.hist64m[tid] = 0ull;
    __syncthreads();
    mx = fmaxf(fmaxf(L.red[0], L.red[1]), fmaxf(L.red[2], L.red[3]));

    if (eslot) {
        // the prefetch estimate: a sample of every 8th position
        int cb = 64;  // none: nothing to prefetch (keys not in LDS)
        if constexpr (U > 0) {
#pragma unroll
            for (int v = 0; v < U / 8; ++v) {
                const float key = kl[8 * (v * 256 + tid)];
                atomicAdd(&L.hist64m[key_bin(key) >> 5], topp_mass(key, mx));
            }
            __syncthreads();
            if (tid < 64) {
                const unsigned long long incl = wave_incl_scan_u64(L.hist64m[63 - tid]);  // from the top
                const unsigned long long ts = topp_target(fminf(1.f, 1.25f * p), __shfl(incl, 63, 64));
                const uint64_t hit = __ballot(incl >= ts);
                cb = hit ? 63 - (__ffsll((long long)hit) - 1) : 0;
            }
        }
        if (tid == 0)
            __hip_atomic_store(eslot, ((uint64_t)epoch << 32) | (uint32_t)cb, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // ---- mass per value bin; the bin b* where the mass from the top reaches T ----
    // (keys in LDS: their bins stay in registers, two per word, for the gather)
    uint32_t kb2[U > 0 ? U / 2 : 1];
    if constexpr (U > 0) {
#pragma unroll
        for (int u0 = 0; u0 < U; u0 += 8) {
            float o[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = kl[(u0 + e) * 256 + tid];
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                const int b0 = key_bin(o[e]), b1 = key_bin(o[e + 1]);
                atomicAdd(&mass[b0], topp_mass(o[e], mx));
                atomicAdd(&mass[b1], topp_mass(o[e + 1], mx));
                kb2[(u0 + e) >> 1] = (uint32_t)b0 | (uint32_t)b1 << 16;
            }
        }
    } else {
        kb2[0] = 0;
        for_keys([&](int, int, float v) { atomicAdd(&mass[key_bin(v)], topp_mass(v, mx)); });
    }
    __syncthreads();
    {
        // thread tid owns bins 8 tid .. 8 tid + 7
        unsigned long long c[8], local = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            c[e] = mass[8 * tid + e];
            local += c[e];
        }
        unsigned long long Z = 0;
        const unsigned long long incl = block_incl_scan_u64(local, L, &Z);
        const unsigned long long Tm = topp_target(p, Z);
        unsigned long long run = Z - incl;  // mass in the bins above this thread's
        if (run < Tm && Tm <= run + local) {
#pragma unroll
            for (int e = 7; e >= 0; --e) {
                if (run < Tm && Tm <= run + c[e]) {
                    sh[0] = 8 * tid + e;
                    sh[3] = 0;
                    L.shm[0] = Tm - run;
                }
                run += c[e];
            }
        }
    }
    __syncthreads();
    const int bs = sh[0];
    unsigned long long need = L.shm[0];
    if (cslot && tid == 0)
        __hip_atomic_store(cslot, ((uint64_t)epoch << 32) | (uint32_t)bs, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    // ---- b*'s keys with their masses ----
    if constexpr (U > 0) {
        static_assert(U <= 32, "one match bit per key");
        uint32_t mb = 0;
#pragma unroll
        for (int u = 0; u < U; ++u) mb |= (uint32_t)((int)((kb2[u >> 1] >> (16 * (u & 1))) & 0xffffu) == bs) << u;
        if (mb) {
            int slot = atomicAdd(&sh[3], __popc(mb));
            for (uint32_t m = mb; m; m &= m - 1) {
                const int j = (__ffs(m) - 1) * 256 + tid;
                if (slot < kToppCand) {
                    const float v = kl[j];
                    L.cand[slot] = (unsigned long long)f2key(v) << 32 | (uint32_t)~j;
                    L.cand_w[slot] = topp_mass(v, mx);
                }
                ++slot;
            }
        }
    } else {
        for_keys([&](int, int j, float v) {
            if (key_bin(v) == bs) {
                const int slot = atomicAdd(&sh[3], 1);
                if (slot < kToppCand) {
                    L.cand[slot] = (unsigned long long)f2key(v) << 32 | (uint32_t)~j;
                    L.cand_w[slot] = topp_mass(v, mx);
                }
            }
        });
    }
    if (tid < 64) L.cand_ahead[tid] = 0ull;
    __syncthreads();
    const int cnt = sh[3];
    if (cnt <= kToppCand) {
        if (cnt <= 64) {
            // wavefront w sums, for each candidate, the masses of its quarter
            // of the candidates ahead of it
            const int c = tid & 63, w = tid >> 6;
            if (c < cnt) {
                const unsigned long long me = L.cand[c];
                unsigned long long ahead = 0;
                for (int m = w * 16; m < min(cnt, w * 16 + 16); ++m)
                    if (L.cand[m] > me) ahead += L.cand_w[m];
                if (ahead) atomicAdd(&L.cand_ahead[c], ahead);
            }
            __syncthreads();
            if (tid < cnt) {
                const unsigned long long a = L.cand_ahead[tid];
                if (a < need && need <= a + L.cand_w[tid]) {
                    const unsigned long long me = L.cand[tid];
                    sh[4] = (int)(uint32_t)(me >> 32);
                    sh[5] = (int)~(uint32_t)me;
                }
            }
        } else {
            for (int c = tid; c < cnt; c += 256) {
                const unsigned long long me = L.cand[c];
                unsigned long long a = 0;
                for (int m = 0; m < cnt; ++m)
                    if (L.cand[m] > me) a += L.cand_w[m];
                if (a < need && need <= a + L.cand_w[c]) {
                    sh[4] = (int)(uint32_t)(me >> 32);
                    sh[5] = (int)~(uint32_t)me;
                }
            }
        }
        __syncthreads();
        const int2 r = make_int2(sh[4], sh[5]);
        __syncthreads();  // sh and the candidates are reused by the next select
        return r;
    }
    // ---- a full bin: radix select on f2key within b*, a mass per digit ----
    uint32_t prefix = 0, pmask = 0;
#pragma unroll 1
    for (int ps = 0; ps < 4; ++ps) {
        const int shift = 24 - 8 * ps;
        mass[tid] = 0ull;
        __syncthreads();
        for (int j = tid; j < F; j += 256) {
            const float v = U > 0 ? kl[j] : s[j];
            const uint32_t key = f2key(v);
            if (key_bin(v) == bs && (key & pmask) == prefix) atomicAdd(&mass[(key >> shift) & 255u], topp_mass(v, mx));
        }
        __syncthreads();
        const unsigned long long cm = mass[255 - tid];  // thread tid owns digit 255 - tid: from the top
        unsigned long long tot = 0;
        const unsigned long long incl = block_incl_scan_u64(cm, L, &tot);
        if (incl - cm < need && need <= incl) {
            sh[0] = 255 - tid;
            L.shm[1] = need - (incl - cm);
        }
        __syncthreads();
        prefix |= (uint32_t)sh[0] << shift;
        pmask |= 0xffu << shift;
        need = L.shm[1];
        __syncthreads();  // mass, sh and shm are rewritten by the next pass
    }
    // the keys equal to the boundary key that the prefix needs: the first
    // ceil(need / their mass) of them in channel order
    const unsigned long long u = topp_mass(key2f(prefix), mx);
    const unsigned long long want = u > 0 ? (need + u - 1) / u : 1ull;
    const int seg = (F + 255) / 256;
    const int i0 = min(F, tid * seg), i1 = min(F, i0 + seg);
    int eq = 0;
    for (int i = i0; i < i1; ++i) eq += f2key(U > 0 ? kl[i] : s[i]) == prefix;
    const int eq_incl = block_incl_scan(eq, L.scan_scratch), before = eq_incl - eq;
    if (tid == 255) sh[2] = eq_incl;
    __syncthreads();
    const int take = (int)min(want, (unsigned long long)max(1, sh[2]));
    if (before < take && take <= before + eq) {
        int left = take - before, cut = i0;
        for (int i = i0; i < i1 && left > 0; ++i)
            if (f2key(U > 0 ? kl[i] : s[i]) == prefix) {
                cut = i;
                --left;
            }
        sh[4] = (int)prefix;
        sh[5] = cut;
    }
    __syncthreads();
    const int2 r = make_int2(sh[4], sh[5]);
    __syncthreads();
    return r;
}

}  // namespace sffn
