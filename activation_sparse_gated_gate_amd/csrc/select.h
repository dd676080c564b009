// Per-token K-th largest key of the Top-K selection, computed by one block of
// 1024 threads (the select kernel of topk.hip).
#pragma once

#include "device_common.h"
#include "topk_wg.h"

namespace sffn {

// ---------------------------------------------------------------------------
// One workgroup (1024 threads) per token.
//
// Stage 1 bins the keys by value: the 2048 equal-width bins of key_bin over
// [kKeyLo, kKeyLo + 8) that the decode select uses (SiLU keys are >= -0.2785;
// keys past either end go to the end bins). The bin of a value is a
// non-decreasing function of it, so every key of a higher bin is at least as
// large as every key of a lower one and the K-th largest lies in the bin where
// the count from the top reaches K (found by a block-wide scan, two bins per
// thread). Equal keys share a bin. SiLU keys crowd into a few exponent values,
// so value bins spread the histogram atomics where a radix digit of the
// leading bits would pile them onto a handful of LDS words.
//
// Stage 2 resolves that bin exactly. Up to 64 candidates are gathered in LDS
// and one wavefront ranks them by (key descending, channel ascending).
// Larger bins go through an MSD radix select restricted to the bin: 8 bits
// per pass over the order-preserving 32-bit keys with a 256-bin histogram
// (radix k-selection as in Alabi, Blanchard, Gordon & Steinbach, "Fast
// k-Selection Algorithms for Graphics Processing Units", 2012), then a block
// scan of the keys equal to the K-th gives the tie cutoff.
//
// KPT > 0: thread j holds keys [KPT j, KPT j + KPT) in registers (F <= 1024
// KPT) and the keys are read from memory once. KPT == 0: any F, the keys are
// re-read at every stage.
// ---------------------------------------------------------------------------
// LDS of one select (a 1024-thread block).
struct __align__(16) SelectLds {
    static constexpr int NB = 2048, CMAX = 64;
    int hist[NB];  // value bins, later 3 x 256 radix bins (read as int4)
    float red[2][16];
    uint32_t cand_key[CMAX];
    int cand_idx[CMAX];
    int sh[4];  // bin of the K-th, keys of it still needed, count in it, gathered; then the result
    int scan_scratch[16];
};

// This thread's keys of the KPT > 0 form: kf[e] = s[KPT tid + e] (0 past F).
template <int KPT>
__device__ __forceinline__ void load_keys(const float *__restrict__ s, int F, float (&kf)[KPT > 0 ? KPT : 1])
{
    if constexpr (KPT > 0) {
        const int i0 = threadIdx.x * KPT;
#pragma unroll
        for (int e = 0; e < KPT; ++e) kf[e] = (i0 + e < F) ? s[i0 + e] : 0.f;
    }
}

// Clears the bins of a select; the caller runs it before loading the keys
// (their loads then overlap it), and select_kth's first barrier orders both.
__device__ __forceinline__ void select_kth_clear(SelectLds &L)
{
    reinterpret_cast<int2 *>(L.hist)[threadIdx.x] = make_int2(0, 0);
}

// The select of one token's keys s[0 .. F) by a block of 1024 threads, with
// this thread's keys in kf (load_keys) when KPT > 0; returns {K-th key, tie
// cutoff} in every thread. The bins must have been cleared by
// select_kth_clear. Contains barriers.
template <int KPT>
__device__ __forceinline__ int2 select_kth(const float *__restrict__ s, int F, int K, SelectLds &L,
                                           const float (&kf)[KPT > 0 ? KPT : 1])
{
    constexpr int NTHR = 1024, CMAX = SelectLds::CMAX;
    static_assert(SelectLds::NB == 2 * NTHR && SelectLds::NB == kKeyBins, "two fixed bins per thread");
    int *hist = L.hist;
    uint32_t *cand_key = L.cand_key;
    int *cand_idx = L.cand_idx;
    int *sh = L.sh;
    int *scan_scratch = L.scan_scratch;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // fn(i, v) over this thread's keys
    auto for_keys = [&](auto &&fn) {
        if constexpr (KPT > 0) {
#pragma unroll
            for (int e = 0; e < KPT; ++e)
                if (tid * KPT + e < F) fn(tid * KPT + e, kf[e]);
        } else {
            for (int i = tid; i < F; i += NTHR) fn(i, s[i]);
        }
    };

    // ---- stage 1: fixed value bins (key_bin), the bin b* of the K-th ----
    // (the bins were cleared by select_kth_clear before the keys were loaded)
    __syncthreads();
    for_keys([&](int, float v) { atomicAdd(&hist[key_bin(v)], 1); });
    __syncthreads();
    {
        // thread tid owns bins 2 tid and 2 tid + 1; the count from the top is
        // F minus the inclusive prefix from bin 0
        const int2 c2 = reinterpret_cast<const int2 *>(hist)[tid];
        const int incl = block_incl_scan(c2.x + c2.y, scan_scratch);
        int run = F - incl;  // keys in the bins above 2 tid + 1
        if (run < K && K <= run + c2.y) {
            sh[0] = 2 * tid + 1;
            sh[1] = K - run;
            sh[2] = c2.y;
            sh[3] = 0;
        }
        run += c2.y;
        if (run < K && K <= run + c2.x) {
            sh[0] = 2 * tid;
            sh[1] = K - run;
            sh[2] = c2.x;
            sh[3] = 0;
        }
    }
    __syncthreads();
    const int bstar = sh[0], cnt = sh[2];
    int need = sh[1];
    auto bin_of = [](float v) { return key_bin(v); };

    // ---- stage 2a: few candidates, ranked by one wavefront ----
    if (cnt <= CMAX) {
        for_keys([&](int i, float v) {
            if (bin_of(v) == bstar) {
                const int slot = atomicAdd(&sh[3], 1);
                cand_key[slot] = f2key(v);
                cand_idx[slot] = i;
            }
        });
        __syncthreads();
        if (wave == 0 && lane < cnt) {
            const uint32_t mk = cand_key[lane];
            const int mi = cand_idx[lane];
            int rank = 0;
            for (int m = 0; m < cnt; ++m) {
                const uint32_t ok = cand_key[m];
                rank += ok > mk || (ok == mk && cand_idx[m] < mi);
            }
            if (rank == need - 1) {
                sh[0] = (int)mk;
                sh[1] = mi;
            }
        }
        __syncthreads();
        const int2 r = make_int2(sh[0], sh[1]);
        __syncthreads();  // sh is reused by the caller's next select
        return r;
    }

    // ---- stage 2b: radix select within the bin ----
    // Three buffers rotate so a pass needs one barrier: every wavefront scans
    // the finished histogram itself, and pass p clears the buffer of pass
    // p + 1, last read in pass p - 2.
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    uint32_t prefix = 0, pmask = 0;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int shift = 24 - 8 * p;
        int *h = hist + 256 * (p % 3);
        if (tid < 256) hist[256 * ((p + 1) % 3) + tid] = 0;
        for_keys([&](int, float v) {
            const uint32_t key = f2key(v);
            if (bin_of(v) == bstar && (key & pmask) == prefix) atomicAdd(&h[(key >> shift) & 255u], 1);
        });
        __syncthreads();
        // lane l owns bins 255-4l .. 252-4l (descending)
        const int4 c4 = *reinterpret_cast<const int4 *>(&h[252 - 4 * lane]);
        const int c[4] = {c4.w, c4.z, c4.y, c4.x};
        const int tot = c[0] + c[1] + c[2] + c[3];
        int run = wave_incl_scan(tot) - tot;
        int my_digit = -1, my_need = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (run < need && need <= run + c[e]) {
                my_digit = 255 - (lane * 4 + e);
                my_need = need - run;
            }
            run += c[e];
        }
        const unsigned long long hit = __ballot(my_digit >= 0);
        const int src = __ffsll((long long)hit) - 1;
        const int digit = __shfl(my_digit, src, 64);
        need = __shfl(my_need, src, 64);
        prefix |= (uint32_t)digit << shift;
        pmask |= 0xffu << shift;
    }
    const uint32_t kth = prefix;

    // need = how many keys equal to the K-th belong to the set: the first
    // `need` of them in channel order. Contiguous segments per thread make
    // "equal keys before mine" an exclusive block scan.
    const int seg = KPT > 0 ? KPT : (F + NTHR - 1) / NTHR;
    const int i0 = min(F, tid * seg), i1 = min(F, i0 + seg);
    int eq_local = 0;
    if constexpr (KPT > 0) {
#pragma unroll
        for (int e = 0; e < KPT; ++e) eq_local += (i0 + e < i1 && f2key(kf[e]) == kth);
    } else {
        for (int i = i0; i < i1; ++i) eq_local += f2key(s[i]) == kth;
    }
    const int eq_before = block_incl_scan(eq_local, scan_scratch) - eq_local;
    __syncthreads();  // sh was read above; it carries the result now
    if (eq_before < need && need <= eq_before + eq_local) {
        int left = need - eq_before, cut = i0;
        if constexpr (KPT > 0) {
#pragma unroll
            for (int e = 0; e < KPT; ++e)
                if (i0 + e < i1 && f2key(kf[e]) == kth && left > 0) {
                    cut = i0 + e;
                    --left;
                }
        } else {
            for (int i = i0; i < i1 && left > 0; ++i)
                if (f2key(s[i]) == kth) {
                    cut = i;
                    --left;
                }
        }
        sh[0] = (int)kth;
        sh[1] = cut;
    }
    __syncthreads();
    const int2 r = make_int2(sh[0], sh[1]);
    __syncthreads();
    return r;
}

}  // namespace sffn

namespace sffn {

// ---------------------------------------------------------------------------
// Top-p: the shortest prefix of the Top-K order (key descending, channel
// ascending) whose softmax mass of the token's keys reaches p. One workgroup
// (1024 threads) per token; the result is the same {boundary key, tie cutoff}
// pair as select_kth, so the Top-K flag rule (topk_on) applies it.
//
// Masses are fixed-point integers, u = round(exp(v - max) * 2^44) (24
// significant bits, as exp is computed in fp32), so every sum is exact and
// independent of order: Z = sum u (< 2^62 for d_ff <= 2^18) and the target
// T = ceil(p * Z). The search is select_kth's with masses in place of counts:
// 2048 value bins carrying a count and a mass each; a wavefront sums them to
// Z and finds the bin where the mass from the top reaches T. Up to 64 candidates in that bin
// are ranked by one wavefront, each summing the masses of the candidates
// ahead of it; the boundary channel is the one whose prefix mass falls short
// of T and reaches it with its own. A larger bin goes through four 8-bit
// radix passes over the order-preserving keys with a mass per digit, which
// fixes the boundary key exactly; the channels equal to it that are needed
// (ceil(mass still needed / their mass)) are taken in channel order.
// ---------------------------------------------------------------------------
struct __align__(16) SelectMassLds {
    static constexpr int NB = 2048, CMAX = 64;
    unsigned long long mass[NB];  // value bins, later 3 x 256 radix digits
    int hist[NB];
    unsigned long long cand_w[CMAX];
    uint32_t cand_key[CMAX];
    int cand_idx[CMAX];
    unsigned long long shm[2];  // mass above the crossing bin; the target T
    float red[2][16];
    unsigned long long scan64[16];
    int sh[4];  // crossing bin, its count, gathered; then the result
    int scan_scratch[16];
};

template <int KPT>
__device__ __forceinline__ int2 select_mass(const float *__restrict__ s, int F, float p, SelectMassLds &L,
                                            const float (&kf)[KPT > 0 ? KPT : 1])
{
    constexpr int NTHR = 1024, NB = SelectMassLds::NB, CMAX = SelectMassLds::CMAX;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    auto for_keys = [&](auto &&fn) {
        if constexpr (KPT > 0) {
#pragma unroll
            for (int e = 0; e < KPT; ++e)
                if (tid * KPT + e < F) fn(tid * KPT + e, kf[e]);
        } else {
            for (int i = tid; i < F; i += NTHR) fn(i, s[i]);
        }
    };

    // ---- range, total mass, target ----
    float lo = INFINITY, hi = -INFINITY;
    for_keys([&](int, float v) {
        lo = fminf(lo, v);
        hi = fmaxf(hi, v);
    });
    lo = wave_minmax<false>(lo);
    hi = wave_minmax<true>(hi);
    if (lane == 0) {
        L.red[0][wave] = lo;
        L.red[1][wave] = hi;
    }
    for (int b = tid; b < NB; b += NTHR) {
        L.hist[b] = 0;
        L.mass[b] = 0ull;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < 16; ++w) {
        lo = fminf(lo, L.red[0][w]);
        hi = fmaxf(hi, L.red[1][w]);
    }
    const float top = hi;
    auto mass_of = [&](float v) -> unsigned long long { return topp_mass(v, top); };
    // the target mass from the total Z (the sum of the bin masses below)
    auto target = [&](unsigned long long Z) { return topp_target(p, Z); };

    // The channels equal to the key kth that the prefix needs, given the
    // mass `need` still missing, are the first ceil(need / u) of them in
    // channel order; returns {kth, last of them}. Contiguous segments per
    // thread make "equal keys before mine" an exclusive block scan.
    auto take_ties = [&](uint32_t kth, unsigned long long need) -> int2 {
        const unsigned long long u = mass_of(key2f(kth));
        const unsigned long long want = u > 0 ? (need + u - 1) / u : 1ull;
        const int seg = KPT > 0 ? KPT : (F + NTHR - 1) / NTHR;
        const int i0 = min(F, tid * seg), i1 = min(F, i0 + seg);
        int eq_local = 0;
        if constexpr (KPT > 0) {
#pragma unroll
            for (int e = 0; e < KPT; ++e) eq_local += (i0 + e < i1 && f2key(kf[e]) == kth);
        } else {
            for (int i = i0; i < i1; ++i) eq_local += f2key(s[i]) == kth;
        }
        const int eq_incl = block_incl_scan(eq_local, L.scan_scratch), eq_before = eq_incl - eq_local;
        if (tid == NTHR - 1) L.sh[3] = eq_incl;  // equal channels in all
        __syncthreads();
        const int n_eq = L.sh[3];
        const int take = (int)min(want, (unsigned long long)max(1, n_eq));
        __syncthreads();  // sh carries the result now
        if (eq_before < take && take <= eq_before + eq_local) {
            int left = take - eq_before, cut = i0;
            if constexpr (KPT > 0) {
#pragma unroll
                for (int e = 0; e < KPT; ++e)
                    if (i0 + e < i1 && f2key(kf[e]) == kth && left > 0) {
                        cut = i0 + e;
                        --left;
                    }
            } else {
                for (int i = i0; i < i1 && left > 0; ++i)
                    if (f2key(s[i]) == kth) {
                        cut = i;
                        --left;
                    }
            }
            L.sh[0] = (int)kth;
            L.sh[1] = cut;
        }
        __syncthreads();
        const int2 r = make_int2(L.sh[0], L.sh[1]);
        __syncthreads();
        return r;
    };

    if (!(hi > lo)) return take_ties(f2key(hi), target((unsigned long long)F << 44));  // every key equal: u = 2^44
    float scale = (float)NB / (hi - lo);
    if (!(scale < 1e30f)) scale = 0.f;  // range too narrow to scale: one bin, resolved below
    auto bin_of = [&](float v) {
        const float q = (v - lo) * scale;  // >= 0
        return q >= (float)NB ? NB - 1 : (int)q;
    };

    // ---- stage 1: count and mass per value bin, bin where the mass from the top reaches T ----
    for_keys([&](int, float v) {
        const int b = bin_of(v);
        atomicAdd(&L.hist[b], 1);
        atomicAdd(&L.mass[b], mass_of(v));
    });
    __syncthreads();
    {
        // thread tid owns bins 2 tid and 2 tid + 1: a block-wide inclusive scan
        // of their masses from bin 0 (16 wavefront scans and their totals);
        // the mass from the top is the total Z minus it
        static_assert(NB == 2 * NTHR, "two bins per thread");
        const unsigned long long m0 = L.mass[2 * tid], m1 = L.mass[2 * tid + 1];
        unsigned long long incl = wave_incl_scan_u64(m0 + m1);
        if (lane == 63) L.scan64[wave] = incl;
        __syncthreads();
        unsigned long long Z = 0;
#pragma unroll
        for (int w = 0; w < 16; ++w) {
            const unsigned long long t = L.scan64[w];
            incl += w < wave ? t : 0ull;
            Z += t;
        }
        const unsigned long long T = target(Z);
        if (tid == 0) L.shm[1] = T;
        unsigned long long run = Z - incl;  // mass in the bins above 2 tid + 1
        if (run < T && T <= run + m1) {
            L.sh[0] = 2 * tid + 1;
            L.sh[1] = L.hist[2 * tid + 1];
            L.sh[2] = 0;
            L.shm[0] = run;
        }
        run += m1;
        if (run < T && T <= run + m0) {
            L.sh[0] = 2 * tid;
            L.sh[1] = L.hist[2 * tid];
            L.sh[2] = 0;
            L.shm[0] = run;
        }
    }
    __syncthreads();
    const int bstar = L.sh[0], cnt = L.sh[1];
    unsigned long long need = L.shm[1] - L.shm[0];  // in (0, mass of bin bstar]

    // ---- stage 2a: few candidates, ranked by one wavefront ----
    if (cnt <= CMAX) {
        for_keys([&](int i, float v) {
            if (bin_of(v) == bstar) {
                const int slot = atomicAdd(&L.sh[2], 1);
                L.cand_key[slot] = f2key(v);
                L.cand_idx[slot] = i;
                L.cand_w[slot] = mass_of(v);
            }
        });
        __syncthreads();
        if (wave == 0 && lane < cnt) {
            const uint32_t mk = L.cand_key[lane];
            const int mi = L.cand_idx[lane];
            unsigned long long ahead = 0;
            for (int m = 0; m < cnt; ++m) {
                const uint32_t ok = L.cand_key[m];
                if (ok > mk || (ok == mk && L.cand_idx[m] < mi)) ahead += L.cand_w[m];
            }
            if (ahead < need && need <= ahead + L.cand_w[lane]) {
                L.sh[0] = (int)mk;
                L.sh[1] = mi;
            }
        }
        __syncthreads();
        const int2 r = make_int2(L.sh[0], L.sh[1]);
        __syncthreads();
        return r;
    }

    // ---- stage 2b: radix passes within the bin, a mass per digit ----
    // Three buffers rotate so a pass needs one barrier (as in select_kth).
    unsigned long long *dm = L.mass;
    if (tid < 256) dm[tid] = 0ull;
    __syncthreads();
    uint32_t prefix = 0, pmask = 0;
#pragma unroll
    for (int ps = 0; ps < 4; ++ps) {
        const int shift = 24 - 8 * ps;
        unsigned long long *h = dm + 256 * (ps % 3);
        if (tid < 256) dm[256 * ((ps + 1) % 3) + tid] = 0ull;
        for_keys([&](int, float v) {
            const uint32_t key = f2key(v);
            if (bin_of(v) == bstar && (key & pmask) == prefix) atomicAdd(&h[(key >> shift) & 255u], mass_of(v));
        });
        __syncthreads();
        // lane l owns digits 255-4l .. 252-4l (descending)
        unsigned long long c[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) c[e] = h[255 - 4 * lane - e];
        const unsigned long long tot = c[0] + c[1] + c[2] + c[3];
        unsigned long long run = wave_incl_scan_u64(tot) - tot;
        int my_digit = -1;
        unsigned long long my_need = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (run < need && need <= run + c[e]) {
                my_digit = 255 - (lane * 4 + e);
                my_need = need - run;
            }
            run += c[e];
        }
        const unsigned long long hit = __ballot(my_digit >= 0);
        const int src = __ffsll((long long)hit) - 1;
        const int digit = __shfl(my_digit, src, 64);
        need = __shfl(my_need, src, 64);
        prefix |= (uint32_t)digit << shift;
        pmask |= 0xffu << shift;
    }
    return take_ties(prefix, need);
}

}  // namespace sffn
