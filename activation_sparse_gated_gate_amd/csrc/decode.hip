// Decode-regime kernels (1..8 tokens): every weight row is streamed from HBM
// once and dotted with all tokens, whose chunks sit in registers.
//
// Pipeline per forward (modes as in include/sffn.h):
//   threshold  k_gate<SELECT_UP>: gate GEMV, shifted-ReLU select, and the W_up
//              rows of the channels just found active -> k_down
//   LoPA       k_lopa_xa (t = x.A, a workgroup per row of A) -> k_gate<SELECT_UP>
//              on B with t -> k_down
//   Top-K      k_gate<KEYS> (SiLU keys) -> k_up_topk (select workgroups find
//              each token's boundary, the rest wait for it; flags + up
//              rows) -> k_down
//   top-p      the same, the select workgroups finding the boundary of the
//              cumulative softmax mass p (wg_topp_boundary)
//   2:8        k_gate<SELECT_NM>: gate GEMV, SiLU keys ranked within each
//              aligned group of 8 channels, and the W_up rows of the 2 kept
//              per group -> k_down
//   dense      k_gate<DENSE> (gate and up rows of every channel) -> k_down
//
// The gate is computed first and in full; only the channels it leaves active
// read their W_up and W_down rows ("Model Casting and Low-Parameter Gating",
// Abstract). Those rows are contiguous in the channel-major weights, so an
// active channel costs two contiguous row reads ("Mixture-of-Channels" blog
// summary, "Dentro il 'mixture'": load only the active channels' weights).
//
// Work is split evenly per compute unit: under full load a CU draws about
// 1/256 of the HBM bandwidth, so a kernel lasts as long as its most loaded CU.
// Active channels are byte flags act[t][i], and any[i] for the union over the
// tokens, with one writer each, so any row partition works without atomics.
// Two kernels have workgroups wait on others of the same launch: the down
// kernel's summing workgroups (for the partial sums, see k_down) and the
// Top-K up kernel's (for the per-token boundary, see k_up_topk); everything
// else passes through global memory to the next kernel.
#include "compact.h"
#include "rowdot.h"
#include "topk_wg.h"

#include <algorithm>
#include <type_traits>

namespace sffn {

// ---------------------------------------------------------------------------
// Cross-workgroup slots inside one launch. A slot is 64 bits: a value in the
// low half and the epoch of the forward that wrote it in the high half. The
// producer writes it with a relaxed device-scope atomic store
// (global_store ... sc1); the consumer polls it with device-scope atomic
// loads until the epoch is the current forward's. Each slot carries its own
// readiness, which per-location coherence alone makes sound: no counter, no
// fence (a device-scope release fence writes back the whole L2 of an XCD),
// and nothing to re-mark, so a value left by an earlier forward is never taken
// for a new one. The epoch is a device counter that the gate kernel, the
// first kernel of every decode forward, advances; the next kernels read it,
// so graph replays get fresh epochs too. A consumer only waits on workgroups
// of lower index that never wait; workgroups are dispatched in index order on
// each XCD, so every wait ends. The polls are bounded anyway: a consumer that
// gives up writes NaN to its outputs and sets bit 0 of the workspace's sticky
// error word.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t ld_slot(const uint64_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_slot(uint64_t *p, uint32_t epoch, float v)
{
    __hip_atomic_store(p, ((uint64_t)epoch << 32) | __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// This forward's epoch, read by one thread into LDS (the caller's next
// barrier publishes it). The gate kernel that wrote it has completed, so a
// plain (cached) load sees it; one load per workgroup, issued after the
// caller's own loads, keeps it off the critical path and off a single memory
// channel (an atomic load from every thread queues there).
__device__ __forceinline__ void read_epoch(const int *ctrl, int tid, uint32_t *epoch_s)
{
    if (tid == 0)
        *epoch_s = (uint32_t)__hip_atomic_load(ctrl + kCtrlEpoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// ---------------------------------------------------------------------------
// Up kernel of the decode Top-K, with the per-token select folded in (no
// separate select launch between the gate and the up rows). The first 8 n
// workgroups select: workgroup b finds the boundary of token b / 8 in the
// keys the gate kernel wrote (wg_topk_boundary) and publishes it in set
// b % 8, tagged with this forward's epoch, in three steps: a prefetch
// estimate from a sample of the keys, the boundary bin b*, the exact pair.
// The other workgroups take the rows; each reads its tokens' slots in set
// b % 8 (one thread per token polls; blocks are dispatched in index order,
// so the select workgroups, which have the lowest indices, are running).
// With the estimate they compute the dot products of the W_up rows it marks
// as likely kept (the coarse bins at or above it, a 25 % margin), before b*
// is known. With b* alone a row is kept if its key's bin is above b* and
// dropped if below (kept rows the estimate missed are computed then); the
// rows in b* itself (a few per token) are computed as if kept and settled by
// the exact pair (topk_on), read after their dot products. Then: the
// flags act[t][i], the union flags any[i] and the W_up rows of the channels
// some token kept: h[i][t] = g * (x_t . W_up[i]). On a block-dispatch order
// of 8 XCDs in turn, set s lies on XCD s with its pollers. A wait that
// reaches the spin limit is no error: that workgroup runs the select itself.
// ---------------------------------------------------------------------------
// At least two rows per wavefront (4 waves x SUB x R rows per workgroup), so
// that the workgroups of a layer fit on the GPU at once while they wait.
template <int NT>
struct TopkRows {
    static constexpr int v = RowsPer<NT>::v < 2 ? 2 : RowsPer<NT>::v;
};

// Slots of token t in set s: {b*, K-th key, cutoff, prefetch estimate}.
__device__ __forceinline__ uint64_t *topk_slot(uint64_t *tslot, int set, int t)
{
    return tslot + ((size_t)set * kDecodeMaxTokens + t) * 4;
}

// Polls a slot until it carries `epoch` or spin_max polls have passed;
// true and the slot's low 32 bits in v when it did.
__device__ __forceinline__ bool topk_poll(const uint64_t *p, uint32_t epoch, int spin_max, uint32_t &v)
{
    uint64_t w = ld_slot(p);
    for (int spin = 0; spin <= spin_max; ++spin) {
        if ((uint32_t)(w >> 32) == epoch) {
            v = (uint32_t)w;
            return true;
        }
        if (spin == spin_max) break;
        __builtin_amdgcn_s_sleep(1);
        w = ld_slot(p);
    }
    return false;
}

// The select workgroups' LDS: counts per value bin (Top-K) or masses (top-p).
template <bool MASS>
using SelLds = typename std::conditional<MASS, ToppLds, TopkLds>::type;

// One token's select by the whole workgroup: its keys staged (U > 0), its
// boundary into thr_s[t] (bs_s[t] = -1: exact), and, with slot, the
// prefetch estimate, b* and then the exact pair published there. MASS: the
// top-p boundary of mass p (wg_topp_boundary), else the Top-K one of K.
template <int U, bool MASS>
__device__ __noinline__ void topk_select_token(const float *__restrict__ gsel, int F, int K, float p,
                                               SelLds<MASS> &L, float *kl, int t, uint64_t *slot, uint32_t epoch,
                                               int2 *thr_s, int *bs_s)
{
    const float *s = gsel + (size_t)t * F;
    if constexpr (U > 0) {
        topk_stage_keys<U>(s, F, kl);
        wait_vm_lgkm<0>();
        __syncthreads();
    }
    int2 r;
    if constexpr (MASS)
        r = wg_topp_boundary<U>(s, F, p, L, kl, slot ? slot + 3 : nullptr, slot, epoch);
    else
        r = wg_topk_boundary<U>(s, F, K, L, kl, slot ? slot + 3 : nullptr, slot, epoch);
    if (threadIdx.x == 0) {
        if (slot) {
            __hip_atomic_store(slot + 1, ((uint64_t)epoch << 32) | (uint32_t)r.x, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(slot + 2, ((uint64_t)epoch << 32) | (uint32_t)r.y, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
        if (thr_s) {
            thr_s[t] = r;
            bs_s[t] = -1;
        }
    }
}

template <typename TW, int NT, int LPR, int U, bool MASS>
__global__ __launch_bounds__(256) void k_up_topk(const TW *__restrict__ x, int n, int d,
                                                 const TW *__restrict__ wu, int F, int K, float p,
                                                 uint8_t *__restrict__ act,
                                                 uint8_t *__restrict__ any, const float *__restrict__ gsel,
                                                 float *__restrict__ hbuf, uint64_t *__restrict__ tslot,
                                                 const int *__restrict__ ctrl, int spin_max)
{
    constexpr int SUB = 64 / LPR;
    constexpr int R = TopkRows<NT>::v;
    __shared__ SelLds<MASS> L;
    __shared__ float kl[U > 0 ? U * 256 : 1];  // a select's keys (U > 0)
    __shared__ int2 thr_s[NT];                 // exact boundaries
    __shared__ int bs_s[NT];                   // boundary bins; -1: thr_s holds the exact pair
    __shared__ int est_s[NT];                  // estimates of the kept coarse bins
    __shared__ int miss_s[2][NT];              // waits that reached the spin limit
    __shared__ int need_s[NT];                 // this workgroup has rows in the token's b*
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int b = blockIdx.x, set = b & 7;

    // this forward's epoch, read by the threads that publish or poll (the
    // gate kernel that wrote it has completed, so a cached load sees it)
    uint32_t epoch = 0;
    if (tid < n) epoch = (uint32_t)__hip_atomic_load(ctrl + kCtrlEpoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (b < 8 * n) {  // a select workgroup
        topk_select_token<U, MASS>(gsel, F, K, p, L, kl, b >> 3, topk_slot(tslot, set, b >> 3), epoch, nullptr,
                             nullptr);  // (thread 0, which publishes, has the epoch)
        return;
    }

    const int q = lane / LPR, li = lane % LPR;
    const int wrow0 = ((b - 8 * n) * 4 + wave) * SUB * R;  // this wavefront's first row
    const int row0 = wrow0 + q * R;
    const int nv = max(0, min(R, F - row0));
    float kv[R][NT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int t = 0; t < NT; ++t) kv[r][t] = (r < nv && t < n) ? gsel[(size_t)t * F + row0 + r] : 0.f;
    if (tid < NT) {
        miss_s[0][tid] = miss_s[1][tid] = 0;
        need_s[tid] = 0;
    }
    // the prefetch estimates, then the dot products of the rows they mark as
    // likely kept, before the boundary bin is known (the rows kept in the
    // end are nearly all among them; the others are computed after b*)
    if (tid < n) {
        uint32_t v = 64;
        est_s[tid] = topk_poll(topk_slot(tslot, set, tid) + 3, epoch, spin_max, v) ? (int)v : 64;
    }
    __syncthreads();
    const TW *rows[R];
#pragma unroll
    for (int r = 0; r < R; ++r) rows[r] = wu + (size_t)(row0 + r) * d;
    uint32_t smask = 0;  // rows computed ahead
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int t = 0; t < NT; ++t)
            if (r < nv && t < n && (key_bin(kv[r][t]) >> 5) >= est_s[t]) smask |= 1u << r;
    RowDot<TW, TW, NT, R, LPR, Batch<TW, TW, NT, R>::v> up;
    if (__ballot(smask != 0)) {
        up.run(rows, smask, d, li, x, d, n);
    } else {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int t = 0; t < NT; ++t) up.acc[r][t] = 0.f;
    }

    // the boundary bins; a wait that reaches the limit selects here
    if (tid < n) {
        uint32_t v = 0;
        if (topk_poll(topk_slot(tslot, set, tid), epoch, spin_max, v))
            bs_s[tid] = (int)v;
        else
            miss_s[0][tid] = 1;
    }
    __syncthreads();
    uint32_t todo = 0;
    for (int t = 0; t < n; ++t) todo |= (uint32_t)miss_s[0][t] << t;
    for (; todo; todo &= todo - 1)  // uniform over the workgroup
        topk_select_token<U, MASS>(gsel, F, K, p, L, kl, __ffs(todo) - 1, nullptr, 0, thr_s, bs_s);
    __syncthreads();

    // the rows kept by bin, and the rows in b* (computed as if kept)
    uint32_t amask = 0;  // rows needed
    uint32_t amb = 0;    // bit r * NT + t: row r is in token t's b*
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int t = 0; t < NT; ++t)
            if (r < nv && t < n) {
                const int bs = bs_s[t];
                const int kb = key_bin(kv[r][t]);
                if (bs >= 0 && kb == bs) {
                    amb |= 1u << (r * NT + t);
                    amask |= 1u << r;
                    need_s[t] = 1;
                } else if (bs < 0 ? topk_on(kv[r][t], row0 + r, thr_s[t]) : kb > bs) {
                    amask |= 1u << r;
                }
            }
    const uint32_t late = amask & ~smask;  // needed, not computed ahead
    if (__ballot(late != 0)) {
        RowDot<TW, TW, NT, R, LPR, Batch<TW, TW, NT, R>::v> up2;
        up2.run(rows, late, d, li, x, d, n);
#pragma unroll
        for (int r = 0; r < R; ++r)
            if ((late >> r) & 1u)
#pragma unroll
                for (int t = 0; t < NT; ++t) up.acc[r][t] = up2.acc[r][t];
    }
    __syncthreads();  // need_s
    // the exact pairs the rows in b* need; a wait that reaches the limit
    // selects here
    if (tid < n && need_s[tid] && bs_s[tid] >= 0) {
        uint32_t key = 0, cut = 0;
        const uint64_t *p = topk_slot(tslot, set, tid);
        if (topk_poll(p + 1, epoch, spin_max, key) && topk_poll(p + 2, epoch, spin_max, cut))
            thr_s[tid] = make_int2((int)key, (int)cut);
        else
            miss_s[1][tid] = 1;
    }
    __syncthreads();
    todo = 0;
    for (int t = 0; t < n; ++t) todo |= (uint32_t)miss_s[1][t] << t;
    for (; todo; todo &= todo - 1)
        topk_select_token<U, MASS>(gsel, F, K, p, L, kl, __ffs(todo) - 1, nullptr, 0, thr_s, bs_s);
    __syncthreads();

    // the flags: kept by bin, or settled by the exact pair in b*
    float gv[R][NT];
    uint32_t kmask = 0;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            gv[r][t] = 0.f;
            if (r < nv && t < n) {
                const int bs = bs_s[t];
                const bool on = (bs < 0 || ((amb >> (r * NT + t)) & 1u)) ? topk_on(kv[r][t], row0 + r, thr_s[t])
                                                                          : key_bin(kv[r][t]) > bs;
                if (li == ((r * NT + t) & (LPR - 1))) act[(size_t)t * F + row0 + r] = on;
                if (on) {
                    gv[r][t] = kv[r][t];
                    kmask |= 1u << r;
                }
            }
        }
#pragma unroll
    for (int r = 0; r < R; ++r)
        if (r < nv && li == (r & (LPR - 1))) any[row0 + r] = (kmask >> r) & 1u;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int t = 0; t < NT; ++t)
            if (((kmask >> r) & 1u) && t < n && li == ((r * NT + t) & (LPR - 1)))
                hbuf[(size_t)(row0 + r) * kDecodeMaxTokens + t] = gv[r][t] * up.acc[r][t];
}

// ---------------------------------------------------------------------------
// Down kernel: the split-channel two-stage reduction in one launch, over
// G = gridDim.y channel groups.
// Stage 1: workgroup (s, g) takes output columns [128 s, 128 s + 128) and
// channels [F g / G, F (g+1) / G). It lists that range's channels some token
// selected (any[i]; every channel in the dense modes) in LDS in ascending
// order, then its 16 row streams (4 per wavefront, 16 lanes x 8 columns each)
// read the 256-byte segments of those W_down rows, UNR rows per stream in
// flight:  P[g][t][c] = sum_i h[i][t] * W_down[i][c]   (fixed order).
// Stage 2: workgroup (s, G-1) sums P[0][t][c], ..., P[G-1][t][c] in that
// order and writes y. The other groups publish their P in epoch-tagged slots
// (above), which the summing workgroup polls, 16 at a time.
// ---------------------------------------------------------------------------
template <typename TW, int NT, int UNR>
__global__ __launch_bounds__(256) void k_down(const TW *__restrict__ wd, int F, int d, int n,
                                              const uint8_t *__restrict__ any, int dense,
                                              const float *__restrict__ hbuf, uint64_t *__restrict__ part,
                                              float *__restrict__ y, int *__restrict__ ctrl, int spin_max)
{
    __shared__ uint16_t list[kDownRangeMax];
    __shared__ float red[4][NT][kDownSliceCols];
    __shared__ int scan_scratch[4];
    __shared__ int total;
    __shared__ uint32_t epoch_s;
    const int s = blockIdx.x, g = blockIdx.y, G = gridDim.y;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int cb = F * g / G, ce = F * (g + 1) / G;  // F * G < 2^31 (F <= 262144, G <= 64)

    // ---- this group's selected channels, ascending (offsets from cb) ----
    const int len = ce - cb;
    const int seg = (len + 255) / 256;  // <= 32: a group has at most kDownRangeMax channels
    const int i0 = cb + min(len, tid * seg), i1 = cb + min(len, tid * seg + seg);
    uint32_t sel = 0;  // bit k: channel i0 + k
    for (int i = i0; i < i1; ++i) sel |= (uint32_t)(dense != 0 || any[i] != 0) << (i - i0);
    read_epoch(ctrl, tid, &epoch_s);
    const int local = __popc(sel);
    const int incl = block_incl_scan(local, scan_scratch);
    int pos = incl - local;
    while (sel) {
        const int b = __ffs(sel) - 1;
        sel &= sel - 1;
        list[pos++] = (uint16_t)(i0 + b - cb);
    }
    if (tid == 255) total = incl;
    __syncthreads();
    const int m = total;
    const uint32_t epoch = epoch_s;
    // ---- stage 1: this group's rows, 256-byte segments ----
    const int rs = wave * 4 + (lane >> 4), c8 = lane & 15;
    const int col = s * kDownSliceCols + c8 * 8;
    const bool colok = col < d;
    float acc[NT][8];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[t][e] = 0.f;
    if (colok) {
        for (int k0 = rs; k0 < m; k0 += 16 * UNR) {
            typename Ld8<TW>::raw qv[UNR];
            float hv[UNR][NT];
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
                const int k = k0 + 16 * u;
                if (k < m) {
                    const int i = cb + (int)list[k];
                    qv[u] = Ld8<TW>::load(wd + (size_t)i * d + col);
#pragma unroll
                    for (int t = 0; t < NT; ++t) hv[u][t] = hbuf[(size_t)i * kDecodeMaxTokens + t];
                } else {
                    qv[u] = Ld8<TW>::zero();
#pragma unroll
                    for (int t = 0; t < NT; ++t) hv[u][t] = 0.f;
                }
            }
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
                float wv[8];
                Ld8<TW>::cvt(qv[u], wv);
#pragma unroll
                for (int t = 0; t < NT; ++t)
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[t][e] = fmaf(hv[u][t], wv[e], acc[t][e]);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float v = acc[t][e];
            v += __shfl_xor(v, 16, 64);
            v += __shfl_xor(v, 32, 64);
            acc[t][e] = v;
        }
    if (lane < 16) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int e = 0; e < 8; ++e) red[wave][t][c8 * 8 + e] = acc[t][e];
    }
    __syncthreads();

    const int c0 = s * kDownSliceCols;
    const size_t gs = (size_t)kDecodeMaxTokens * d;  // stride of one group's slab
    constexpr int PER = (NT * kDownSliceCols + 255) / 256;  // elements per thread
    if (g < G - 1) {
        // ---- stage 1 only: publish this group's slice of P ----
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int e = tid + 256 * q;
            const int t = e / kDownSliceCols, c = e - t * kDownSliceCols;
            if (t < n && c0 + c < d) {
                const float v = ((red[0][t][c] + red[1][t][c]) + red[2][t][c]) + red[3][t][c];
                st_slot(part + (size_t)g * gs + (size_t)t * d + c0 + c, epoch, v);
            }
        }
        return;
    }
    // ---- stage 2: ordered sum over the groups ----
    constexpr int B = 16;  // slots polled together (32 at once made the wait twice as long)
    bool gave_up = false;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        const int e = tid + 256 * q;
        const int t = e / kDownSliceCols, c = e - t * kDownSliceCols;
        if (t < n && c0 + c < d) {
            const float own = ((red[0][t][c] + red[1][t][c]) + red[2][t][c]) + red[3][t][c];
            const uint64_t *p = part + (size_t)t * d + c0 + c;
            float v = 0.f;
            bool ok = true;
            for (int g0 = 0; g0 < G - 1; g0 += B) {
                uint64_t b[B];
#pragma unroll
                for (int u = 0; u < B; ++u) b[u] = g0 + u < G - 1 ? ld_slot(p + (size_t)(g0 + u) * gs) : 0u;
                bool ready = false;
                for (int spin = 0; spin <= spin_max; ++spin) {
                    ready = true;
#pragma unroll
                    for (int u = 0; u < B; ++u) ready = ready && (g0 + u >= G - 1 || (uint32_t)(b[u] >> 32) == epoch);
                    if (ready || spin == spin_max) break;
                    __builtin_amdgcn_s_sleep(1);
#pragma unroll
                    for (int u = 0; u < B; ++u)
                        if (g0 + u < G - 1 && (uint32_t)(b[u] >> 32) != epoch)
                            b[u] = ld_slot(p + (size_t)(g0 + u) * gs);
                }
                ok = ok && ready;
#pragma unroll
                for (int u = 0; u < B; ++u)
                    if (g0 + u < G - 1) v += __uint_as_float((uint32_t)b[u]);
            }
            y[(size_t)t * d + c0 + c] = ok ? v + own : __builtin_nanf("");
            gave_up = gave_up || !ok;
        }
    }
    if (gave_up) atomicOr(ctrl + kCtrlError, kErrDownWait);
}

// ---------------------------------------------------------------------------
// LoPA first product t[t][k] = x_t . A[k] (fp32) for the r rows of A, stored
// [r][d]: one workgroup per row, its 4 wavefronts each dotting a quarter of
// the row with all tokens (read once), summed in wavefront order; the gate
// kernel then dots the rows of B with t. A row per workgroup keeps r
// workgroups in flight (one row per wavefront left most CUs idle at r = 256).
// ---------------------------------------------------------------------------
template <typename TW, int NT>
__global__ __launch_bounds__(256) void k_lopa_xa(const TW *__restrict__ x, int n, int d, const TW *__restrict__ a,
                                                 int r, float *__restrict__ tvec)
{
    __shared__ float part[4][NT];
    const int row = blockIdx.x, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int q = (d + 31) / 32 * 8;  // a multiple of 8 elements, 4 q >= d
    const int j0 = min(d, wave * q), len = min(d, j0 + q) - j0;
    const TW *rows[1] = {a + (size_t)row * d + j0};
    RowDot<TW, TW, NT, 1, 64, Batch<TW, TW, NT, 1>::v> dot;
    dot.run(rows, len > 0 ? 1u : 0u, len, lane, x + j0, d, n);
    if (lane == 0) {
#pragma unroll
        for (int t = 0; t < NT; ++t) part[wave][t] = dot.acc[0][t];
    }
    __syncthreads();
    if (threadIdx.x < NT && (int)threadIdx.x < n) {
        const int t = threadIdx.x;
        tvec[(size_t)t * r + row] = ((part[0][t] + part[1][t]) + part[2][t]) + part[3][t];
    }
}

// ---------------------------------------------------------------------------
// Optional outputs: each token's ascending active list and count (every
// channel in the dense modes), and the union size. Workgroup b < n handles
// token b; workgroup n counts the union.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_emit_lists(const uint8_t *__restrict__ act, int F, int n, int dense,
                                                    int32_t *__restrict__ active_idx,
                                                    int32_t *__restrict__ active_cnt,
                                                    int32_t *__restrict__ union_cnt)
{
    __shared__ int scratch[5];
    const int b = blockIdx.x;
    const uint8_t *a = act + (size_t)b * F;
    auto token = [&](int i0, bool f[8]) {
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = i0 + e < F && (dense || a[i0 + e] != 0);
    };
    auto any = [&](int i0, bool f[8]) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            bool v = i0 + e < F && (dense || n > 0);
            if (v && !dense) {
                v = false;
                for (int t = 0; t < n; ++t) v |= act[(size_t)t * F + i0 + e] != 0;
            }
            f[e] = v;
        }
    };
    if (b < n) {
        const int c = emit_ordered(F, token, active_idx ? active_idx + (size_t)b * F : nullptr, scratch);
        if (threadIdx.x == 0 && active_cnt) active_cnt[b] = c;
    } else {
        const int c = emit_ordered(F, any, nullptr, scratch);
        if (threadIdx.x == 0 && union_cnt) *union_cnt = c;
    }
}

__global__ void k_zero_ints(int *__restrict__ p, int count)
{
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < count; i += gridDim.x * blockDim.x) p[i] = 0;
}

// ===========================================================================
// Host side
// ===========================================================================
static int lpr_for(int len)
{
    if (len >= 512) return 64;
    if (len >= 256) return 32;
    return 16;
}

static int nt_for(int n) { return n <= 1 ? 1 : n <= 2 ? 2 : n <= 4 ? 4 : 8; }

hipError_t device_setup(sffn_ctx &c)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    int cu = 0;
    e = hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    c.n_cu = cu > 0 ? cu : 1;
    return hipSuccess;
}

__global__ void k_zero_u64(uint64_t *__restrict__ p, size_t count)
{
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < count; i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0;
}

hipError_t launch_init(sffn_ctx &c, hipStream_t s)
{
    // slots start with epoch 0, which no forward uses (the gate kernel's
    // epochs start at 1 and skip 0 when they wrap)
    hipLaunchKernelGGL(k_zero_u64, dim3(256), dim3(256), 0, s, reinterpret_cast<uint64_t *>(c.ws + c.L.part),
                       c.L.part_slots);
    hipLaunchKernelGGL(k_zero_u64, dim3(1), dim3(256), 0, s, reinterpret_cast<uint64_t *>(c.ws + c.L.tslot),
                       (size_t)kTopkSlots);
    hipLaunchKernelGGL(k_zero_ints, dim3(4), dim3(256), 0, s, reinterpret_cast<int *>(c.ws + c.L.ctrl), kCtrlInts);
    hipLaunchKernelGGL(k_zero_ints, dim3(16), dim3(256), 0, s, reinterpret_cast<int *>(c.ws + c.L.ubits), c.L.words);
    return hipGetLastError();
}

template <typename TW, int NT>
static hipError_t run_decode(sffn_ctx &c, const FwdArgs &a)
{
    const sffn_shape &S = c.shape;
    const int d = S.d_model, F = S.d_ff, n = a.n;
    char *ws = c.ws;
    uint8_t *act = reinterpret_cast<uint8_t *>(ws + c.L.act);
    float *gsel = reinterpret_cast<float *>(ws + c.L.gsel);
    float *hbuf = reinterpret_cast<float *>(ws + c.L.hbuf);
    uint8_t *any = reinterpret_cast<uint8_t *>(ws + c.L.any);
    const TW *x = static_cast<const TW *>(a.x);
    const TW *wg = static_cast<const TW *>(a.w.w_gate);
    const TW *wu = static_cast<const TW *>(a.w.w_up);
    const TW *wdn = static_cast<const TW *>(a.w.w_down);
    hipStream_t st = a.stream;
    const bool dense = a.mode == SFFN_DENSE || a.mode == SFFN_DENSE_SILU;
    hipError_t e;

    // ---- gate (+ select, + up for threshold / LoPA / dense) ----
    GateArgs g{};
    g.dtype = S.dtype;
    g.nt = NT;
    g.n = n;
    g.xg = x;
    g.L = d;
    g.xu = x;
    g.d = d;
    g.wg = wg;
    g.wu = wu;
    g.F = F;
    g.mode = a.mode;
    g.tau = a.tau;
    g.gsel = gsel;
    g.act = act;
    g.any = any;
    g.hbuf = hbuf;
    g.debug_z = a.debug_z;
    g.stream = st;
    g.ev_start = c.ev_start;
    g.ev_stop = c.ev_stop;
    g.ctrl = reinterpret_cast<int *>(ws + c.L.ctrl);
    g.lpr = lpr_for(d);
    const bool ranked = a.mode == SFFN_TOPK || a.mode == SFFN_TOPP;  // keys, then a per-token select
    g.kind = dense ? DENSE : ranked ? KEYS : a.mode == SFFN_TOPK_2_8 ? SELECT_NM : SELECT_UP;
    if (g.kind == SELECT_NM && g.lpr == 64 && RowsPer<NT>::v < 2) g.lpr = 32;  // whole 2:8 groups per workgroup
    if (a.mode == SFFN_LOPA) {
        const int r = S.rank;
        float *tvec = reinterpret_cast<float *>(ws + c.L.tvec);
        hipLaunchKernelGGL((k_lopa_xa<TW, NT>), dim3(r), dim3(256), 0, st, x, n, d,
                           static_cast<const TW *>(a.w.lopa_a), r, tvec);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        // gate rows are B (length r) dotted with t = x.A; the gate rows and
        // the up rows (length d) share the lane groups, sized for the shorter
        g.lopa = true;
        g.xg = tvec;
        g.L = r;
        g.wg = a.w.lopa_b;
        g.lpr = lpr_for(min(r, d));
    }
    if ((e = launch_gate(g)) != hipSuccess) return e;

    // ---- Top-K and top-p: the select folded into the up rows ----
    if (a.mode == SFFN_TOPK || a.mode == SFFN_TOPP) {
        const int lpr = lpr_for(d);
        const dim3 ugrid(8 * n + row_blocks(F, lpr, TopkRows<NT>::v));  // 8 select workgroups per token, then the rows
        uint64_t *tslot = reinterpret_cast<uint64_t *>(ws + c.L.tslot);
        const int *ctrl = reinterpret_cast<const int *>(ws + c.L.ctrl);
        auto go = [&](auto lpr_c, auto u_c, auto mass_c) {
            hipLaunchKernelGGL(
                (k_up_topk<TW, NT, decltype(lpr_c)::value, decltype(u_c)::value, decltype(mass_c)::value>), ugrid,
                dim3(256), 0, st, x, n, d, wu, F, a.k, a.tau, act, any, gsel, hbuf, tslot, ctrl, c.spin_max);
        };
        auto go_lpr = [&](auto u_c, auto mass_c) {
            if (lpr == 64) go(std::integral_constant<int, 64>{}, u_c, mass_c);
            else if (lpr == 32) go(std::integral_constant<int, 32>{}, u_c, mass_c);
            else go(std::integral_constant<int, 16>{}, u_c, mass_c);
        };
        auto go_u = [&](auto mass_c) {
            // the select workgroups keep a token's keys in LDS, or stream them for wider layers
            if (F <= kTopkLdsKeys) go_lpr(std::integral_constant<int, kTopkLdsKeys / 256>{}, mass_c);
            else go_lpr(std::integral_constant<int, 0>{}, mass_c);
        };
        if (a.mode == SFFN_TOPP) go_u(std::true_type{});
        else go_u(std::false_type{});
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }

    // ---- down projection: group partials and their ordered sum ----
    uint64_t *part = reinterpret_cast<uint64_t *>(ws + c.L.part);
    const int slices = (d + kDownSliceCols - 1) / kDownSliceCols;
    hipLaunchKernelGGL((k_down<TW, NT, 8>), dim3(slices, down_groups(c.shape.d_ff)), dim3(256), 0, st, wdn, F, d, n, any,
                       dense ? 1 : 0, hbuf, part, a.y, reinterpret_cast<int *>(ws + c.L.ctrl),
                       c.spin_max);
    if ((e = hipGetLastError()) != hipSuccess) return e;

    // ---- optional outputs ----
    if (a.active_idx || a.active_cnt || a.union_cnt) {
        hipLaunchKernelGGL(k_emit_lists, dim3(n + 1), dim3(256), 0, st, act, F, n, dense ? 1 : 0, a.active_idx,
                           a.active_cnt, a.union_cnt);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

template <typename TW>
static hipError_t run_decode_nt(sffn_ctx &c, const FwdArgs &a)
{
    switch (nt_for(a.n)) {
    case 1: return run_decode<TW, 1>(c, a);
    case 2: return run_decode<TW, 2>(c, a);
    case 4: return run_decode<TW, 4>(c, a);
    default: return run_decode<TW, 8>(c, a);
    }
}

hipError_t launch_decode(sffn_ctx &c, const FwdArgs &a)
{
    if (c.shape.dtype == SFFN_BF16) return run_decode_nt<bf16_t>(c, a);
    return run_decode_nt<float>(c, a);
}

}  // namespace sffn
