// Decode-regime kernels (1..8 tokens): every weight row is streamed from HBM
// once and dotted with all tokens, whose chunks sit in registers.
//
// Pipeline per forward (modes as in include/sffn.h):
//   threshold  k_gate<SELECT_UP>: gate GEMV, shifted-ReLU select, and the W_up
//              rows of the channels just found active -> k_down
//   LoPA       k_lopa_xa (t = x.A) -> k_gate<SELECT_UP> on B with t -> k_down
//   Top-K      k_gate<KEYS> (SiLU keys) -> k_topk_thr (select of each token's
//              K-th key) -> k_up (flags + up rows) -> k_down
//   top-p      as Top-K, with k_topp_thr (the boundary of the cumulative
//              softmax mass p) in place of k_topk_thr
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
// Only the down kernel's summing workgroups wait on other workgroups (for
// their partial sums, see k_down); everything else passes through global
// memory to the next kernel.
#include "compact.h"
#include "rowdot.h"

namespace sffn {

// ---------------------------------------------------------------------------
// Up kernel (Top-K): the gate kernel's row partition. Each lane group applies
// the tokens' Top-K thresholds to its channels' keys (topk_on), writes the
// flags act[t][i], and reads the W_up rows of its channels that some token
// selected. h[i][t] = g[t][i] * (x_t . W_up[i]) if token t selected i, else 0.
// ---------------------------------------------------------------------------
template <typename TW, int NT, int LPR>
__global__ __launch_bounds__(256) void k_up(const TW *__restrict__ x, int n, int d,
                                            const TW *__restrict__ wu, int F,
                                            const int2 *__restrict__ thr, uint8_t *__restrict__ act,
                                            uint8_t *__restrict__ any, const float *__restrict__ gsel,
                                            float *__restrict__ hbuf)
{
    constexpr int SUB = 64 / LPR;
    constexpr int R = RowsPer<NT>::v;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int q = lane / LPR, li = lane % LPR;
    const int row0 = ((blockIdx.x * 4 + wave) * SUB + q) * R;
    const int nv = max(0, min(R, F - row0));
    float gv[R][NT];
    uint32_t amask = 0;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            gv[r][t] = 0.f;
            if (r < nv && t < n) {
                const size_t o = (size_t)t * F + row0 + r;
                const float g = gsel[o];
                const bool on = topk_on(g, row0 + r, thr[t]);
                if (li == ((r * NT + t) & (LPR - 1))) act[o] = on;
                if (on) {
                    gv[r][t] = g;
                    amask |= 1u << r;
                }
            }
        }
#pragma unroll
    for (int r = 0; r < R; ++r)
        if (r < nv && li == (r & (LPR - 1))) any[row0 + r] = (amask >> r) & 1u;
    if (__ballot(amask != 0) == 0) return;
    const TW *rows[R];
#pragma unroll
    for (int r = 0; r < R; ++r) rows[r] = wu + (size_t)(row0 + r) * d;
    RowDot<TW, TW, NT, R, LPR, Batch<TW, TW, NT, R>::v> up;
    up.run(rows, amask, d, li, x, d, n);
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int t = 0; t < NT; ++t)
            if (((amask >> r) & 1u) && t < n && li == ((r * NT + t) & (LPR - 1)))
                hbuf[(size_t)(row0 + r) * kDecodeMaxTokens + t] = gv[r][t] * up.acc[r][t];
}

// ---------------------------------------------------------------------------
// Cross-workgroup slots inside one launch. A slot holds the marker, all ones
// (a NaN bit pattern no sum of finite products has), until its producer
// writes it with a relaxed device-scope atomic store (global_store ... sc1);
// the consumer polls it with device-scope atomic loads (global_load ... sc1)
// and writes the marker back after reading. Each slot carries its own
// readiness, which per-location coherence alone makes sound: no counter, no
// fence (a device-scope release fence writes back the whole L2 of an XCD). A
// consumer only waits on workgroups of lower index that never wait;
// workgroups are dispatched in index order on each XCD, so every wait ends.
// The polls are bounded anyway (kSpinMax), after which the marker itself (a
// NaN) is used.
// ---------------------------------------------------------------------------
constexpr uint32_t kSlotMarker = 0xffffffffu;
constexpr int kSpinMax = 1 << 18;

__device__ __forceinline__ uint32_t ld_slot(const uint32_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_slot(uint32_t *p, uint32_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Down kernel: the split-channel two-stage reduction in one launch.
// Stage 1: workgroup (s, g) takes output columns [128 s, 128 s + 128) and
// channels [F g / G, F (g+1) / G). It lists that range's channels some token
// selected (any[i]; every channel in the dense modes) in LDS in ascending
// order, then its 16 row streams (4 per wavefront, 16 lanes x 8 columns each)
// read the 256-byte segments of those W_down rows, UNR rows per stream in
// flight:  P[g][t][c] = sum_i h[i][t] * W_down[i][c]   (fixed order).
// Stage 2: workgroup (s, G-1) sums P[0][t][c], ..., P[G-1][t][c] in that
// order and writes y. The other groups publish their P in marker-tagged slots
// (above), which the summing workgroup polls, reads and re-marks.
// Only the G-1 groups' summing workgroups wait, on workgroups that never wait.
// ---------------------------------------------------------------------------
template <typename TW, int NT, int UNR>
__global__ __launch_bounds__(256) void k_down(const TW *__restrict__ wd, int F, int d, int n,
                                              const uint8_t *__restrict__ any, int dense,
                                              const float *__restrict__ hbuf, uint32_t *__restrict__ part,
                                              float *__restrict__ y)
{
    extern __shared__ __align__(16) char smem[];
    int *list = reinterpret_cast<int *>(smem);
    __shared__ float red[4][NT][kDownSliceCols];
    __shared__ int scan_scratch[4];
    __shared__ int total;
    const int s = blockIdx.x, g = blockIdx.y, G = gridDim.y;
    const int cb = (int)(((long long)F * g) / G), ce = (int)(((long long)F * (g + 1)) / G);
    const int tid = threadIdx.x;

    // ---- channels of this group selected by some token, ascending ----
    const int len = ce - cb;
    const int seg = (len + blockDim.x - 1) / blockDim.x;  // <= 32, fixed on the host
    const int i0 = cb + min(len, tid * seg), i1 = cb + min(len, tid * seg + seg);
    uint32_t sel = 0;  // bit k: channel i0 + k
    for (int i = i0; i < i1; ++i) sel |= (uint32_t)(dense != 0 || any[i] != 0) << (i - i0);
    const int local = __popc(sel);
    const int incl = block_incl_scan(local, scan_scratch);
    int pos = incl - local;
    while (sel) {
        const int b = __ffs(sel) - 1;
        sel &= sel - 1;
        list[pos++] = i0 + b;
    }
    if (tid == blockDim.x - 1) total = incl;
    __syncthreads();
    const int cnt = total;

    const int wave = tid >> 6, lane = tid & 63;
    const int rs = wave * 4 + (lane >> 4), c8 = lane & 15;
    const int col = s * kDownSliceCols + c8 * 8;
    const bool colok = col < d;

    float acc[NT][8];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[t][e] = 0.f;

    if (colok) {
        for (int k0 = rs; k0 < cnt; k0 += 16 * UNR) {
            typename Ld8<TW>::raw qv[UNR];
            float hv[UNR][NT];
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
                const int k = k0 + 16 * u;
                if (k < cnt) {
                    const int i = list[k];
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
                st_slot(part + (size_t)g * gs + (size_t)t * d + c0 + c, __float_as_uint(v));
            }
        }
        return;
    }
    // ---- stage 2: ordered sum over the groups ----
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        const int e = tid + 256 * q;
        const int t = e / kDownSliceCols, c = e - t * kDownSliceCols;
        if (t < n && c0 + c < d) {
            const float own = ((red[0][t][c] + red[1][t][c]) + red[2][t][c]) + red[3][t][c];
            uint32_t *p = part + (size_t)t * d + c0 + c;
            float v = 0.f;
            for (int g0 = 0; g0 < G - 1; g0 += 16) {
                uint32_t b[16];
#pragma unroll
                for (int u = 0; u < 16; ++u)
                    b[u] = g0 + u < G - 1 ? ld_slot(p + (size_t)(g0 + u) * gs) : 0u;
                for (int spin = 0; spin < kSpinMax; ++spin) {
                    bool ready = true;
#pragma unroll
                    for (int u = 0; u < 16; ++u) ready = ready && b[u] != kSlotMarker;
                    if (ready) break;
                    __builtin_amdgcn_s_sleep(1);
#pragma unroll
                    for (int u = 0; u < 16; ++u)
                        if (b[u] == kSlotMarker)
                            b[u] = ld_slot(p + (size_t)(g0 + u) * gs);
                }
#pragma unroll
                for (int u = 0; u < 16; ++u)
                    if (g0 + u < G - 1) {
                        v += __uint_as_float(b[u]);
                        st_slot(p + (size_t)(g0 + u) * gs, kSlotMarker);
                    }
            }
            y[(size_t)t * d + c0 + c] = v + own;
        }
    }
}

// ---------------------------------------------------------------------------
// LoPA first product t[t][k] = x_t . A[k] (fp32) for the r rows of A, stored
// [r][d]: one row per wavefront, read once for all tokens; the gate kernel
// then dots the rows of B with t.
// ---------------------------------------------------------------------------
template <typename TW, int NT>
__global__ __launch_bounds__(256) void k_lopa_xa(const TW *__restrict__ x, int n, int d, const TW *__restrict__ a,
                                                 int r, float *__restrict__ tvec)
{
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const TW *rows[1] = {a + (size_t)min(row, r - 1) * d};
    RowDot<TW, TW, NT, 1, 64, Batch<TW, TW, NT, 1>::v> dot;
    dot.run(rows, row < r ? 1u : 0u, d, lane, x, d, n);
#pragma unroll
    for (int t = 0; t < NT; ++t)
        if (row < r && t < n && lane == t) tvec[(size_t)t * r + row] = dot.acc[0][t];
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

// 16 channel groups, more for very wide layers so that a thread of the list
// prologue scans at most 32 channels of its group.
static int down_groups(const sffn_ctx &c)
{
    const int F = c.shape.d_ff;
    const int G = max(16, (F + 256 * 32 - 1) / (256 * 32));
    return max(1, min(min(G, kDownGroupsMax), F));
}

static size_t down_lds(const sffn_ctx &c)
{
    const int F = c.shape.d_ff, G = down_groups(c);
    return (size_t)4 * ((F + G - 1) / G + 1);
}

hipError_t device_setup(sffn_ctx &c)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    int cu = 0, lds = 0;
    e = hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
    if (e != hipSuccess) return e;
    c.n_cu = cu > 0 ? cu : 1;
    // Dynamic LDS stays within 64 KB per workgroup (static LDS comes on top).
    c.lds_max = (size_t)min(lds, 65536) - 4096;
    return hipSuccess;
}

bool decode_fits(const sffn_ctx &c, int, int) { return down_lds(c) <= c.lds_max; }

__global__ void k_fill_u32(uint32_t *__restrict__ p, size_t count, uint32_t v)
{
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < count; i += (size_t)gridDim.x * blockDim.x)
        p[i] = v;
}

hipError_t launch_init(sffn_ctx &c, hipStream_t s)
{
    // the down projection's group slots start out holding their marker
    hipLaunchKernelGGL(k_fill_u32, dim3(256), dim3(256), 0, s, reinterpret_cast<uint32_t *>(c.ws + c.L.part),
                       c.L.part_words, kSlotMarker);
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
    g.lpr = lpr_for(d);
    const bool ranked = a.mode == SFFN_TOPK || a.mode == SFFN_TOPP;  // keys, then a per-token select
    g.kind = dense ? DENSE : ranked ? KEYS : a.mode == SFFN_TOPK_2_8 ? SELECT_NM : SELECT_UP;
    if (g.kind == SELECT_NM && g.lpr == 64 && RowsPer<NT>::v < 2) g.lpr = 32;  // whole 2:8 groups per workgroup
    if (a.mode == SFFN_LOPA) {
        const int r = S.rank;
        float *tvec = reinterpret_cast<float *>(ws + c.L.tvec);
        hipLaunchKernelGGL((k_lopa_xa<TW, NT>), dim3((r + 3) / 4), dim3(256), 0, st, x, n, d,
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

    // ---- Top-K / top-p: select, then the up rows ----
    if (ranked) {
        int2 *thr = reinterpret_cast<int2 *>(ws + c.L.thr);
        e = a.mode == SFFN_TOPK ? launch_topk_thr(gsel, n, F, a.k, thr, st)
                                : launch_topp_thr(gsel, n, F, a.tau, thr, st);
        if (e != hipSuccess) return e;
        const int lpr = lpr_for(d);
        const dim3 ugrid(row_blocks(F, lpr, RowsPer<NT>::v));
        if (lpr == 64)
            hipLaunchKernelGGL((k_up<TW, NT, 64>), ugrid, dim3(256), 0, st, x, n, d, wu, F, thr, act, any, gsel,
                               hbuf);
        else if (lpr == 32)
            hipLaunchKernelGGL((k_up<TW, NT, 32>), ugrid, dim3(256), 0, st, x, n, d, wu, F, thr, act, any, gsel,
                               hbuf);
        else
            hipLaunchKernelGGL((k_up<TW, NT, 16>), ugrid, dim3(256), 0, st, x, n, d, wu, F, thr, act, any, gsel,
                               hbuf);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }

    // ---- down projection: group partials and their ordered sum ----
    uint32_t *part = reinterpret_cast<uint32_t *>(ws + c.L.part);
    const int slices = (d + kDownSliceCols - 1) / kDownSliceCols;
    const int G = down_groups(c);
    hipLaunchKernelGGL((k_down<TW, NT, 8>), dim3(slices, G), dim3(256), down_lds(c), st, wdn, F, d, n, any,
                       dense ? 1 : 0, hbuf, part, a.y);
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
