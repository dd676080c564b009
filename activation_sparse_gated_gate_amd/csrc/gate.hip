// Gate kernel of the decode regime (1..8 tokens): gate GEMV fused with the
// activation, the threshold select and the up rows of the channels just found
// active ("Model Casting and Low-Parameter Gating", Abstract: the gate is
// computed first and only the channels it leaves active read their W_up and
// W_down rows). Launched through launch_gate (sffn_internal.h).
#include <hip/hip_ext.h>

#include <type_traits>

#include "rowdot.h"

namespace sffn {

// ---------------------------------------------------------------------------
// Gate kernel. Lane group q of wavefront gw (4 wavefronts per workgroup, LPR
// lanes per group) owns rows (gw * 64/LPR + q) * R .. + R-1: every wavefront
// gets the same small share, and there are many wavefronts per CU.
//   z = x . W_gate[i]   (or t . B[i] for LoPA, t = x.A in fp32)
//   KEYS:      g = SiLU(z) for the Top-K select that follows
//   SELECT_UP: active = z > tau, g = z - tau; then the group reads the W_up
//              rows of its channels that some token selected and writes
//              h[i][t] = g * (x_t . W_up[i]) for the selecting tokens, else 0
//   DENSE:     every channel; gate and up rows are read together,
//              g = max(z - tau, 0) or SiLU(z), h = g * u
//   SELECT_NM: g = SiLU(z); the workgroup's rows are whole aligned groups of
//              8 channels (LPR <= 32, or enough rows per lane group); the keys
//              go through LDS and each (channel, token) is ranked within its
//              group by (key descending, channel ascending); the 2 first are
//              active. Then as SELECT_UP: flags, union flag, up rows.
// h is stored channel-major, hbuf[i][t] (8 token slots per channel); SELECT_UP
// and SELECT_NM also write any[i], whether some token selected channel i.
// RG rows per lane group: RowsPer<NT> for long gate rows; 2 or 4 for short
// ones (LoPA's rows of B, 2048-wide layers), so that one wavefront per lane
// group's rows keeps the layer within the wavefronts the GPU holds at once
// and the kernel takes one memory round trip instead of two or three. Then
// each selected up row is read by the whole wavefront, one row at a time
// (ROWWISE_UP): at high sparsity a wavefront has none or one.
// ---------------------------------------------------------------------------
template <typename TW, typename TX, int NT, int LPR, int KIND, int RG>
__global__ __launch_bounds__(256) void k_gate(const TX *__restrict__ xg, int n, int L,
                                              const TW *__restrict__ xu, int d,
                                              const TW *__restrict__ wg, const TW *__restrict__ wu,
                                              int F, int mode, float tau,
                                              float *__restrict__ gsel, uint8_t *__restrict__ act,
                                              uint8_t *__restrict__ any, float *__restrict__ hbuf,
                                              float *__restrict__ debug_z, int *__restrict__ ctrl)
{
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        // this forward's epoch for the down projection's slots (never 0)
        uint32_t e = (uint32_t)__hip_atomic_load(ctrl + kCtrlEpoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
        __hip_atomic_store(ctrl + kCtrlEpoch, (int)(e == 0 ? 1u : e), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    constexpr int SUB = 64 / LPR;
    constexpr int R = RG;
    constexpr bool ROWWISE_UP = RG > RowsPer<NT>::v;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int q = lane / LPR, li = lane % LPR;
    const int row0 = ((blockIdx.x * 4 + wave) * SUB + q) * R;
    const int nv = max(0, min(R, F - row0));
    const uint32_t vmask = (1u << nv) - 1u;

    float zz[R][NT], uu[R][NT];
    if constexpr (KIND == DENSE) {
        const TW *rows[2 * R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            rows[r] = wg + (size_t)(row0 + r) * L;
            rows[R + r] = wu + (size_t)(row0 + r) * L;
        }
        RowDot<TW, TX, NT, 2 * R, LPR, Batch<TW, TX, NT, 2 * R>::v> dot;
        dot.run(rows, vmask | (vmask << R), L, li, xg, L, n);
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                zz[r][t] = dot.acc[r][t];
                uu[r][t] = dot.acc[R + r][t];
            }
    } else {
        const TW *rows[R];
#pragma unroll
        for (int r = 0; r < R; ++r) rows[r] = wg + (size_t)(row0 + r) * L;
        RowDot<TW, TX, NT, R, LPR, Batch<TW, TX, NT, R>::v> dot;
        dot.run(rows, vmask, L, li, xg, L, n);
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int t = 0; t < NT; ++t) zz[r][t] = dot.acc[r][t];
    }

    // ---- 2:8: every key of the workgroup's groups into LDS ----
    constexpr int WGROWS = 4 * SUB * R;  // rows of one workgroup, a multiple of 8 for SELECT_NM
    static_assert(KIND != SELECT_NM || WGROWS % kNmGroup == 0, "2:8 needs whole groups per workgroup");
    __shared__ float nm_keys[KIND == SELECT_NM ? WGROWS : 1][NT];
    const int wg_row0 = blockIdx.x * WGROWS;
    if constexpr (KIND == SELECT_NM) {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int t = 0; t < NT; ++t)
                if (li == ((r * NT + t) & (LPR - 1))) nm_keys[row0 + r - wg_row0][t] = silu(zz[r][t]);
        __syncthreads();
    }

    // ---- activation and selection (every lane of the group has every z) ----
    float gv[R][NT];      // gate value of a selected (row, token), else 0
    uint32_t amask = 0;   // rows some token selected
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int i = row0 + r;
            const float z = zz[r][t];
            float g;
            bool a;
            if constexpr (KIND == SELECT_UP) {
                a = z > tau;
                g = z - tau;
            } else if constexpr (KIND == SELECT_NM) {
                g = nm_keys[i - wg_row0][t];
                const int b = (i & ~(kNmGroup - 1)) - wg_row0;
                int rank = 0;
#pragma unroll
                for (int e = 0; e < kNmGroup; ++e) {
                    const float o = nm_keys[b + e][t];
                    const int j = wg_row0 + b + e;
                    rank += j < F && (o > g || (o == g && j < i));
                }
                a = rank < kNmKeep;
            } else if constexpr (KIND == KEYS) {
                a = false;
                g = silu(z);
            } else {
                a = true;
                g = mode == SFFN_DENSE ? fmaxf(z - tau, 0.f) : silu(z);
            }
            const bool live = r < nv && t < n;
            a = a && live;
            gv[r][t] = a ? g : 0.f;
            if (a) amask |= 1u << r;
            if (live && li == ((r * NT + t) & (LPR - 1))) {
                gsel[(size_t)t * F + i] = g;
                if (debug_z) debug_z[(size_t)t * F + i] = z;
                if constexpr (KIND == SELECT_UP || KIND == SELECT_NM) act[(size_t)t * F + i] = a ? 1 : 0;
                if constexpr (KIND == DENSE) hbuf[(size_t)i * kDecodeMaxTokens + t] = g * uu[r][t];
            }
        }
    if constexpr (KIND == SELECT_UP || KIND == SELECT_NM) {
#pragma unroll
        for (int r = 0; r < R; ++r)
            if (r < nv && li == (r & (LPR - 1))) any[row0 + r] = (amask >> r) & 1u;
        if (__ballot(amask != 0) == 0) return;  // nothing selected in this wavefront
        if constexpr (ROWWISE_UP) {
            // lane group q2's selected rows in turn, each by all 64 lanes (one
            // batch of loads for a row of up to 512 MAXS elements); group q2's
            // gate values come from its first lane
            for (int q2 = 0; q2 < SUB; ++q2) {
                const uint32_t qm = (uint32_t)__shfl((int)amask, q2 * LPR, 64);
                const int qrow0 = ((blockIdx.x * 4 + wave) * SUB + q2) * R;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    if (!((qm >> r) & 1u)) continue;  // the same in every lane
                    const TW *ur[1] = {wu + (size_t)(qrow0 + r) * d};
                    RowDot<TW, TW, NT, 1, 64, Batch<TW, TW, NT, 1>::v> up;
                    up.run(ur, 1u, d, lane, xu, d, n);
#pragma unroll
                    for (int t = 0; t < NT; ++t) {
                        const float gq = __shfl(gv[r][t], q2 * LPR, 64);
                        if (t < n && lane == t) hbuf[(size_t)(qrow0 + r) * kDecodeMaxTokens + t] = gq * up.acc[0][t];
                    }
                }
            }
            return;
        }
        const TW *urows[R];
#pragma unroll
        for (int r = 0; r < R; ++r) urows[r] = wu + (size_t)(row0 + r) * d;
        RowDot<TW, TW, NT, R, LPR, Batch<TW, TW, NT, R>::v> up;
        up.run(urows, amask, d, li, xu, d, n);
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int t = 0; t < NT; ++t)
                if (((amask >> r) & 1u) && t < n && li == ((r * NT + t) & (LPR - 1)))
                    hbuf[(size_t)(row0 + r) * kDecodeMaxTokens + t] = gv[r][t] * up.acc[r][t];
    }
}

// The gate kernel; with profiling events set, they take the kernel's own
// begin and end timestamps (hipExtLaunchKernelGGL), not separate markers.
template <typename TW, typename TX, int NT, int KIND, int RG>
static void launch_gate_k(hipStream_t st, hipEvent_t ev0, hipEvent_t ev1, int lpr, const TX *xg, int n, int L,
                        const TW *xu, int d, const TW *wg, const TW *wu, int F, int mode, float tau, float *gsel,
                        uint8_t *act, uint8_t *any, float *hbuf, float *dz, int *ctrl)
{
    const dim3 grid(row_blocks(F, lpr, RG));
#define SFFN_G(LP)                                                                                                   \
    do {                                                                                                             \
        if (ev0)                                                                                                     \
            hipExtLaunchKernelGGL((k_gate<TW, TX, NT, LP, KIND, RG>), grid, dim3(256), 0, st, ev0, ev1, 0, xg, n, L, \
                                  xu, d, wg, wu, F, mode, tau, gsel, act, any, hbuf, dz, ctrl);                     \
        else                                                                                                         \
            hipLaunchKernelGGL((k_gate<TW, TX, NT, LP, KIND, RG>), grid, dim3(256), 0, st, xg, n, L, xu, d, wg, wu,  \
                               F, mode, tau, gsel, act, any, hbuf, dz, ctrl);                                        \
    } while (0)
    // 2:8 needs whole groups of 8 rows per workgroup: 64 lanes per row only
    // with at least two rows per lane group (the host picks 32 otherwise)
    constexpr bool full64 = KIND != SELECT_NM || RG >= 2;
    if constexpr (full64) {
        if (lpr == 64) {
            SFFN_G(64);
            return;
        }
    }
    if constexpr (RG == RowsPer<NT>::v) {
        if (lpr == 16) {
            SFFN_G(16);
            return;
        }
    }
    SFFN_G(32);  // the host takes more rows per lane group only for lpr 32 and 64
#undef SFFN_G
}

// Rows per lane group of the gate kernel: more than RowsPer<NT> only for bf16
// gate rows of at most 4 KB at one or two tokens, and then the fewest (2 or
// 4) that keep the layer's wavefronts at or below 4096 (the GPU holds about
// 5000 of this kernel at once). Long rows stay at RowsPer<NT>: the kernel is
// bandwidth-bound there, and more rows per wavefront measured slower.
static int gate_rows_per_group(int dtype, int nt, int L, int F, int lpr)
{
    if (dtype != SFFN_BF16 || nt > 2 || L * 2 > 4096 || lpr < 32) return nt <= 2 ? 1 : nt / 2;
    const long long per_wave = 64 / lpr;
    for (int rg = 1; rg < 4; rg *= 2)
        if ((F + per_wave * rg - 1) / (per_wave * rg) <= 4096) return rg;
    return 4;
}

hipError_t launch_gate(const GateArgs &g)
{
    hipStream_t st = g.stream;
    hipEvent_t ev0 = static_cast<hipEvent_t>(g.ev_start), ev1 = static_cast<hipEvent_t>(g.ev_stop);
    const int rg = gate_rows_per_group(g.dtype, g.nt, g.L, g.F, g.lpr);
    auto run_rg = [&](auto tw, auto tx, auto nt, auto rg_c) {
        typedef decltype(tw) TW;
        typedef decltype(tx) TX;
        constexpr int NT = decltype(nt)::value, RG = decltype(rg_c)::value;
        const TX *xg = static_cast<const TX *>(g.xg);
        const TW *xu = static_cast<const TW *>(g.xu), *wg = static_cast<const TW *>(g.wg);
        const TW *wu = static_cast<const TW *>(g.wu);
        switch (g.kind) {
        case KEYS:
            launch_gate_k<TW, TX, NT, KEYS, RG>(st, ev0, ev1, g.lpr, xg, g.n, g.L, xu, g.d, wg, wu, g.F,
                                                g.mode, g.tau, g.gsel, g.act, g.any, g.hbuf, g.debug_z, g.ctrl);
            break;
        case DENSE:
            launch_gate_k<TW, TX, NT, DENSE, RG>(st, ev0, ev1, g.lpr, xg, g.n, g.L, xu, g.d, wg, wu, g.F,
                                                 g.mode, g.tau, g.gsel, g.act, g.any, g.hbuf, g.debug_z, g.ctrl);
            break;
        case SELECT_NM:
            if constexpr (std::is_same<TX, TW>::value)  // 2:8 takes the full gate
                launch_gate_k<TW, TX, NT, SELECT_NM, RG>(st, ev0, ev1, g.lpr, xg, g.n, g.L, xu, g.d, wg, wu, g.F,
                                                         g.mode, g.tau, g.gsel, g.act, g.any, g.hbuf, g.debug_z,
                                                         g.ctrl);
            break;
        default:
            launch_gate_k<TW, TX, NT, SELECT_UP, RG>(st, ev0, ev1, g.lpr, xg, g.n, g.L, xu, g.d, wg, wu, g.F,
                                                     g.mode, g.tau, g.gsel, g.act, g.any, g.hbuf, g.debug_z, g.ctrl);
            break;
        }
    };
    auto run = [&](auto tw, auto tx, auto nt) {
        constexpr int NT = decltype(nt)::value;
        if constexpr (NT <= 2 && sizeof(decltype(tw)) == 2) {  // short bf16 gate rows: 2 or 4 rows per lane group
            if (rg == 4) {
                run_rg(tw, tx, nt, std::integral_constant<int, 4>{});
                return;
            }
            if (rg == 2) {
                run_rg(tw, tx, nt, std::integral_constant<int, 2>{});
                return;
            }
        }
        run_rg(tw, tx, nt, std::integral_constant<int, RowsPer<NT>::v>{});
    };
    auto by_nt = [&](auto tw, auto tx) {
        switch (g.nt) {
        case 1: run(tw, tx, std::integral_constant<int, 1>{}); break;
        case 2: run(tw, tx, std::integral_constant<int, 2>{}); break;
        case 4: run(tw, tx, std::integral_constant<int, 4>{}); break;
        default: run(tw, tx, std::integral_constant<int, 8>{}); break;
        }
    };
    if (g.dtype == SFFN_BF16) {
        if (g.lopa) by_nt(bf16_t{}, float{});
        else by_nt(bf16_t{}, bf16_t{});
    } else {
        by_nt(float{}, float{});
    }
    return hipGetLastError();
}

}  // namespace sffn
