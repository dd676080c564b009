// Row-dot engine of the decode (GEMV) kernels, shared by the gate kernel
// (gate.hip) and the Top-K up kernel (decode.hip).
#pragma once

#include "device_common.h"
#include "sffn_internal.h"

namespace sffn {

enum GateKind { KEYS = 0, SELECT_UP = 1, DENSE = 2, SELECT_NM = 3 };

// Rows of one 2:8 group: the SELECT_NM gate kernel needs whole groups in a
// workgroup (it ranks each group's keys through LDS).
constexpr int kNmGroup = 8, kNmKeep = 2;

// ---------------------------------------------------------------------------
// Row-dot engine. A lane group of LPR lanes owns R rows; lane li covers the
// 8-element chunks j = 8*li + s*8*LPR of every row. Each batch issues all its
// weight loads (128-bit, non-temporal: weights are read once per forward) and
// the matching x chunks of the NT tokens (small and cache-resident) before any
// arithmetic; rows whose bit is clear in `valid` are not read. Products
// accumulate in fp32 per lane (packed bf16 dot2 when both sides are bf16) and
// are summed over the lane group, so every lane of a group ends with all
// R x NT results.
// ---------------------------------------------------------------------------
template <typename TW, typename TX, int NT, int R, int LPR, int MAXS>
struct RowDot {
    static constexpr int STEP = LPR * 8;
    float acc[R][NT];

    // x: token t starts at x + t*ldx; tokens >= n read as zero.
    __device__ __forceinline__ void run(const TW *const rows[R], uint32_t valid, int len, int li, const TX *x,
                                        int ldx, int n)
    {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int t = 0; t < NT; ++t) acc[r][t] = 0.f;
        for (int jb = li * 8; jb < len; jb += MAXS * STEP) {
            typename Ld8<TW>::raw w[MAXS][R];
            typename Ld8<TX>::raw xv[MAXS][NT];
#pragma unroll
            for (int s = 0; s < MAXS; ++s)
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const int j = jb + s * STEP;
                    w[s][r] = (((valid >> r) & 1u) && j < len) ? Ld8<TW>::load_nt(rows[r] + j) : Ld8<TW>::zero();
                }
#pragma unroll
            for (int s = 0; s < MAXS; ++s)
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const int j = jb + s * STEP;
                    xv[s][t] = (t < n && j < len) ? Ld8<TX>::load(x + (size_t)t * ldx + j) : Ld8<TX>::zero();
                }
#pragma unroll
            for (int s = 0; s < MAXS; ++s)
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int t = 0; t < NT; ++t) acc[r][t] = dot8<TW, TX>(w[s][r], xv[s][t], acc[r][t]);
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int t = 0; t < NT; ++t) acc[r][t] = group_sum<LPR>(acc[r][t]);
    }
};

// Rows per lane group by token count: x chunks are reused over the rows.
template <int NT>
struct RowsPer {
    static constexpr int v = NT <= 2 ? 1 : NT / 2;
};

// Chunks per batch, keeping the weight and x registers of a batch near 96.
template <typename TW, typename TX, int NT, int R>
struct Batch {
    static constexpr int per = R * (sizeof(TW) == 2 ? 4 : 8) + NT * (sizeof(TX) == 2 ? 4 : 8);
    static constexpr int raw = 96 / per;
    static constexpr int v = raw >= 8 ? 8 : raw >= 4 ? 4 : raw >= 2 ? 2 : 1;
};

// Workgroups (4 wavefronts) for a row partition of `rows` rows in groups of
// R rows per LPR lanes.
inline int row_blocks(int rows, int lpr, int R)
{
    const int per_wave = (64 / lpr) * R;
    const int waves = (rows + per_wave - 1) / per_wave;
    return max(1, (waves + 3) / 4);
}

}  // namespace sffn
