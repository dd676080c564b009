// Batched / prefill regime (more than 8 tokens): the union of the tokens'
// active channels, computed on bf16 MFMA.
//
//   1. gate GEMM   Z = X . W_gate^T (fp32 accumulate); epilogue: select from
//                  the fp32 value, store the gate value G (bf16, 0 when the
//                  channel is off for that token) and OR the union bitmap
//                  (Top-K: store the SiLU keys; each token's K-th key is
//                  found next and the flags follow from it; 2:8: store the
//                  keys, then each group of 8 keeps its 2 largest)
//   2. up GEMM     each workgroup reads the union bitmap and lists its own
//                  tile's part of the ascending union list U (writing it,
//                  and the union size, for what follows); Uu = X . W_up[U]^T
//                  over the gathered rows; epilogue
//                  H[t][j] = bf16(g[t][U[j]] * Uu[t][j])
//   3. down GEMM   Y = H . W_down[U, :] (rows gathered by U, fp32 output);
//                  it also clears the bitmap for the next forward
//
// Up to 64 tokens the up GEMM's tiles can instead run in the gate GEMM's
// launch over every channel (it does not depend on the gate): where the
// mode makes the union nearly every channel the down GEMM then runs over
// every channel too; otherwise, on a layer whose W_up streams in about one
// launch's fixed cost, the sum of the up partials keeps the union's channels
// in the union's order and the down GEMM runs over the union as above.
//
// A channel that no token selected reads neither W_up nor W_down: the gate is
// computed first and the other two matrices only for what it kept ("Model
// Casting and Low-Parameter Gating", Abstract; "Mixture-of-Channels" blog
// summary, "Dentro il 'mixture'"). Over a batch the kept set is the union of
// the tokens' sets; the selection itself is per token and taken from the fp32
// accumulator, never from a rounded value.
//
// GEMM tiles use v_mfma_f32_32x32x16_bf16 (operand lane l: row l%32, k
// 8*(l/32)..+7; accumulator register i: row 8*(i/4) + 4*(l/32) + i%4, column
// l%32). Tiles of A and B go straight from global memory to LDS through a
// ring of stages; the down projection's N-contiguous W_down rows are read
// out of LDS with transpose reads. When the grid would be too small, K is
// split and the fp32 partials are summed in order by a second kernel that
// applies the same epilogue.
#include <cmath>
#include <type_traits>

#include "compact.h"
#include "device_common.h"
#include "sffn_internal.h"

namespace sffn {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
typedef __attribute__((address_space(3))) bf16x4_t lbf16x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t_;



// Forward: gate, up, down. Backward (train.hip): BWD = the product
// dH = dY . W_down[U]^T with the gate derivative applied (dU, dZ and H, token
// major and transposed), DOWN_ACC = the down form adding into Y, WGRAD =
// C[m][n] added into row U[n] of a weight gradient (M = d_model).
enum EpiKind { EPI_GATE = 0, EPI_UP = 1, EPI_DOWN = 2, EPI_BWD = 3, EPI_DOWN_ACC = 4, EPI_WGRAD = 5 };

struct EpiArgs {
    int kind;
    int upart;          // gate or up GEMM in two launches (0: in one): 1 = the whole rounds of tiles, 2 = the rest
    int ncu, smax;      // (upart) compute units, and the most K splits of the rest
    int rest_u;         // (upart) N extent: the gate's d_ff; < 0: the union size, *ucount (up)
    int mode;           // sffn_mode (gate)
    float tau;
    int T, F, d;
    uint16_t *G;        // [T][F] bf16 gate values, 0 where off (gate or Top-K flags write, up reads)
    float *keys;        // [T][F] fp32 SiLU keys (Top-K gate writes)
    float *debug_z;     // [T][F] optional
    uint32_t *ubits;    // union bitmap (gate and Top-K flags set it, up reads it, down clears it)
    int32_t *uidx;      // union list (up writes, down and the split-K sum read)
    int *ucount;        // union size (up writes)
    int all_ch;         // up and down: every channel instead of the union (a small batch whose union is
                        // nearly every channel; G is 0 where off); the down GEMM's block 0 writes the
                        // bitmap's size to *utrue
    int *utrue;
    // gate GEMM with the up GEMM in the same launch (every channel, split K):
    // N tiles past the gate's read B2 (W_up) and write their partials to part2
    int dual;
    const bf16_t *B2;
    float *part2;
    // (gate split-K sum, every channel) the up half's partials [S][M][F]: the
    // sum also writes H = G u, the pad columns and the identity union list
    const float *up_part;
    uint16_t *H;        // [T][hld] bf16 (up writes)
    int hld;            // H row stride, d_ff rounded up to 8 (16-byte rows)
    float *Y;           // [T][d] fp32 (down writes; WGRAD: the gradient [F][d], added into)
    float *usave;       // optional [T][F] fp32: the up values x . W_up[i] (up writes, training forward)
    const int *tmap;    // optional: token of GEMM row m, for the rows of G the up epilogue reads and
                        // of Y the down epilogue writes (token groups: the products run in group order)
    // backward (EPI_BWD): mode is the derivative kind (0: g = z - tau,
    // g' = 1; 1: SiLU), ZU[t][i] the stored (z, u) of channel i (z NaN where
    // channel i is off for token t); writes dU into H and dZ into H2 (token
    // major, row stride hld) and dU, dZ, g(z) u transposed into DUT, DZT, HT
    // ([union position][token], row stride tp)
    const float2 *ZU;
    uint16_t *H2, *DUT, *DZT, *HT;
    int tp;
};

// Large gate and up GEMMs in two launches. One launch of BN-wide tiles over N
// columns can end with a round of tiles that few CUs work on (2048 prefill
// tokens of a 28672-channel layer: the gate's 896 tiles of 256 x 256 are 3.5
// rounds on 256 CUs; its union covering 38 % of the channels, the up GEMM's
// 344 tiles are 1.3 rounds). The first launch takes the N tiles of the whole
// rounds (ncu / MT N tiles of MT M tiles each, per round), the second the
// rest, its K split S ways so that rest x S tiles still fill the CUs (never
// more than ncu tiles: the partial buffer holds ncu tiles of BM x BN). The up
// GEMM's N, the union (U entries), is known only on the device: the split is
// taken there, from the union size.
struct RestSplit {
    int nfull, ntt, S;  // N tiles of the whole rounds, N tiles in all, K splits of the rest
};
__host__ __device__ inline RestSplit rest_split(int U, int BN, int MT, int ncu, int smax)
{
    const int ntt = (U + BN - 1) / BN;
    const int per = ncu / MT > 1 ? ncu / MT : 1;
    const int nfull = ntt / per * per;
    const int rest = (ntt - nfull) * MT;
    int S = rest > 0 ? ncu / rest : 1;
    S = S < 1 ? 1 : (S > smax ? smax : S);
    return {nfull, ntt, S};
}

// Backward values of one (token, channel) from the product v = dy . W_down[i]:
// du = v g(z), dz = v u g'(z), h = g(z) u; zero where the channel is off.
__device__ __forceinline__ void bwd_values(const EpiArgs &e, int m, int ch, float v, float &du, float &dz, float &h)
{
    du = dz = h = 0.f;
    const float2 zu = e.ZU[(size_t)m * e.F + ch];
    if (zu.x != zu.x) return;  // off
    float g, gp;
    if (e.mode == 0) {
        g = zu.x - e.tau;
        gp = 1.f;
    } else {
        const float sg = 1.f / (1.f + expf(-zu.x));
        g = zu.x * sg;
        gp = sg * (1.f + zu.x * (1.f - sg));
    }
    du = v * g;
    dz = v * zu.y * gp;
    h = g * zu.y;
}

// One output element. Returns the union bit for the gate (1 if the channel is
// kept for this token).
__device__ __forceinline__ bool epilogue(const EpiArgs &e, int m, int n, float v)
{
    if (e.kind == EPI_GATE) {
        const size_t o = (size_t)m * e.F + n;
        if (e.debug_z) e.debug_z[o] = v;
        if (e.mode == SFFN_TOPK || e.mode == SFFN_TOPK_2_8 || e.mode == SFFN_TOPP) {
            e.keys[o] = silu(v);
            return false;
        }
        if (e.mode == SFFN_THRESHOLD) {
            const bool a = v > e.tau;
            e.G[o] = a ? f2bf(v - e.tau) : (uint16_t)0;
            return a;
        }
        e.G[o] = f2bf(e.mode == SFFN_DENSE ? fmaxf(v - e.tau, 0.f) : silu(v));
        return true;
    }
    if (e.kind == EPI_UP) {
        const int i = e.all_ch ? n : e.uidx[n];
        const int tr = e.tmap ? e.tmap[m] : m;
        e.H[(size_t)m * e.hld + n] = f2bf(bf2f(e.G[(size_t)tr * e.F + i]) * v);
        if (e.usave) e.usave[(size_t)tr * e.F + i] = v;
        return false;
    }
    if (e.kind == EPI_BWD) {
        float du, dz, h;
        bwd_values(e, m, e.uidx[n], v, du, dz, h);
        e.H[(size_t)m * e.hld + n] = f2bf(du);
        e.H2[(size_t)m * e.hld + n] = f2bf(dz);
        const size_t o = (size_t)n * e.tp + m;
        e.DUT[o] = f2bf(du);
        e.DZT[o] = f2bf(dz);
        e.HT[o] = f2bf(h);
        return false;
    }
    if (e.kind == EPI_DOWN_ACC) {
        e.Y[(size_t)m * e.d + n] += v;
        return false;
    }
    if (e.kind == EPI_WGRAD) {
        e.Y[(size_t)e.uidx[n] * e.d + m] += v;
        return false;
    }
    e.Y[(size_t)(e.tmap ? e.tmap[m] : m) * e.d + n] = v;
    return false;
}

// ---------------------------------------------------------------------------
// Tile epilogue shared by the GEMM kernels. Element (i, j, r) of lane `lane`
// is row rowof(i, r), column colof(j) of the tile (MFMA accumulator layout).
// With S > 1 (split K) the fp32 tile goes to the partial buffer, element
// (m, n) at poff + (m - m0) part_ld + (n - n0); otherwise the
// epilogue kind EK (and for the gate the mode GM) is applied. Both are
// template parameters, and the branches sit outside the unrolled element
// loops, so the accumulators stay in registers.
// ---------------------------------------------------------------------------
template <int MF, int TM, int TN, int NTHR, int BN, int EK, int GM, typename AccT>
__device__ __forceinline__ void tile_epilogue(AccT (&acc)[TM][TN], int tid, int lane, int m0, int n0, int arow,
                                              int bcol, int M, int nlim, int S, float *__restrict__ part,
                                              size_t poff, int part_ld, const EpiArgs &epi, uint32_t *ubits_lds,
                                              const int *uloc)
{
    constexpr int ACC = MF == 32 ? 16 : 4;
    auto rowof = [&](int i, int r) {
        const int rr = MF == 32 ? (r / 4) * 8 + (lane / 32) * 4 + (r % 4) : (lane / 16) * 4 + r;
        return m0 + arow + i * MF + rr;
    };
    auto colof = [&](int j) { return n0 + bcol + j * MF + lane % MF; };
    if (S > 1) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int r = 0; r < ACC; ++r) {
                    const int m = rowof(i, r), n = colof(j);
                    if (m < M && n < nlim) part[poff + (size_t)(m - m0) * part_ld + (n - n0)] = acc[i][j][r];
                }
        return;
    }
    // tok(m): the token of GEMM row m. The row map (token groups) is tested
    // once here, so each element loop below is compiled for one case; a load
    // of the map inside the loop would also have to be repeated after every
    // store, which the compiler cannot prove it does not alias.
    auto with_rows = [&](auto &&body) {
        if (epi.tmap) {
            const int *__restrict__ tm = epi.tmap;
            body([tm](int m) { return tm[m]; });
        } else {
            body([](int m) { return m; });
        }
    };
    if constexpr (EK == EPI_DOWN || EK == EPI_DOWN_ACC) {
        with_rows([&](auto tok) {
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int n = colof(j);
                if (n >= nlim) continue;
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int r = 0; r < ACC; ++r) {
                        const int m = rowof(i, r);
                        if (m >= M) continue;
                        float *o = epi.Y + (size_t)tok(m) * epi.d + n;
                        if constexpr (EK == EPI_DOWN_ACC) *o += acc[i][j][r];
                        else *o = acc[i][j][r];
                    }
            }
        });
    } else if constexpr (EK == EPI_WGRAD) {
        // column n is union entry n: row U[n] of the gradient; rows m are
        // model dimensions, four consecutive ones per lane and register group
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int n = colof(j);
            if (n >= nlim) continue;
            float *row = epi.Y + (size_t)epi.uidx[n] * epi.d;
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int r = 0; r < ACC; ++r) {
                    const int m = rowof(i, r);
                    if (m < M) row[m] += acc[i][j][r];
                }
        }
    } else if constexpr (EK == EPI_BWD) {
        // rows m are tokens, column n union entry n (channel U[n]); pad
        // columns up to a multiple of 8 get zeros (the dx products read dU
        // and dZ in 8-wide chunks). Registers 4q .. 4q+3 of a lane hold four
        // consecutive tokens of one column (32 x 32 tiles): their transposed
        // values go out as one 8-byte store (tokens past M are zeros there,
        // inside the row's padding to tp, a multiple of 8).
        static_assert(MF == 32, "the packed transposed stores assume 32 x 32 tiles");
        const int padlim = (nlim + 7) & ~7;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int n = colof(j);
            if (n >= padlim) continue;
            const bool live = n < nlim;
            const int ch = live ? epi.uidx[n] : 0;
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int q = 0; q < ACC / 4; ++q) {
                    const int mb = rowof(i, 4 * q);  // multiple of 4
                    if (mb >= M) continue;
                    uint32_t pu[2] = {0u, 0u}, pz[2] = {0u, 0u}, ph[2] = {0u, 0u};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int m = mb + e;
                        float du = 0.f, dz = 0.f, h = 0.f;
                        if (live && m < M) bwd_values(epi, m, ch, acc[i][j][4 * q + e], du, dz, h);
                        const uint16_t bu = f2bf(du), bz = f2bf(dz), bh = f2bf(h);
                        if (m < M) {
                            epi.H[(size_t)m * epi.hld + n] = bu;
                            epi.H2[(size_t)m * epi.hld + n] = bz;
                        }
                        pu[e / 2] |= (uint32_t)bu << (16 * (e & 1));
                        pz[e / 2] |= (uint32_t)bz << (16 * (e & 1));
                        ph[e / 2] |= (uint32_t)bh << (16 * (e & 1));
                    }
                    if (live) {
                        const size_t o = (size_t)n * epi.tp + mb;
                        *reinterpret_cast<uint2 *>(epi.DUT + o) = make_uint2(pu[0], pu[1]);
                        *reinterpret_cast<uint2 *>(epi.DZT + o) = make_uint2(pz[0], pz[1]);
                        *reinterpret_cast<uint2 *>(epi.HT + o) = make_uint2(ph[0], ph[1]);
                    }
                }
            __builtin_amdgcn_sched_barrier(0);
        }
    } else if constexpr (EK == EPI_UP) {
        const int padlim = (nlim + 7) & ~7;
        with_rows([&](auto tok) {
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int n = colof(j);
                if (n >= padlim) continue;
                const bool live = n < nlim;
                const int src = live ? uloc[n - n0] : 0;  // this tile's part of the union list (LDS)
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int r = 0; r < ACC; ++r) {
                        const int m = rowof(i, r);
                        if (m >= M) continue;
                        uint16_t h = 0;  // pad columns: the down GEMM reads H in 8-wide chunks
                        if (live) {
                            const int tr = tok(m);
                            h = f2bf(bf2f(epi.G[(size_t)tr * epi.F + src]) * acc[i][j][r]);
                            if (epi.usave) epi.usave[(size_t)tr * epi.F + src] = acc[i][j][r];
                        }
                        epi.H[(size_t)m * epi.hld + n] = h;
                    }
                // keep each sub-tile's gathered G loads from being hoisted over
                // the whole tile (register pressure)
                __builtin_amdgcn_sched_barrier(0);
            }
        });
    } else {
        // gate; GM is the mode, a template parameter so each instantiation
        // carries one straight-line epilogue
        const float tau = epi.tau;
        float *dz = epi.debug_z;
        if constexpr (GM == SFFN_THRESHOLD) {
            for (int w = tid; w < BN / 32; w += NTHR) ubits_lds[w] = 0;
            __syncthreads();
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int n = colof(j);
            if (n >= nlim) continue;
            bool any = false;
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int r = 0; r < ACC; ++r) {
                    const int m = rowof(i, r);
                    if (m >= M) continue;
                    const float v = acc[i][j][r];
                    const size_t o = (size_t)m * epi.F + n;
                    if (dz) dz[o] = v;
                    if constexpr (GM == SFFN_THRESHOLD) {
                        const bool a = v > tau;
                        epi.G[o] = a ? f2bf(v - tau) : (uint16_t)0;
                        any |= a;
                    } else if constexpr (GM == SFFN_TOPK) {
                        epi.keys[o] = silu(v);
                    } else if constexpr (GM == SFFN_DENSE) {
                        epi.G[o] = f2bf(fmaxf(v - tau, 0.f));
                    } else {
                        epi.G[o] = f2bf(silu(v));
                    }
                }
            if constexpr (GM == SFFN_THRESHOLD)
                if (any) atomicOr(&ubits_lds[(bcol + j * MF + lane % MF) / 32], 1u << (n & 31));
        }
        if constexpr (GM == SFFN_THRESHOLD) {
            __syncthreads();
            for (int w = tid; w < BN / 32; w += NTHR)
                if (ubits_lds[w]) atomicOr(&epi.ubits[n0 / 32 + w], ubits_lds[w]);
        }
    }
}


// ---------------------------------------------------------------------------
// GEMM C[M x N] = A[M x K] . B on v_mfma_f32_32x32x16_bf16, A row-major (K
// contiguous, leading dim lda):
//   BNN = false (gate, up): B rows are the N outputs, K contiguous, gathered
//                through bidx (or identity); N limited by *ncount if set.
//   BNN = true  (down):     B rows are the K inputs, N contiguous, gathered
//                through bidx; K limited by *ncount.
// Rows m < M. Split-K: blockIdx.z takes K range [klim z / S, klim (z+1) / S)
// rounded to the K step; with S > 1 the fp32 tile goes to part[z][m][n].
//
// Tiles move from global memory straight into LDS (direct-to-LDS loads, no
// register staging) through a ring of three stages, so the loads of K steps
// i+1 and i+2 are in flight while step i is multiplied. Each stage is its
// own LDS array and the stage index is a compile-time constant (the main
// loop is unrolled by three): the compiler can then tell the stages apart
// and does not wait for every outstanding load before each LDS read; the
// only waits are the explicit ones below (it tells at most eight such
// targets apart, so A and B of a stage share one array).
//
// LDS serves a 128-bit read 16 lanes at a time, from a 256-byte bank window
// (two 128-byte tile rows). K-contiguous tiles (A; B when BNN = false): one
// 16-byte load instruction of a wavefront fills 8 tile rows (1 KB); lane l
// writes slot l%8 of row l/8, loading the K chunk that belongs there: row r
// keeps chunk p at slot p ^ ((r >> 1) & 7). A fragment read (32 rows, one
// chunk) then puts each 16 consecutive rows on 16 distinct bank slots.
//
// N-contiguous B (BNN = true): one instruction fills 64/CPR K rows of CPR =
// BN/8 chunks; K row r holds N chunk p at slot p ^ nswz(r). A fragment (8
// consecutive K values of one column per lane) is two LDS transpose reads;
// 32 lanes of such a read cover 4 K rows x 64 bytes, and the swizzle puts
// those 16 pieces on distinct bank slots.
// The gathered row indices of K step s travel with the loads of step s-2
// (one 4-byte load per lane into a three-slot LDS ring), so they are in LDS
// when step s's loads are issued.
//
// Chunks outside the operands (rows past M or past the union, K past the
// end) are loaded from a zero block.
// ---------------------------------------------------------------------------

// Source of the chunks outside the operands; never written.
static __device__ __align__(16) uint4 g_zero16[1] = {};

template <int TM, int TN, int WM, int WN, int BKT, int NS, int OCC, bool BNN, int EK, int GM>
__global__ __launch_bounds__(64 * WM *WN, OCC) void k_mfma_dma(int M, int N, int K, const bf16_t *__restrict__ A,
                                                              int lda,
                                                         const bf16_t *__restrict__ B, int ldb,
                                                         const int32_t *__restrict__ bidx,
                                                         const int *__restrict__ ncount, float *__restrict__ part,
                                                         int part_ld, EpiArgs epi)
{
    constexpr int MF = 32, NW = WM * WN, NTHR = 64 * NW;
    constexpr int BM = MF * TM * WM, BN = MF * TN * WN, BK = BKT;
    static_assert(BK == 64 || (BK == 32 && !BNN), "K step 64, or 32 for the K-contiguous form");
    static_assert(NS == 2 || NS == 3 || (NS == 4 && !BNN), "two or three stages, or four for the K-contiguous form");
    constexpr int CH = BK / 8;                      // K chunks per tile row
    constexpr int SWS = BK == 64 ? 1 : 2;           // log2(tile rows per 256-byte bank window)
    constexpr int CPR = BN / 8, RPI = 64 / CPR;     // BNN: chunks per K row, K rows per instruction
    constexpr int APW = BM * (BK / 8) / 64 / NW;    // 16-byte load instructions per wavefront and stage: A
    constexpr int BPW = BN * (BK / 8) / 64 / NW;    // and B
    constexpr int LPS = APW + BPW + (BNN ? 1 : 0);  // vector-memory operations per wavefront and stage
    static_assert(APW * 64 * NW == BM * (BK / 8) && BPW * 64 * NW == BN * (BK / 8), "rows split over wavefronts");
    static_assert(!BNN || (CPR <= 64 && BPW * RPI * NW == BK), "K rows split over wavefronts");
    typedef __attribute__((ext_vector_type(16))) float accv;
    // stage s: A tile at 0, B tile at BM * BK (one array per stage: the
    // compiler tells at most eight direct-to-LDS targets apart)
    __shared__ __align__(16) bf16_t St0[(BM + BN) * BK], St1[(BM + BN) * BK], St2[NS > 2 ? (BM + BN) * BK : 8],
        St3[NS > 3 ? (BM + BN) * BK : 8];
    __shared__ __align__(16) int Is0[BNN ? BK : 1], Is1[BNN ? BK : 1], Is2[BNN && NS == 3 ? BK : 1];
    __shared__ uint32_t ubits_lds[BN / 32];
    __shared__ int uloc[EK == EPI_UP ? BN : 1];  // up: union entries n0 .. n0 + BN - 1
    __shared__ int utot;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    // XCD-aware tile order: the M tiles of one N tile run on one XCD
    const int MT = (M + BM - 1) / BM, NTT = (N + BN - 1) / BN;
    int mi, ni, z = blockIdx.z, S = gridDim.z, tile_p = -1;
    if ((EK == EPI_UP || EK == EPI_GATE) && epi.upart == 2) {
        // the rest after the whole rounds (the union size comes from the up
        // GEMM's first launch): list position p = (split, N tile, M tile),
        // dealt to the XCDs in contiguous runs (a run shares weight rows)
        const RestSplit u = rest_split(epi.rest_u >= 0 ? epi.rest_u : *epi.ucount, BN, MT, epi.ncu, epi.smax);
        const int tiles = (u.ntt - u.nfull) * MT, len = tiles * u.S, run = (len + 7) / 8;
        const int slot = blockIdx.x / 8, p = (blockIdx.x % 8) * run + slot;
        if (slot >= run || p >= len) return;
        z = p / tiles;
        S = u.S;
        mi = (p % tiles) % MT;
        ni = u.nfull + (p % tiles) / MT;
        tile_p = p;
    } else {
        const int xcd = blockIdx.x % 8, jt = blockIdx.x / 8;
        mi = jt % MT;
        ni = (jt / MT) * 8 + xcd;
        if (ni >= (EK == EPI_GATE && epi.dual ? 2 : 1) * NTT) return;
        if (EK == EPI_GATE && epi.dual && ni >= NTT) {
            // an up tile of the gate launch
            ni -= NTT;
            B = epi.B2;
            part = epi.part2;
        }
    }
    const int m0 = mi * BM, n0 = ni * BN;
    int nlim = N, klim = K;
    if constexpr (EK == EPI_UP) {
        // The union list, ascending: entry e is the e-th set bit of the
        // bitmap (every channel in the dense modes). Wavefront 0 holds words
        // w0 + 64 q + lane (up to 16 per lane in one batch of loads). First
        // the total, so that tiles past the union leave at once; then round
        // q by round q a wavefront scan of the popcounts plus the carry of
        // the earlier rounds gives each word's first entry, and the lanes
        // whose word meets entries [n0, n0 + BN) extract its bits (a tile's
        // words lie on different lanes, so in parallel), up to the round
        // that passes the tile.
        const int F = epi.F, W = (F + 31) / 32;
        if (epi.mode == SFFN_DENSE || epi.mode == SFFN_DENSE_SILU || epi.all_ch) {
            for (int j = tid; j < BN; j += 64 * WM * WN) uloc[j] = n0 + j;
            if (tid == 0) utot = F;
        } else if (wave == 0) {
            const uint32_t *ub = epi.ubits;
            uint32_t u[16];
            auto load = [&](int w0) {
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    const int w = w0 + 64 * q + lane;
                    u[q] = w < W ? ub[w] : 0u;
                }
            };
            load(0);
            int tot = 0;
            for (int w0 = 0;;) {
                int c = 0;
#pragma unroll
                for (int q = 0; q < 16; ++q) c += __popc(u[q]);
#pragma unroll
                for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o, 64);
                tot += c;
                w0 += 1024;
                if (w0 >= W) break;
                load(w0);
            }
            if (lane == 0) utot = tot;
            if (n0 < tot) {
                int carry = 0;
                for (int w0 = 0; w0 < W && carry < n0 + BN; w0 += 1024) {
                    if (W > 1024) load(w0);  // one batch: still in registers
#pragma unroll
                    for (int q = 0; q < 16; ++q) {
                        if (w0 + 64 * q >= W || carry >= n0 + BN) break;
                        const int pc = __popc(u[q]);
                        const int incl = wave_incl_scan(pc);
                        int rank = carry + incl - pc;
                        if (rank < n0 + BN && rank + pc > n0) {
                            const int w = w0 + 64 * q + lane;
                            uint32_t v = u[q];
                            while (v) {
                                const int b = __ffs(v) - 1;
                                v &= v - 1;
                                if (rank >= n0 && rank < n0 + BN) uloc[rank - n0] = w * 32 + b;
                                ++rank;
                            }
                        }
                        carry += __shfl(incl, 63, 64);
                    }
                }
            }
        }
        __syncthreads();
        nlim = min(N, utot);
        if (epi.upart == 1) nlim = min(nlim, rest_split(utot, BN, MT, epi.ncu, epi.smax).nfull * BN);
        // one workgroup per N tile publishes its part; the first, the size
        if (z == 0 && mi == 0) {
            for (int j = tid; j < BN && n0 + j < nlim; j += 64 * WM * WN) epi.uidx[n0 + j] = uloc[j];
            if (n0 == 0 && tid == 0 && epi.upart != 2) *epi.ucount = utot;
        }
    } else if (ncount) {
        if constexpr (BNN) klim = min(K, *ncount);
        else nlim = min(N, *ncount);
    }
    if constexpr (EK == EPI_DOWN) {
        // the up GEMM has read the bitmap: clear it for the next forward (over
        // every channel, the union's own size for the caller is counted first)
        if (blockIdx.x == 0 && blockIdx.z == 0) {
            const int W = (epi.F + 31) / 32;
            if (epi.all_ch) {
                if (wave == 0) {
                    int c = 0;
                    for (int w = lane; w < W; w += 64) {
                        c += __popc(epi.ubits[w]);
                        epi.ubits[w] = 0;
                    }
#pragma unroll
                    for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o, 64);
                    if (lane == 0) *epi.utrue = c;
                }
            } else {
                for (int w = tid; w < W; w += 64 * WM * WN) epi.ubits[w] = 0;
            }
        }
    }
    if (n0 >= nlim || m0 >= M) return;
    int kb = 0, ke = klim;
    if (S > 1) {
        const int steps = (klim + BK - 1) / BK;
        kb = (int)(((long long)steps * z) / S) * BK;
        ke = min(klim, (int)(((long long)steps * (z + 1)) / S) * BK);
    }
    // split K: this tile's partials (the up GEMM's rest: tile p at [p][BM][BN])
    const size_t poff = tile_p >= 0 ? (size_t)tile_p * BM * BN : ((size_t)z * M + m0) * part_ld + n0;
    const int pld = tile_p >= 0 ? BN : part_ld;
    const int nsteps = ke > kb ? (ke - kb + BK - 1) / BK : 0;
    const bf16_t *zero = reinterpret_cast<const bf16_t *>(g_zero16);
    // BNN: K row r keeps N chunk p at slot p ^ nswz(r)
    auto nswz = [](int r) { return CPR >= 16 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); };

    // ---- per-lane sources ----
    // K-major tiles: tile row r keeps K chunk p at slot p ^ ((r >> SWS) & (CH - 1))
    const int lr = lane / CH;
    auto kchunk = [&](int row) { return ((lane % CH) ^ ((row >> SWS) & (CH - 1))) * 8; };
    const bf16_t *asrc[APW];
    int alc[APW];
#pragma unroll
    for (int j = 0; j < APW; ++j) {
        const int r = (wave * APW + j) * (64 / CH) + lr, m = m0 + r;
        alc[j] = kchunk(r);
        asrc[j] = m < M ? A + (size_t)m * lda + alc[j] : nullptr;
    }
    const bf16_t *bsrc[BNN ? 1 : BPW];
    int blc[BNN ? 1 : BPW];
    int bkr[BNN ? BPW : 1];  // BNN: local K row of each B instruction
    int bnc[BNN ? BPW : 1];  // and the first column of the chunk this lane loads into it
    if constexpr (!BNN) {
#pragma unroll
        for (int j = 0; j < BPW; ++j) {
            const int r = (wave * BPW + j) * (64 / CH) + lr, n = n0 + r;
            blc[j] = kchunk(r);
            const int row = EK == EPI_UP ? uloc[r] : (bidx && n < nlim) ? bidx[n] : n;
            bsrc[j] = n < nlim ? B + (size_t)row * ldb + blc[j] : nullptr;
        }
    } else {
#pragma unroll
        for (int j = 0; j < BPW; ++j) {
            bkr[j] = (wave * BPW + j) * RPI + lane / CPR;
            bnc[j] = n0 + ((lane % CPR) ^ nswz(bkr[j])) * 8;
        }
    }

    auto As = [&](auto stage) -> bf16_t * {
        constexpr int SI = decltype(stage)::value;
        return SI == 0 ? St0 : SI == 1 ? St1 : SI == 2 ? St2 : St3;
    };
    auto Bs = [&](auto stage) -> bf16_t * { return As(stage) + BM * BK; };
    auto Is = [&](auto stage) -> int * {
        constexpr int SI = decltype(stage)::value;
        return SI == 0 ? Is0 : SI == 1 ? Is1 : Is2;
    };
    // BNN: the row indices of K step `step` into index slot `stage`
    auto issue_idx = [&](auto stage, int step) {
        const int k = kb + step * BK + lane;
        const int32_t *src = k < ke ? bidx + k : reinterpret_cast<const int32_t *>(g_zero16);
        __builtin_amdgcn_global_load_lds((gmem_t *)src, (lmem_t *)Is(stage), 4, 0, 0);
    };
    // the tiles of K step `step` into stage `stage`; BNN: their row indices
    // are in index slot `stage`
    auto issue = [&](auto stage, int step) {
        bf16_t *la = As(stage), *lb = Bs(stage);
        const int k = kb + step * BK;
#pragma unroll
        for (int j = 0; j < APW; ++j) {
            const bf16_t *src = (asrc[j] && k + alc[j] < ke) ? asrc[j] + k : zero;
            __builtin_amdgcn_global_load_lds((gmem_t *)src, (lmem_t *)(la + (wave * APW + j) * 512), 16, 0, 0);
        }
        if constexpr (!BNN) {
#pragma unroll
            for (int j = 0; j < BPW; ++j) {
                const bf16_t *src = (bsrc[j] && k + blc[j] < ke) ? bsrc[j] + k : zero;
                __builtin_amdgcn_global_load_lds((gmem_t *)src, (lmem_t *)(lb + (wave * BPW + j) * 512), 16, 0, 0);
            }
        } else {
            const int *is = Is(stage);
#pragma unroll
            for (int j = 0; j < BPW; ++j) {
                const bool ok = k + bkr[j] < ke && bnc[j] < nlim;
                const bf16_t *src = ok ? B + (size_t)is[bkr[j]] * ldb + bnc[j] : zero;
                __builtin_amdgcn_global_load_lds((gmem_t *)src, (lmem_t *)(lb + (wave * BPW + j) * 512), 16, 0, 0);
            }
        }
    };

    accv acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int arow = wm * MF * TM, bcol = wn * MF * TN;
    // BNN: element offsets (K substep 0) of this lane's two transpose reads
    // per B fragment. ds_read_b64_tr_b16: in each group of 16 lanes, lane
    // 4a+b receives element b of the 8-byte reads of lanes 4e+a, e = 0..3.
    // Lane s therefore points at K row 8 (s/32) + 4 half + (s%16)/4, columns
    // 16 ((s/16)%2) + 4 (s%4) .. +3 of its fragment; lane l then holds
    // K values 8 (l/32) + 4 half + 0..3 of column l%32, the operand layout.
    int btr[BNN ? TN : 1][2];
    if constexpr (BNN) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int kr = 8 * (lane >> 5) + 4 * h + ((lane & 15) >> 2);
                const int n = bcol + j * MF + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
                btr[j][h] = kr * BN + ((((n >> 3) ^ nswz(kr)) << 3) | (n & 7));
            }
    }
    // Fragments of K substep ks of a stage.
    auto frags = [&](const bf16_t *sa, const bf16_t *sb, int ks, bf16x8_t (&af)[TM], bf16x8_t (&bfr)[TN]) {
        const int sw = ((2 * ks + (lane >> 5)) ^ (((lane & 31) >> SWS) & (CH - 1))) * 8;
#pragma unroll
        for (int i = 0; i < TM; ++i)
            af[i] = *reinterpret_cast<const bf16x8_t *>(sa + (arow + i * MF + (lane & 31)) * BK + sw);
        if constexpr (!BNN) {
#pragma unroll
            for (int j = 0; j < TN; ++j)
                bfr[j] = *reinterpret_cast<const bf16x8_t *>(sb + (bcol + j * MF + (lane & 31)) * BK + sw);
        } else {
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lbf16x4_t *)(sb + ks * 16 * BN + btr[j][0]));
                const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lbf16x4_t *)(sb + ks * 16 * BN + btr[j][1]));
                bfr[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            }
        }
    };
    auto mma = [&](const bf16x8_t (&af)[TM], const bf16x8_t (&bfr)[TN]) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    };
    // The fragments of substep ks+1 are read while substep ks is multiplied
    // (two register sets), so LDS latency hides behind the MFMAs.
    auto compute = [&](auto stage) {
        const bf16_t *sa = As(stage), *sb = Bs(stage);
        if constexpr (OCC > 1 || BK / 16 < 2) {
            // two workgroups per CU: the other one's wavefronts hide LDS
            // latency, and one fragment set keeps the registers within half
#pragma unroll
            for (int ks = 0; ks < BK / 16; ++ks) {
                bf16x8_t a0[TM], b0[TN];
                frags(sa, sb, ks, a0, b0);
                mma(a0, b0);
            }
        } else {
            bf16x8_t a0[TM], b0[TN], a1[TM], b1[TN];
            frags(sa, sb, 0, a0, b0);
#pragma unroll
            for (int ks = 0; ks < BK / 16; ks += 2) {
                frags(sa, sb, ks + 1, a1, b1);
                mma(a0, b0);
                if (ks + 2 < BK / 16) frags(sa, sb, ks + 2, a0, b0);
                mma(a1, b1);
            }
        }
    };
    // K step i: its loads (issued NS-1 steps earlier) have landed in every
    // wavefront once each has waited for all but the later steps' groups of
    // loads and passed the barrier; the barrier also ends every read of the
    // stage (and index slot) that this step refills, last read in step i-1.
    // Every step issues and waits the same way: the step count is padded to
    // a multiple of three, and steps past the end load the zero block, so
    // every path through the loop has the same loads in flight.
    auto step = [&](auto stage, int i) {
        constexpr int SI = decltype(stage)::value;
        wait_vm_lgkm<LPS * (NS - 2)>();
        __builtin_amdgcn_s_barrier();
        issue(std::integral_constant<int, (SI + NS - 1) % NS>{}, i + NS - 1);
        if constexpr (BNN) {
            // three stages: indices two groups ahead of their tiles (slot
            // (i+4) % 3, last read in step i-1); two stages: one group ahead
            // (slot (i+2) % 2, last read before this step's barrier)
            if constexpr (NS == 3) issue_idx(std::integral_constant<int, (SI + 1) % 3>{}, i + 4);
            else issue_idx(std::integral_constant<int, SI>{}, i + 2);
        }
        compute(stage);
    };
    if constexpr (BNN && NS == 3) {
        // indices of steps 0..2, then the tiles of steps 0 and 1 with the
        // indices of step 3 (slot 0, after every wavefront has read step 0's)
        issue_idx(std::integral_constant<int, 0>{}, 0);
        issue_idx(std::integral_constant<int, 1>{}, 1);
        issue_idx(std::integral_constant<int, 2>{}, 2);
        wait_vm_lgkm<0>();
        issue(std::integral_constant<int, 0>{}, 0);
        issue(std::integral_constant<int, 1>{}, 1);
        wait_vm_lgkm<2 * (APW + BPW)>();  // no vector-memory wait: only the index reads above
        __builtin_amdgcn_s_barrier();
        issue_idx(std::integral_constant<int, 0>{}, 3);
    } else if constexpr (BNN) {
        // indices of steps 0 and 1, then the tiles of step 0 (each step then
        // waits for everything in flight)
        issue_idx(std::integral_constant<int, 0>{}, 0);
        issue_idx(std::integral_constant<int, 1>{}, 1);
        wait_vm_lgkm<0>();
        issue(std::integral_constant<int, 0>{}, 0);
    } else {
        issue(std::integral_constant<int, 0>{}, 0);
        if constexpr (NS > 2) issue(std::integral_constant<int, 1>{}, 1);
        if constexpr (NS > 3) issue(std::integral_constant<int, 2>{}, 2);
    }
    const int nstp = (nsteps + NS - 1) / NS * NS;
    for (int i = 0; i < nstp; i += NS) {
        step(std::integral_constant<int, 0>{}, i);
        step(std::integral_constant<int, 1>{}, i + 1);
        if constexpr (NS > 2) step(std::integral_constant<int, 2>{}, i + 2);
        if constexpr (NS > 3) step(std::integral_constant<int, 3>{}, i + 3);
    }
    wait_vm_lgkm<0>();  // the trailing (zero) loads land before the LDS is given up
    tile_epilogue<MF, TM, TN, NTHR, BN, EK, GM>(acc, tid, lane, m0, n0, arow, bcol, M, nlim, S, part, poff, pld,
                                                epi, ubits_lds, uloc);
}

// Sum of the rest launch's split partials (tile p at part[p][BM][BN]) in
// split order, with the gate or up epilogue (gate: also the union bits; up:
// zeros in the pad columns up to a multiple of 8). Its extent and split
// count follow from the N extent as in the GEMM; with one split the GEMM has
// applied the epilogue itself. BN = 256: a lane takes 4 columns of a tile
// row, a wavefront 4 rows (their loads in flight together), a workgroup
// step 16 rows of one tile; the union bits of a step go out as one atomic
// per word.
template <int EK>
__global__ __launch_bounds__(256) void k_rest_sum(const float *__restrict__ part, int M, int BM, int BN, EpiArgs epi)
{
    constexpr int RW = 4, RB = 4 * RW;
    __shared__ uint32_t ub[4][8];
    const int U = epi.rest_u >= 0 ? epi.rest_u : *epi.ucount, MT = (M + BM - 1) / BM;
    const RestSplit u = rest_split(U, BN, MT, epi.ncu, epi.smax);
    if (u.S < 2) return;
    const int tiles = (u.ntt - u.nfull) * MT, padlim = EK == EPI_UP ? (U + 7) & ~7 : U;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const bool bits = EK == EPI_GATE && epi.mode == SFFN_THRESHOLD;
    const size_t zs = (size_t)tiles * BM * BN;
    for (int r0 = blockIdx.x * RB; r0 < tiles * BM; r0 += gridDim.x * RB) {
        const int t = r0 / BM, rb = r0 % BM + wv * RW;  // BM is a multiple of RB: one tile
        const int n = (u.nfull + t / MT) * BN + 4 * lane, mb = (t % MT) * BM + rb;
        const float *src = part + ((size_t)t * BM + rb) * BN + 4 * lane;
        float4 p[RW][4];
#pragma unroll
        for (int i = 0; i < RW; ++i)
#pragma unroll
            for (int s = 0; s < 4; ++s)
                if (s < u.S) p[i][s] = *reinterpret_cast<const float4 *>(src + (size_t)i * BN + zs * s);
        uint32_t b = 0;
        // the gate's four columns with one vector store per output (d_ff a
        // multiple of 4, all four inside it)
        const bool vec = EK == EPI_GATE && (epi.F & 3) == 0 && n + 3 < U;
#pragma unroll
        for (int i = 0; i < RW; ++i) {
            const int m = mb + i;
            if (m >= M || n >= padlim) continue;
            float v[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s)
                if (s < u.S) {
                    v[0] += p[i][s].x;
                    v[1] += p[i][s].y;
                    v[2] += p[i][s].z;
                    v[3] += p[i][s].w;
                }
            if constexpr (EK == EPI_UP) {
                // four bf16 of H in one 8-byte store (n and the row stride are multiples of 4)
                const int tr = epi.tmap ? epi.tmap[m] : m;
                uint16_t h[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    h[c] = 0;
                    if (n + c < U) {
                        const int ch = epi.uidx[n + c];
                        h[c] = f2bf(bf2f(epi.G[(size_t)tr * epi.F + ch]) * v[c]);
                        if (epi.usave) epi.usave[(size_t)tr * epi.F + ch] = v[c];
                    }
                }
                *reinterpret_cast<uint2 *>(epi.H + (size_t)m * epi.hld + n) =
                    make_uint2(h[0] | (uint32_t)h[1] << 16, h[2] | (uint32_t)h[3] << 16);
            } else if (vec) {
                const size_t o = (size_t)m * epi.F + n;
                if (epi.debug_z) *reinterpret_cast<float4 *>(epi.debug_z + o) = make_float4(v[0], v[1], v[2], v[3]);
                if (epi.mode == SFFN_TOPK || epi.mode == SFFN_TOPK_2_8 || epi.mode == SFFN_TOPP) {
                    *reinterpret_cast<float4 *>(epi.keys + o) = make_float4(silu(v[0]), silu(v[1]), silu(v[2]), silu(v[3]));
                } else {
                    uint16_t g[4];
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        if (epi.mode == SFFN_THRESHOLD) {
                            const bool a = v[c] > epi.tau;
                            g[c] = a ? f2bf(v[c] - epi.tau) : (uint16_t)0;
                            b |= (uint32_t)a << c;
                        } else {
                            g[c] = f2bf(epi.mode == SFFN_DENSE ? fmaxf(v[c] - epi.tau, 0.f) : silu(v[c]));
                        }
                    }
                    *reinterpret_cast<uint2 *>(epi.G + o) =
                        make_uint2(g[0] | (uint32_t)g[1] << 16, g[2] | (uint32_t)g[3] << 16);
                }
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    if (n + c < U && epilogue(epi, m, n + c, v[c])) b |= 1u << c;
            }
        }
        if (bits) {
            // word k of the tile's 256 columns: lanes 8k .. 8k+7, 4 bits each
            uint32_t w = b << (4 * (lane & 7));
            w |= __shfl_xor(w, 1, 64);
            w |= __shfl_xor(w, 2, 64);
            w |= __shfl_xor(w, 4, 64);
            if ((lane & 7) == 0) ub[wv][lane >> 3] = w;
            __syncthreads();
            if (threadIdx.x < 8) {
                const uint32_t o = ub[0][threadIdx.x] | ub[1][threadIdx.x] | ub[2][threadIdx.x] | ub[3][threadIdx.x];
                if (o) atomicOr(&epi.ubits[((u.nfull + t / MT) * BN) / 32 + threadIdx.x], o);
            }
            __syncthreads();
        }
    }
}

// Sum the split-K partials in order and apply the epilogue (gate: also the
// union bits, one atomic per word and block).
template <int SM>
__global__ __launch_bounds__(256) void k_splitk_epilogue(const float *__restrict__ part, int S, int M, int N,
                                                         int part_ld, const int *__restrict__ ncount, EpiArgs epi)
{
    __shared__ uint32_t ub[8];
    const int nlim = ncount ? min(N, *ncount) : N;
    const int n = blockIdx.x * 256 + threadIdx.x;
    const int m = blockIdx.y;
    if (threadIdx.x < 8) ub[threadIdx.x] = 0;
    if (epi.kind == EPI_UP && epi.all_ch && m == 0) {
        // every channel: the identity union list and its size for the down GEMM
        if (n < N) epi.uidx[n] = n;
        if (n == 0) *epi.ucount = N;
    }
    __syncthreads();
    const bool up = epi.kind == EPI_GATE && epi.up_part;
    if (n < nlim) {
        // all S (<= SM) partial loads in flight at once (with the up half's),
        // then summed in split order; splits past S re-read the last one and
        // are not added
        float p[SM], q[SM];
#pragma unroll
        for (int s = 0; s < SM; ++s) {
            const size_t o = ((size_t)min(s, S - 1) * M + m) * part_ld + n;
            p[s] = part[o];
            q[s] = up ? epi.up_part[o] : 0.f;
        }
        float v = 0.f, u = 0.f;
#pragma unroll
        for (int s = 0; s < SM; ++s)
            if (s < S) {
                v += p[s];
                u += q[s];
            }
        if (epilogue(epi, m, n, v) && epi.kind == EPI_GATE && epi.mode == SFFN_THRESHOLD)
            atomicOr(&ub[threadIdx.x / 32], 1u << (n & 31));
        if (up) {
            const size_t o = (size_t)m * epi.F + n;
            epi.H[(size_t)m * epi.hld + n] = f2bf(bf2f(epi.G[o]) * u);
            if (epi.usave) epi.usave[o] = u;
            if (m == 0) epi.uidx[n] = n;
        }
    } else if (up && n < ((nlim + 7) & ~7)) {
        epi.H[(size_t)m * epi.hld + n] = 0;
    } else if ((epi.kind == EPI_UP || epi.kind == EPI_BWD) && n < ((nlim + 7) & ~7)) {
        epi.H[(size_t)m * epi.hld + n] = 0;
        if (epi.kind == EPI_BWD) epi.H2[(size_t)m * epi.hld + n] = 0;
    }
    __syncthreads();
    if (epi.kind == EPI_GATE && epi.mode == SFFN_THRESHOLD && threadIdx.x < 8 && ub[threadIdx.x])
        atomicOr(&epi.ubits[blockIdx.x * 8 + threadIdx.x], ub[threadIdx.x]);
    if (up && n == 0 && m == 0) *epi.ucount = N;
}

// The up GEMM's split-K partials over every channel (computed in the gate's
// launch, before the select) summed for the union's channels only, into the
// union's compacted order: channel n at union position (set bits of the
// bitmap below n) takes H = G u there, row 0 writes the union list and each
// row's first block its size and the zero padding up to a multiple of 8. The
// down GEMM then runs over the union as after the gathered up GEMM. A block
// takes 256 channels (8 bitmap words) of one token row; the entries before
// them are counted from the bitmap, which the select has finished.
template <int SM>
__global__ __launch_bounds__(256) void k_up_compact(const float *__restrict__ part, int S, int M, int N, EpiArgs epi)
{
    __shared__ int wpre[8], red[4];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int W = (N + 31) / 32, w0 = blockIdx.x * 8, m = blockIdx.y, n = blockIdx.x * 256 + tid;
    const uint32_t *ub = epi.ubits;
    // entries before this block (block 0: the union's size instead)
    const int wlim = blockIdx.x == 0 ? W : w0;
    int c = 0;
    for (int w = tid; w < wlim; w += 256) c += __popc(ub[w]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o, 64);
    if (lane == 0) red[wv] = c;
    if (tid < 8) wpre[tid] = w0 + tid < W ? __popc(ub[w0 + tid]) : 0;
    __syncthreads();
    const int cnt = red[0] + red[1] + red[2] + red[3];
    const int base = blockIdx.x == 0 ? 0 : cnt;
    int before = 0;
    for (int j = 0; j < (tid >> 5); ++j) before += wpre[j];
    const uint32_t word = n < N ? ub[n >> 5] : 0u;
    const bool on = (word >> (n & 31)) & 1u;
    if (n < N && (on || epi.usave)) {
        float p[SM];
#pragma unroll
        for (int s = 0; s < SM; ++s) p[s] = part[((size_t)min(s, S - 1) * M + m) * N + n];
        float v = 0.f;
#pragma unroll
        for (int s = 0; s < SM; ++s)
            if (s < S) v += p[s];
        if (epi.usave) epi.usave[(size_t)m * epi.F + n] = v;
        if (on) {
            const int pos = base + before + __popc(word & ((1u << (n & 31)) - 1u));
            epi.H[(size_t)m * epi.hld + pos] = f2bf(bf2f(epi.G[(size_t)m * epi.F + n]) * v);
            if (m == 0) epi.uidx[pos] = n;
        }
    }
    if (blockIdx.x == 0) {
        if (tid < ((cnt + 7) & ~7) - cnt) epi.H[(size_t)m * epi.hld + cnt + tid] = 0;
        if (m == 0 && tid == 0) *epi.ucount = cnt;
    }
}

static hipError_t launch_up_compact(hipStream_t st, const float *part, int S, int M, int N, const EpiArgs &e)
{
    const dim3 grid((N + 255) / 256, M), block(256);
    if (S <= 2) hipLaunchKernelGGL(k_up_compact<2>, grid, block, 0, st, part, S, M, N, e);
    else if (S <= 4) hipLaunchKernelGGL(k_up_compact<4>, grid, block, 0, st, part, S, M, N, e);
    else if (S <= 8) hipLaunchKernelGGL(k_up_compact<8>, grid, block, 0, st, part, S, M, N, e);
    else hipLaunchKernelGGL(k_up_compact<16>, grid, block, 0, st, part, S, M, N, e);
    return hipGetLastError();
}

// Optional outputs for a batch: token t's ascending active list and count;
// block T writes the union size.
__global__ __launch_bounds__(256) void k_emit_batched(const uint16_t *__restrict__ G, const uint8_t *__restrict__ act,
                                                      int T, int F, int mode, const int *__restrict__ ncount,
                                                      const int *__restrict__ utrue,
                                                      int32_t *__restrict__ active_idx,
                                                      int32_t *__restrict__ active_cnt, int32_t *__restrict__ union_cnt)
{
    __shared__ int scratch[5];
    const int t = blockIdx.x;
    if (t == T) {
        if (threadIdx.x == 0 && union_cnt) *union_cnt = utrue ? *utrue : *ncount;
        return;
    }
    const bool dense = mode == SFFN_DENSE || mode == SFFN_DENSE_SILU;
    const bool topk = mode == SFFN_TOPK || mode == SFFN_TOPK_2_8 || mode == SFFN_TOPP;
    const uint16_t *g = G + (size_t)t * F;
    const uint8_t *a = act + (size_t)t * F;
    auto on8 = [&](int i0, bool f[8]) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int i = i0 + e;
            f[e] = i < F && (dense || (topk ? a[i] != 0 : g[i] != 0));
        }
    };
    const int c = emit_ordered(F, on8, active_idx ? active_idx + (size_t)t * F : nullptr, scratch);
    if (threadIdx.x == 0 && active_cnt) active_cnt[t] = c;
}

// ===========================================================================
// Host side
// ===========================================================================
// Above this many tokens the Top-K / top-p union comes from the flags in a
// separate pass instead of per-token atomics.
constexpr int kUnionAtomicMaxTokens = 64;
// W_up bytes that stream at the HBM rate in about one launch's fixed cost
// (~5 us): up to this size the up GEMM of a small batch runs over every
// channel in the gate's launch whatever the union's size
constexpr long long kSpecUpBytes = 32ll << 20;

// Tile shape of k_mfma_dma: TM x TN 32 x 32 MFMA tiles per wavefront, WM x WN
// wavefronts.
struct Cfg {
    int tm, tn, wm, wn;
    int bm() const { return 32 * tm * wm; }
    int bn() const { return 32 * tn * wn; }
};

// Tile shapes by batch size (M = tokens). Large batches take 256 x 256 tiles
// of 8 wavefronts (fewer tile-fill bytes per FLOP: the loads from L2, not
// the MFMAs, bound the loop): K step 32 through four stages for the
// K-contiguous GEMMs (gate, up), K step 64 through two stages for the down
// GEMM (its gathered-row index ring is sized for K step 64).
static Cfg cfg_for(int M)
{
    if (M >= 512) return {4, 2, 2, 4};  // 256 x 256, 8 wavefronts
    if (M >= 128) return {2, 2, 4, 1};  // 256 x 64
    if (M > 64) return {2, 1, 2, 2};    // 128 x 64
    return {1, 1, 1, 2};                // 32 x 64, 2 wavefronts (two M tiles above 32)
}

// The down GEMM's N is d_model: 256 x 256 tiles while they give every CU a
// workgroup, else 256 x 128 (twice the tiles), or 256 x 64 where 256 x 128
// ones would still leave half the CUs idle and the narrower ones fit in one
// round (2048 tokens at d_model 2048: 256 tiles instead of 128).
static Cfg down_cfg(const sffn_ctx &c, const Cfg &cf, int T, int d)
{
    if (cf.tn == 1 && cf.wm == 1) return Cfg{1, 1, 1, 4};  // up to 64 tokens: 32 x 128, four wavefronts
    if (cf.wn != 4) return cf;
    const long long mt = (T + 255) / 256;
    if (mt * ((d + 255) / 256) >= c.n_cu) return cf;
    if (2 * mt * ((d + 127) / 128) <= c.n_cu && mt * ((d + 63) / 64) <= c.n_cu) return Cfg{2, 2, 4, 1};
    return Cfg{4, 2, 2, 2};
}

// 256 x 192 tiles (K-contiguous GEMMs) where 256 x 256 ones leave more than a
// quarter of the CUs idle and the narrower ones still fit in one round
// (2048 x 5632 outputs: 240 tiles instead of 176).
static Cfg narrow_for(const sffn_ctx &c, const Cfg &cf, int M, int N)
{
    if (cf.wn != 4) return cf;
    const long long mt = (M + 255) / 256, t256 = mt * ((N + 255) / 256), t192 = mt * ((N + 191) / 192);
    if (4 * t256 < 3LL * c.n_cu && t192 <= c.n_cu && t192 > t256) return Cfg{2, 3, 4, 2};
    return cf;
}

template <int TM, int TN, int WM, int WN, int BKT, int NS, int OCC, bool BNN, int EK, int GM>
static void launch_dma(dim3 grid, hipStream_t st, int M, int N, int K, const bf16_t *A, int lda, const bf16_t *B,
                       int ldb, const int32_t *bidx, const int *ncount, float *part, int part_ld, const EpiArgs &e)
{
    hipLaunchKernelGGL((k_mfma_dma<TM, TN, WM, WN, BKT, NS, OCC, BNN, EK, GM>), grid, dim3(64 * WM * WN), 0, st, M, N,
                       K, A, lda, B, ldb, bidx, ncount, part, part_ld, e);
}

template <bool BNN, int EK, int GM>
static void dispatch_cfg(const Cfg &c, dim3 grid, hipStream_t st, int M, int N, int K, const bf16_t *A, int lda,
                         const bf16_t *B, int ldb, const int32_t *bidx, const int *ncount, float *part, int pld,
                         const EpiArgs &e)
{
#define SFFN_D(TM, TN, WM, WN, BK, NS) \
    launch_dma<TM, TN, WM, WN, BK, NS, 1, BNN, EK, GM>(grid, st, M, N, K, A, lda, B, ldb, bidx, ncount, part, pld, e)
    // small batches (tn == 1): 32 or 128 x 64 tiles, K step 64, four stages
    // (three for the gathered-row down GEMM)
    constexpr int NSS = BNN ? 3 : 4;
    if (c.tn == 1) {
        if (c.wm == 2) SFFN_D(2, 1, 2, 2, 64, NSS);
        else if (BNN && c.wn == 4) SFFN_D(1, 1, 1, 4, 64, NSS);
        else SFFN_D(1, 1, 1, 2, 64, NSS);
    } else if constexpr (!BNN) {
        if (c.wn == 4) SFFN_D(4, 2, 2, 4, 32, 4);
        else if (c.tn == 3) SFFN_D(2, 3, 4, 2, 64, 2);  // 256 x 192
        else SFFN_D(2, 2, 4, 1, 64, 3);
    } else {
        if (c.wn == 4) SFFN_D(4, 2, 2, 4, 64, 2);
        else if (c.tm == 4) SFFN_D(4, 2, 2, 2, 64, 3);
        else SFFN_D(2, 2, 4, 1, 64, 3);
    }
#undef SFFN_D
}

template <bool BNN, int EK>
static void dispatch_mfma(const Cfg &c, dim3 grid, hipStream_t st, int M, int N, int K, const bf16_t *A, int lda,
                          const bf16_t *B, int ldb, const int32_t *bidx, const int *ncount, float *part, int pld,
                          const EpiArgs &e)
{
    if constexpr (EK != EPI_GATE) {
        dispatch_cfg<BNN, EK, 0>(c, grid, st, M, N, K, A, lda, B, ldb, bidx, ncount, part, pld, e);
    } else {
        switch (e.mode) {
        case SFFN_THRESHOLD:
            dispatch_cfg<BNN, EK, SFFN_THRESHOLD>(c, grid, st, M, N, K, A, lda, B, ldb, bidx, ncount, part, pld, e);
            break;
        case SFFN_TOPK:
        case SFFN_TOPK_2_8:
        case SFFN_TOPP:  // these write the SiLU keys; the selection follows
            dispatch_cfg<BNN, EK, SFFN_TOPK>(c, grid, st, M, N, K, A, lda, B, ldb, bidx, ncount, part, pld, e);
            break;
        case SFFN_DENSE:
            dispatch_cfg<BNN, EK, SFFN_DENSE>(c, grid, st, M, N, K, A, lda, B, ldb, bidx, ncount, part, pld, e);
            break;
        default:
            dispatch_cfg<BNN, EK, SFFN_DENSE_SILU>(c, grid, st, M, N, K, A, lda, B, ldb, bidx, ncount, part, pld,
                                                   e);
            break;
        }
    }
}

// Sum of S split-K partial slices [S][M][part_ld] with the epilogue applied.
static hipError_t launch_splitk_sum(hipStream_t st, const float *part, int S, int M, int N, int part_ld,
                                    const int *ncount, const EpiArgs &e)
{
    const dim3 grid((N + 255) / 256, M), block(256);
    if (S <= 2) hipLaunchKernelGGL(k_splitk_epilogue<2>, grid, block, 0, st, part, S, M, N, part_ld, ncount, e);
    else if (S <= 4) hipLaunchKernelGGL(k_splitk_epilogue<4>, grid, block, 0, st, part, S, M, N, part_ld, ncount, e);
    else if (S <= 8) hipLaunchKernelGGL(k_splitk_epilogue<8>, grid, block, 0, st, part, S, M, N, part_ld, ncount, e);
    else hipLaunchKernelGGL(k_splitk_epilogue<16>, grid, block, 0, st, part, S, M, N, part_ld, ncount, e);
    return hipGetLastError();
}

// One block per (M tile, N tile), padded so the N tiles split evenly over 8 XCDs.
static dim3 tile_grid(int nt, int mt, int sk) { return dim3(8 * ((nt + 7) / 8) * mt, 1, sk); }

// Split K so that the grid has at least ~2 workgroups per CU (at most 8
// splits, and K steps of at least 8 tiles per split). Below 128 tokens the
// weights stream once through many small workgroups: up to splits_max
// splits, ~3 workgroups per CU, at least 4 K steps of 64 per split.
static int split_for(const sffn_ctx &c, long long tiles, int K, int M, int part_rows = -1)
{
    int S = 1;
    if (part_rows < 0) part_rows = c.L.bpart_rows;
    const int smax = min(splits_max(M), part_rows / M);  // and what the partial buffer holds
    if (M < 128) {
        while (2 * S <= smax && tiles * S < c.n_cu && (K / 64) / (2 * S) >= 4) S *= 2;
        return S;
    }
    while (2 * S <= smax && tiles * S < 2LL * c.n_cu && (K / 32) / (2 * S) >= 8) S *= 2;
    return S;
}

// Gate or up GEMM on 256 x 256 tiles in two launches, whole rounds and the
// K-split rest (rest_split), plus the rest's partial sum. u_host: the gate's
// N (d_ff), or -1 for the up GEMM (N = the union, at most d_ff, counted on
// the device). Returns false, having launched nothing, where the split does
// not apply: other tiles, no whole round, a rest that one launch runs as
// well, or a partial buffer smaller than a round of tiles.
template <int EK>
static bool launch_rounds_rest(const sffn_ctx &c, const Cfg &cf, int mt, hipStream_t st, int T, int F, int d,
                               const bf16_t *x, const bf16_t *w, float *part, EpiArgs ep, int u_host, hipError_t &e)
{
    constexpr int smax = 4;
    const int BN = cf.bn(), nt = (F + BN - 1) / BN, per = max(1, c.n_cu / mt), nfull_max = nt / per * per;
    if (cf.wn != 4 || BN != 256 || cf.bm() % 16 || nfull_max == 0 || c.L.bpart_elems < (size_t)c.n_cu * cf.bm() * BN)
        return false;
    // the rest's largest list and row count over the N extents it may meet
    int len_max = 0, rows_max = 0;
    for (int u = u_host >= 0 ? nt : 1; u <= nt; ++u) {
        const RestSplit s = rest_split(u * BN, BN, mt, c.n_cu, smax);
        const int tiles = (s.ntt - s.nfull) * mt;
        len_max = max(len_max, tiles * s.S);
        if (s.S > 1) rows_max = max(rows_max, tiles * cf.bm());
    }
    if (u_host >= 0 && rows_max == 0) return false;  // no rest, or one split: one launch
    ep.ncu = c.n_cu;
    ep.smax = smax;
    ep.rest_u = u_host;
    if (u_host >= 0) {
        // the gate: the whole rounds are known here
        const int nfull = rest_split(u_host, BN, mt, c.n_cu, smax).nfull;
        ep.upart = 0;
        dispatch_mfma<false, EK>(cf, tile_grid(nfull, mt, 1), st, T, nfull * BN, d, x, d, w, d, nullptr, nullptr, part,
                                 F, ep);
    } else {
        ep.upart = 1;
        dispatch_mfma<false, EK>(cf, tile_grid(nfull_max, mt, 1), st, T, F, d, x, d, w, d, nullptr, nullptr, part, F,
                                 ep);
    }
    if ((e = hipGetLastError()) != hipSuccess) return true;
    if (len_max > 0) {
        ep.upart = 2;
        dispatch_mfma<false, EK>(cf, dim3(8 * ((len_max + 7) / 8)), st, T, F, d, x, d, w, d, nullptr, nullptr, part, F,
                                 ep);
        if ((e = hipGetLastError()) != hipSuccess) return true;
    }
    if (rows_max > 0) {  // 16 tile rows per workgroup
        hipLaunchKernelGGL(k_rest_sum<EK>, dim3(min(8192, (rows_max + 15) / 16)), dim3(256), 0, st, part, T, cf.bm(),
                           BN, ep);
        e = hipGetLastError();
    }
    return true;
}

// The share of channels a small batch of iid tokens leaves out of its union,
// where the mode fixes it: (1 - K/F)^T for Top-K, 0.75^T for 2:8 (1 for the
// others: unknown before the gate). Up to 64 tokens the up and down GEMMs run
// over every channel when it is small: no up tile waits for the union bitmap,
// the gate values are 0 where a channel is off (y is the same sum up to the
// order of additions), and the up GEMM's tiles can join the gate's launch.
// With that launch every channel pays from a union of ~75 % (MoC layer, 16
// tokens: Top-K K = 704, union 88 %, 45.6 -> 37.4 us); without it only from
// ~97 % (the up GEMM over every channel alone: 9.3 us against 11.9 over an
// 88 % union, 12.6 against 14.9 at 100 %).
static double union_miss(int mode, int T, int F, int K)
{
    if (T < 2 || T > 64) return 1.0;
    if (mode == SFFN_TOPK) return std::pow(1.0 - (double)K / F, T);
    if (mode == SFFN_TOPK_2_8) return std::pow(0.75, T);
    return 1.0;
}

hipError_t launch_batched(sffn_ctx &c, const FwdArgs &a)
{
    const sffn_shape &S = c.shape;
    const int T = a.n, d = S.d_model, F = S.d_ff;
    char *ws = c.ws;
    uint16_t *G = reinterpret_cast<uint16_t *>(ws + c.L.gsel);
    uint16_t *H = reinterpret_cast<uint16_t *>(ws + c.L.hbuf);
    float *keys = reinterpret_cast<float *>(ws + c.L.keys);
    uint8_t *act = reinterpret_cast<uint8_t *>(ws + c.L.act);
    uint32_t *ubits = reinterpret_cast<uint32_t *>(ws + c.L.ubits);
    int32_t *uidx = reinterpret_cast<int32_t *>(ws + c.L.uidx);
    int *ncount = reinterpret_cast<int *>(ws + c.L.ctrl) + kCtrlUnionSize;
    float *part = reinterpret_cast<float *>(ws + c.L.bpart);
    const bf16_t *x = static_cast<const bf16_t *>(a.x);
    const bf16_t *wg = static_cast<const bf16_t *>(a.w.w_gate);
    const bf16_t *wu = static_cast<const bf16_t *>(a.w.w_up);
    const bf16_t *wdn = static_cast<const bf16_t *>(a.w.w_down);
    hipStream_t st = a.stream;
    const bool dense = a.mode == SFFN_DENSE || a.mode == SFFN_DENSE_SILU;
    hipEvent_t ev0 = static_cast<hipEvent_t>(c.ev_start), ev1 = static_cast<hipEvent_t>(c.ev_stop);
    hipError_t e;

    EpiArgs ep{};
    ep.mode = a.mode;
    ep.tau = a.tau;
    ep.T = T;
    ep.F = F;
    ep.d = d;
    ep.G = G;
    ep.keys = keys;
    ep.debug_z = a.debug_z;
    ep.ubits = ubits;
    ep.uidx = uidx;
    ep.ucount = ncount;
    ep.H = H;
    ep.hld = (F + 7) / 8 * 8;
    ep.Y = a.y;
    ep.usave = a.usave;

    const Cfg cf = cfg_for(T);
    Cfg cfd = cf;
    // the down GEMM's N is d_model: keep 256 x 256 tiles only while they
    // still give every CU a workgroup, else 256 x 128 (twice the tiles)
    cfd = down_cfg(c, cfd, T, d);
    const int mt = (T + cf.bm() - 1) / cf.bm(), mtd = (T + cfd.bm() - 1) / cfd.bm();

    // ---- 1. gate GEMM ----
    int gate_split = 0;  // > 0: the select sums this many split-K partials of the gate GEMM
    // every channel for the up and down GEMMs (not with token groups, which
    // take their own unions)
    const double miss = union_miss(a.mode, T, F, a.k);
    bool all_ch = miss <= 0.25 && !(c.token_groups > 1 && T >= c.token_groups * kTokenGroupMinTokens);
    const bool dense_small = dense && T <= kUnionAtomicMaxTokens;  // every channel by definition
    // a union of unknown size (top-p, threshold) or well short of every
    // channel: while all of W_up streams in about the time of one launch of its
    // own, the up GEMM still runs over every channel in the gate's launch and
    // its sum keeps the union's channels only (the down GEMM stays on the union)
    const bool spec = !dense && !all_ch && T <= kUnionAtomicMaxTokens && (long long)F * d * 2 <= kSpecUpBytes &&
                      !(c.token_groups > 1 && T >= c.token_groups * kTokenGroupMinTokens);
    // top-p and the threshold there run over every channel as well: the select
    // kernel (top-p) or the gate's split-K sum (threshold) then writes the
    // product rows itself (no compaction launch), and on such a layer all of
    // W_down streams in about the time that launch took
    if (spec && (a.mode == SFFN_TOPP || a.mode == SFFN_THRESHOLD)) all_ch = true;
    int dual_s = 0;  // > 0: the up GEMM ran in the gate's launch, with this many K splits
    {
        ep.kind = EPI_GATE;
        // 256 <= T < 512: the gate GEMM reads every weight row once either
        // way, but 256 x 64 tiles re-read the activation block for every
        // 64 channels; 256 x 256 tiles split K in two instead
        const bool wide = T >= 256 && T < 512 && c.L.bpart_rows >= 2 * T;
        const Cfg cg = wide ? Cfg{4, 2, 2, 4} : narrow_for(c, cf, T, F);
        const int nt = (F + cg.bn() - 1) / cg.bn(), mtg = (T + cg.bm() - 1) / cg.bm();
        const int sk = wide ? 2 : split_for(c, (long long)mt * nt, d, T);
        if (ev0) hipEventRecord(ev0, st);
        if (!wide && launch_rounds_rest<EPI_GATE>(c, cg, mtg, st, T, F, d, x, wg, part, ep, F, e)) {
            if (e != hipSuccess) return e;
        } else {
            // every channel: the up GEMM's tiles join the gate's launch (it does
            // not depend on the gate), each half of the partial buffer for one
            // (at least two splits: the up tiles leave partials for their sum, which applies the gate values)
            const bool join = (all_ch || dense_small || spec) && !wide;
            int skd = join ? split_for(c, 2LL * mtg * nt, d, T, c.L.bpart_rows / 2) : 0;
            if (join && skd < 2 && 4 * T <= c.L.bpart_rows) skd = 2;
            int s_used = sk;
            if (skd > 1 && T <= kUnionAtomicMaxTokens && sum_select_fits(F, skd)) {
                ep.dual = 1;
                ep.B2 = wu;
                ep.part2 = part + (size_t)skd * T * F;
                dual_s = s_used = skd;
                dispatch_mfma<false, EPI_GATE>(cg, tile_grid(2 * nt, mtg, skd), st, T, F, d, x, d, wg, d, nullptr,
                                               nullptr, part, F, ep);
            } else {
                dispatch_mfma<false, EPI_GATE>(cg, tile_grid(nt, mtg, sk), st, T, F, d, x, d, wg, d, nullptr, nullptr,
                                               part, F, ep);
            }
            if ((e = hipGetLastError()) != hipSuccess) return e;
            if (!dual_s && miss > 0.03) all_ch = false;  // every channel pays only with the joined launch
            // small Top-K / top-p / 2:8 batches: the select sums the partials itself
            gate_split = !wide && T <= kUnionAtomicMaxTokens &&
                                 (a.mode == SFFN_TOPK || a.mode == SFFN_TOPP || a.mode == SFFN_TOPK_2_8) &&
                                 sum_select_fits(F, s_used) ? s_used : 0;
            if (s_used > 1 && !gate_split) {
                // over every channel (dense, or the threshold on a small layer)
                // the gate's sum applies the gate values to the up half as well
                if (dual_s > 0 && (dense || all_ch)) ep.up_part = ep.part2;
                if ((e = launch_splitk_sum(st, part, s_used, T, F, F, nullptr, ep)) != hipSuccess) return e;
            }
        }
        if (ev1) hipEventRecord(ev1, st);
    }
    // ---- Top-K / top-p: per-token select, its flags and the union of the
    // flags (above 64 tokens the union comes from one pass over the flags:
    // per-token atomics on the same few bitmap words would serialise) ----
    // over every channel with the up GEMM in the gate's launch, the select
    // kernel also applies the gate values to the up partials (a token's
    // product row needs only that token's select)
    UpHalf uh{};
    if (dual_s > 0 && all_ch && gate_split == dual_s && !dense &&
        (a.mode == SFFN_TOPK_2_8 || gate_split <= kSelectUpMaxSplits))
        uh = UpHalf{ep.part2, H, ep.hld, a.usave, uidx, ncount};
    if (gate_split && a.mode != SFFN_TOPK_2_8) {
        e = launch_sum_select_flags(part, gate_split, T, F, a.mode, a.k, a.tau, a.debug_z, act, G, ubits, st, uh);
        if (e != hipSuccess) return e;
    } else if (a.mode == SFFN_TOPK || a.mode == SFFN_TOPP) {
        uint32_t *ub = T > kUnionAtomicMaxTokens ? nullptr : ubits;
        e = a.mode == SFFN_TOPK ? launch_topk_select_flags(keys, T, F, a.k, act, G, ub, st)
                                : launch_topp_select_flags(keys, T, F, a.tau, act, G, ub, st);
        if (e != hipSuccess) return e;
        if (!ub && (e = launch_union_flags(act, T, F, ubits, st)) != hipSuccess) return e;
    }
    // ---- 2:8: the top 2 of each group of 8 keys, its flags and the union ----
    if (a.mode == SFFN_TOPK_2_8) {
        e = gate_split ? launch_nm_flags(keys, T, F, act, G, ubits, st, part, gate_split, a.debug_z, uh)
                       : launch_nm_flags(keys, T, F, act, G, ubits, st);
        if (e != hipSuccess) return e;
    }
    // ---- token groups: each group's up and down products over its own union ----
    const int ng = c.token_groups;
    if (ng > 1 && !dense && T >= ng * kTokenGroupMinTokens) {
        GroupArgs ga{};
        ga.T = T;
        ga.F = F;
        ga.d = d;
        ga.ng = ng;
        ga.G = G;
        ga.x = x;
        ga.ubits = ubits;
        ga.ncount = ncount;
        ga.Mb = reinterpret_cast<uint32_t *>(ws + c.L.gbits);
        ga.cnt = reinterpret_cast<int *>(ws + c.L.gcnt);
        ga.nsz = reinterpret_cast<int *>(ws + c.L.gstat);
        ga.Q = reinterpret_cast<long long *>(ws + c.L.gstat + 4 * kMaxTokenGroups);
        ga.grp = reinterpret_cast<int *>(ws + c.L.grp);
        ga.tmap = reinterpret_cast<int *>(ws + c.L.tmap);
        ga.xp = reinterpret_cast<uint16_t *>(ws + c.L.xp);
        ga.gub = reinterpret_cast<uint32_t *>(ws + c.L.gub);
        ga.stream = st;
        int nh[kMaxTokenGroups] = {};
        if ((e = launch_token_groups(ga, nh)) != hipSuccess) return e;
        const int W = (F + 31) / 32;
        int s0 = 0;
        for (int g = 0; g < ng; s0 += nh[g], ++g) {
            const int Tg = nh[g];
            if (Tg <= 0) continue;
            EpiArgs eg = ep;
            eg.T = Tg;
            eg.ubits = ga.gub + (size_t)g * W;
            eg.uidx = reinterpret_cast<int32_t *>(ws + c.L.guidx) + (size_t)g * F;
            eg.ucount = reinterpret_cast<int *>(ws + c.L.gcount) + g;
            eg.H = H + (size_t)s0 * ep.hld;
            eg.tmap = ga.tmap + s0;
            const Cfg cg = cfg_for(Tg);
            Cfg cgd = cg;
            if (cgd.wn == 4 && ((Tg + 255) / 256) * ((d + 255) / 256) < c.n_cu) cgd = Cfg{4, 2, 2, 2};
            const int mtg = (Tg + cg.bm() - 1) / cg.bm(), mtgd = (Tg + cgd.bm() - 1) / cgd.bm();
            eg.kind = EPI_UP;
            int nt = (F + cg.bn() - 1) / cg.bn();
            int sk = split_for(c, (long long)mtg * nt / 2, d, Tg);
            dispatch_mfma<false, EPI_UP>(cg, tile_grid(nt, mtg, sk), st, Tg, F, d, ga.xp + (size_t)s0 * d, d, wu, d,
                                         nullptr, nullptr, part, F, eg);
            if ((e = hipGetLastError()) != hipSuccess) return e;
            if (sk > 1 && (e = launch_splitk_sum(st, part, sk, Tg, F, F, eg.ucount, eg)) != hipSuccess) return e;
            eg.kind = EPI_DOWN;
            nt = (d + cgd.bn() - 1) / cgd.bn();
            sk = split_for(c, (long long)mtgd * nt, F / 2, Tg);
            dispatch_mfma<true, EPI_DOWN>(cgd, tile_grid(nt, mtgd, sk), st, Tg, d, F, eg.H, ep.hld, wdn, d, eg.uidx,
                                          eg.ucount, part, d, eg);
            if ((e = hipGetLastError()) != hipSuccess) return e;
            if (sk > 1 && (e = launch_splitk_sum(st, part, sk, Tg, d, d, nullptr, eg)) != hipSuccess) return e;
        }
        if (a.active_idx || a.active_cnt || a.union_cnt) {
            hipLaunchKernelGGL(k_emit_batched, dim3(T + 1), dim3(256), 0, st, G, act, T, F, a.mode, ncount, nullptr,
                               a.active_idx, a.active_cnt, a.union_cnt);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        return hipSuccess;
    }
    // ---- 2. up GEMM over the union rows (each workgroup lists its part) ----
    {
        ep.kind = EPI_UP;
        const bool compact = dual_s > 0 && !all_ch && !dense;
        ep.all_ch = all_ch || (dual_s > 0 && !compact) ? 1 : 0;
        ep.utrue = reinterpret_cast<int *>(ws + c.L.ctrl) + kCtrlUnionTrue;
        const int nt = (F + cf.bn() - 1) / cf.bn();
        if (uh.part || ep.up_part) {
            // the select kernel or the gate's sum wrote the product rows and
            // the identity union list
        } else if (compact) {
            // the up partials came with the gate's launch: the union's channels
            // summed into the union's order, with its list and size
            if ((e = launch_up_compact(st, ep.part2, dual_s, T, F, ep)) != hipSuccess) return e;
        } else if (dual_s > 0) {
            // the up partials came with the gate's launch: their sum with the
            // gate values applied (and the identity union list for the down GEMM)
            if ((e = launch_splitk_sum(st, ep.part2, dual_s, T, F, F, nullptr, ep)) != hipSuccess) return e;
        } else if (launch_rounds_rest<EPI_UP>(c, cf, mt, st, T, F, d, x, wu, part, ep, -1, e)) {
            // 256 x 256 tiles: the whole rounds, then the rest split along K
            if (e != hipSuccess) return e;
        } else {
            const Cfg cu = narrow_for(c, cf, T, F);  // the union is at most F
            const int ntu = (F + cu.bn() - 1) / cu.bn();
            const int sk = split_for(c, (long long)mt * ntu / 2, d, T);  // the union is a fraction of F
            dispatch_mfma<false, EPI_UP>(cu, tile_grid(ntu, mt, sk), st, T, F, d, x, d, wu, d, nullptr, nullptr, part,
                                          F, ep);
            if ((e = hipGetLastError()) != hipSuccess) return e;
            if (sk > 1) {
                if ((e = launch_splitk_sum(st, part, sk, T, F, F, ncount, ep)) != hipSuccess) return e;
            }
        }
    }
    // ---- 3. down GEMM, K = union ----
    {
        ep.kind = EPI_DOWN;
        const int nt = (d + cfd.bn() - 1) / cfd.bn();
        // K: every channel; a union compacted from every channel (top-p,
        // threshold: mostly most of them at these sizes) as if it were; else
        // half of them (the union's size is known only on the device)
        const int sk = split_for(c, (long long)mtd * nt, ep.all_ch || dual_s > 0 ? F : F / 2, T);
        dispatch_mfma<true, EPI_DOWN>(cfd, tile_grid(nt, mtd, sk), st, T, d, F, H, ep.hld, wdn, d, uidx, ncount, part,
                                      d, ep);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (sk > 1) {
            if ((e = launch_splitk_sum(st, part, sk, T, d, d, nullptr, ep)) != hipSuccess) return e;
        }
    }
    // ---- optional outputs ----
    if (a.active_idx || a.active_cnt || a.union_cnt) {
        hipLaunchKernelGGL(k_emit_batched, dim3(T + 1), dim3(256), 0, st, G, act, T, F, a.mode, ncount,
                           all_ch ? ep.utrue : nullptr, a.active_idx,
                           a.active_cnt, a.union_cnt);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

// ===========================================================================
// Training
// ===========================================================================
// The forward on the union path with the dense z and the union's up values
// kept in the training workspace, then each token's stored rows.
hipError_t launch_forward_train(sffn_ctx &c, FwdArgs a, const Saved &sv, char *tws)
{
    const sffn_shape &S = c.shape;
    const TrainLayout TL = make_train_layout(S);
    const size_t TF = (size_t)S.max_tokens * S.d_ff;
    float *zd = reinterpret_cast<float *>(tws + TL.zu);
    float *ud = zd + TF;
    a.debug_z = zd;
    a.usave = ud;
    hipError_t e = launch_batched(c, a);
    if (e != hipSuccess) return e;
    const uint8_t *act = reinterpret_cast<const uint8_t *>(c.ws + c.L.act);
    return launch_save(zd, ud, act, a.n, S.d_ff, a.mode, a.tau, sv, a.stream);
}

// Backward over the stored rows, on the union U of the stored channels:
//   dH  = dY . W_down[U]^T        (T x |U|); epilogue: du = dh g(z),
//                                 dz = dh u g'(z), h = g(z) u, zero where off
//   dX  = dU . W_up[U] + dZ . W_gate[U]   (two down-form products, the second adds)
//   dW_down[U] += H^T dY,  dW_up[U] += dU^T X,  dW_gate[U] += dZ^T X
// The weight gradients are C = X^T . dU (M = d_model, N = |U|, K = tokens)
// with both operands token-contiguous, written into row U[n].
hipError_t launch_backward(sffn_ctx &c, const BwdArgs &a)
{
    const sffn_shape &S = c.shape;
    const TrainLayout TL = make_train_layout(S);
    const int T = a.n, d = S.d_model, F = S.d_ff;
    const int FP = (F + 7) / 8 * 8, tp = (T + 7) / 8 * 8;
    char *tws = a.tws;
    float2 *ZU = reinterpret_cast<float2 *>(tws + TL.zu);
    uint16_t *dU = reinterpret_cast<uint16_t *>(tws + TL.du), *dZ = reinterpret_cast<uint16_t *>(tws + TL.dz);
    uint16_t *DUT = reinterpret_cast<uint16_t *>(tws + TL.dut), *DZT = reinterpret_cast<uint16_t *>(tws + TL.dzt);
    uint16_t *HT = reinterpret_cast<uint16_t *>(tws + TL.ht);
    uint16_t *XT = reinterpret_cast<uint16_t *>(tws + TL.xt), *DYT = reinterpret_cast<uint16_t *>(tws + TL.dyt);
    uint32_t *ubits = reinterpret_cast<uint32_t *>(tws + TL.ubits);
    int32_t *uidx = reinterpret_cast<int32_t *>(tws + TL.uidx);
    int *ucount = reinterpret_cast<int *>(tws + TL.ctrl);
    float *part = reinterpret_cast<float *>(tws + TL.part);
    const bf16_t *x = static_cast<const bf16_t *>(a.x), *dy = static_cast<const bf16_t *>(a.dy);
    const bf16_t *wg = static_cast<const bf16_t *>(a.w.w_gate), *wu = static_cast<const bf16_t *>(a.w.w_up);
    const bf16_t *wdn = static_cast<const bf16_t *>(a.w.w_down);
    hipStream_t st = a.stream;
    hipError_t e;

    e = launch_bwd_setup(a.sv, T, F, d, tp, ZU, ubits, uidx, ucount, DUT, DZT, HT,
                         reinterpret_cast<const uint16_t *>(x), reinterpret_cast<const uint16_t *>(dy),
                         XT, DYT, st);
    if (e != hipSuccess) return e;

    EpiArgs ep{};
    ep.mode = (a.mode == SFFN_THRESHOLD || a.mode == SFFN_DENSE) ? 0 : 1;  // derivative kind
    ep.tau = a.tau;
    ep.T = T;
    ep.F = F;
    ep.d = d;
    ep.ubits = ubits;
    ep.uidx = uidx;
    ep.ucount = ucount;
    ep.H = dU;
    ep.H2 = dZ;
    ep.hld = FP;
    ep.ZU = ZU;
    ep.DUT = DUT;
    ep.DZT = DZT;
    ep.HT = HT;
    ep.tp = tp;

    const Cfg cf = cfg_for(T);
    Cfg cfd = cf;
    cfd = down_cfg(c, cfd, T, d);
    const int mt = (T + cf.bm() - 1) / cf.bm(), mtd = (T + cfd.bm() - 1) / cfd.bm();

    // ---- dH = dY . W_down[U]^T, with the derivative epilogue ----
    {
        ep.kind = EPI_BWD;
        const Cfg cb = narrow_for(c, cf, T, F);
        const int nt = (F + cb.bn() - 1) / cb.bn();
        const int sk = split_for(c, (long long)mt * nt / 2, d, T, TL.part_rows);
        dispatch_mfma<false, EPI_BWD>(cb, tile_grid(nt, mt, sk), st, T, F, d, dy, d, wdn, d, uidx, ucount, part, F,
                                      ep);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (sk > 1 && (e = launch_splitk_sum(st, part, sk, T, F, F, ucount, ep)) != hipSuccess) return e;
    }
    // ---- dX = dU . W_up[U], then += dZ . W_gate[U] ----
    {
        const int nt = (d + cfd.bn() - 1) / cfd.bn();
        const int sk = split_for(c, (long long)mtd * nt, F / 2, T, TL.part_rows);
        ep.Y = a.dx;
        ep.kind = EPI_DOWN;
        dispatch_mfma<true, EPI_DOWN>(cfd, tile_grid(nt, mtd, sk), st, T, d, F, dU, FP, wu, d, uidx, ucount, part, d,
                                      ep);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (sk > 1 && (e = launch_splitk_sum(st, part, sk, T, d, d, nullptr, ep)) != hipSuccess) return e;
        ep.kind = EPI_DOWN_ACC;
        dispatch_mfma<true, EPI_DOWN_ACC>(cfd, tile_grid(nt, mtd, sk), st, T, d, F, dZ, FP, wg, d, uidx, ucount, part,
                                          d, ep);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (sk > 1 && (e = launch_splitk_sum(st, part, sk, T, d, d, nullptr, ep)) != hipSuccess) return e;
    }
    // ---- weight gradients: C[d][|U|] over K = tokens, added into rows U[n] ----
    {
        const Cfg cw = narrow_for(c, cfg_for(d), d, F);
        const int nt = (F + cw.bn() - 1) / cw.bn(), mw = (d + cw.bm() - 1) / cw.bm();
        ep.kind = EPI_WGRAD;
        const struct {
            const uint16_t *a, *b;
            float *out;
        } prods[3] = {{DYT, HT, a.dwd}, {XT, DUT, a.dwu}, {XT, DZT, a.dwg}};
        for (const auto &p : prods) {
            ep.Y = p.out;
            dispatch_mfma<false, EPI_WGRAD>(cw, tile_grid(nt, mw, 1), st, d, F, tp, reinterpret_cast<const bf16_t *>(p.a),
                                            tp, reinterpret_cast<const bf16_t *>(p.b), tp, nullptr, ucount, part, F,
                                            ep);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

}  // namespace sffn
