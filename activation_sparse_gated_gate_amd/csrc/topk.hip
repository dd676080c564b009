// Per-token Top-K and top-p selection of a batch over the SiLU gate keys
// ("Mixture-of-Channels" blog summary, "Dentro il 'mixture'": each token
// keeps its K channels of largest SiLU(gate)), and the batched 2:8
// structured selection (the same summary's 2:8 option: the top 2 of every
// aligned group of 8 channels). (At one to eight tokens the selects run
// inside the up kernel's launch, decode.hip.)
//
// The select finds, per token, the K-th largest key and a tie cutoff (one
// 1024-thread workgroup per token, select_kth in select.h; from 256 tokens
// up, one 256-thread workgroup, wg_topk_boundary in topk_wg.h). Channel i of
// token t is then selected iff
//   key > kth  or  (key == kth and i <= cut)
// (topk_on), so ties at the K-th value go to the lower channel indices and
// exactly K channels are selected. The select kernels apply it right after
// the select, to the keys they hold, and write the batch's flags, gate
// values and union bitmap. Top-p (k_topp_select_flags) finds the same pair
// by cumulative softmax mass instead of a count (select_mass).
#include <algorithm>
#include <type_traits>

#include "select.h"
#include "topk_wg.h"
#include "sffn_internal.h"

namespace sffn {

// Batched: token t's flags act[t][i], the gate values the up GEMM reads
// (G[t][i] = bf16 key where selected, else 0) and its bits of the union
// bitmap, ORed in with one atomic per 32-bit word and wavefront (the bitmap is
// all zero on entry: the down GEMM clears it after use; ubits null: no union
// bits, k_union_flags builds the bitmap afterwards), from the boundary r of a
// select; the keys are kf (KPT > 0) or re-read from s.
template <int KPT>
__device__ __forceinline__ void write_flags(const float *__restrict__ s, int F, int2 r,
                                            const float (&kf)[KPT > 0 ? KPT : 1], uint8_t *__restrict__ a,
                                            uint16_t *__restrict__ g, uint32_t *__restrict__ ubits)
{
    const int tid = threadIdx.x, lane = tid & 63;
    if constexpr (KPT > 0) {
        // channels KPT tid .. + KPT-1: one 32-bit word, shared by 32 / KPT lanes
        const int i0 = tid * KPT;
        uint32_t m = 0;
        if (KPT % 8 == 0 && (F & 7) == 0 && i0 + KPT <= F) {
            // whole groups of 8: the flags in one 8-byte store and the gate
            // values in one 16-byte store per group (the rows are aligned)
#pragma unroll
            for (int e0 = 0; e0 + 8 <= KPT; e0 += 8) {
                uint32_t fl[2] = {0u, 0u}, gw[4] = {0u, 0u, 0u, 0u};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const bool on = topk_on(kf[e0 + e], i0 + e0 + e, r);
                    fl[e >> 2] |= (uint32_t)on << (8 * (e & 3));
                    gw[e >> 1] |= (uint32_t)(on ? f2bf(kf[e0 + e]) : (uint16_t)0) << (16 * (e & 1));
                    m |= (uint32_t)on << (e0 + e);
                }
                *reinterpret_cast<uint2 *>(a + i0 + e0) = make_uint2(fl[0], fl[1]);
                *reinterpret_cast<uint4 *>(g + i0 + e0) = make_uint4(gw[0], gw[1], gw[2], gw[3]);
            }
        } else {
#pragma unroll
            for (int e = 0; e < KPT; ++e) {
                const int i = i0 + e;
                if (i < F) {
                    const bool on = topk_on(kf[e], i, r);
                    a[i] = on;
                    g[i] = on ? f2bf(kf[e]) : (uint16_t)0;
                    m |= (uint32_t)on << e;
                }
            }
        }
        m <<= i0 & 31;
#pragma unroll
        for (int o = 1; o < 32 / KPT; o <<= 1) m |= __shfl_xor(m, o, 64);
        if (ubits && (lane & (32 / KPT - 1)) == 0 && m) atomicOr(&ubits[i0 >> 5], m);
    } else {
        for (int i0 = tid - lane; i0 < F; i0 += 1024) {
            const int i = i0 + lane;
            bool on = false;
            if (i < F) {
                const float k = s[i];
                on = topk_on(k, i, r);
                a[i] = on;
                g[i] = on ? f2bf(k) : (uint16_t)0;
            }
            const unsigned long long b = __ballot(on);
            const uint32_t bits = (uint32_t)(b >> (lane & 32));
            if (ubits && (lane & 31) == 0 && bits) atomicOr(&ubits[i >> 5], bits);
        }
    }
}

// Batched Top-K: the select of token t (one 1024-thread workgroup per token),
// then its flags.
template <int KPT>
__global__ __launch_bounds__(1024) void k_topk_select_flags(const float *__restrict__ keys, int F, int K,
                                                            uint8_t *__restrict__ act, uint16_t *__restrict__ G,
                                                            uint32_t *__restrict__ ubits)
{
    __shared__ SelectLds L;
    const int t = blockIdx.x;
    const float *s = keys + (size_t)t * F;
    float kf[KPT > 0 ? KPT : 1];
    select_kth_clear(L);
    load_keys<KPT>(s, F, kf);
    const int2 r = select_kth<KPT>(s, F, K, L, kf);
    write_flags<KPT>(s, F, r, kf, act + (size_t)t * F, G + (size_t)t * F, ubits);
}

// Token t's row of split-K partials [S][T][F] summed over the S splits in
// split order (exactly as the split-K sum kernel adds them), this thread's
// channels KPT tid .. + KPT-1, 0 past F.
template <int KPT, int SM>
__device__ __forceinline__ void sum_split_rows(const float *__restrict__ part, int S, int T, int F, int t,
                                               float (&sum)[KPT])
{
    static_assert(KPT % 4 == 0, "whole float4 groups per thread");
    constexpr int EB = SM >= 32 ? 1 : 32 / SM < KPT ? 32 / SM : KPT;  // channels whose partials are in flight together
    static_assert(KPT % EB == 0 && (EB % 4 == 0 || EB < 4), "whole batches");
    const int i0 = threadIdx.x * KPT;
    const bool vec = (F & 3) == 0;  // rows of the partials 16-byte aligned
#pragma unroll
    for (int e0 = 0; e0 < KPT; e0 += EB) {
        float p[SM][EB];
#pragma unroll
        for (int s = 0; s < SM; ++s) {
            const float *row = part + ((size_t)min(s, S - 1) * T + t) * F;
            if (EB >= 4 && vec) {
#pragma unroll
                for (int e = 0; e < EB; e += 4) {
                    const int i = i0 + e0 + e;  // i < F implies i + 3 < F (F, i multiples of 4)
                    const float4 q = i < F ? *reinterpret_cast<const float4 *>(row + i) : make_float4(0.f, 0.f, 0.f, 0.f);
                    p[s][e] = q.x;
                    p[s][e + 1] = q.y;
                    p[s][e + 2] = q.z;
                    p[s][e + 3] = q.w;
                }
            } else {
#pragma unroll
                for (int e = 0; e < EB; ++e) {
                    const int i = i0 + e0 + e;
                    p[s][e] = i < F ? row[i] : 0.f;
                }
            }
        }
#pragma unroll
        for (int e = 0; e < EB; ++e) {
            float v = 0.f;
#pragma unroll
            for (int s = 0; s < SM; ++s)
                if (s < S) v += p[s][e];
            sum[e0 + e] = v;
        }
    }
}

// Token t's keys from the gate GEMM's split-K partials (the form for small
// batches, whose gate GEMM splits K): the sums as sum_split_rows takes them,
// then SiLU; the pre-activations also into debug_z when it is set. The
// select that follows then needs no separate sum launch.
template <int KPT, int SM>
__device__ __forceinline__ void sum_split_keys(const float *__restrict__ part, int S, int T, int F, int t,
                                               float *__restrict__ debug_z, float (&kf)[KPT])
{
    static_assert(KPT % 4 == 0, "whole float4 groups per thread");
    constexpr int EB = SM >= 32 ? 1 : 32 / SM < KPT ? 32 / SM : KPT;  // channels whose partials are in flight together
    static_assert(KPT % EB == 0 && (EB % 4 == 0 || EB < 4), "whole batches");
    const int i0 = threadIdx.x * KPT;
    const bool vec = (F & 3) == 0;  // rows of the partials 16-byte aligned
#pragma unroll
    for (int e0 = 0; e0 < KPT; e0 += EB) {
        float p[SM][EB];
#pragma unroll
        for (int s = 0; s < SM; ++s) {
            const float *row = part + ((size_t)min(s, S - 1) * T + t) * F;
            if (EB >= 4 && vec) {
#pragma unroll
                for (int e = 0; e < EB; e += 4) {
                    const int i = i0 + e0 + e;  // i < F implies i + 3 < F (F, i multiples of 4)
                    const float4 q = i < F ? *reinterpret_cast<const float4 *>(row + i) : make_float4(0.f, 0.f, 0.f, 0.f);
                    p[s][e] = q.x;
                    p[s][e + 1] = q.y;
                    p[s][e + 2] = q.z;
                    p[s][e + 3] = q.w;
                }
            } else {
#pragma unroll
                for (int e = 0; e < EB; ++e) {
                    const int i = i0 + e0 + e;
                    p[s][e] = i < F ? row[i] : 0.f;
                }
            }
        }
#pragma unroll
        for (int e = 0; e < EB; ++e) {
            const int i = i0 + e0 + e;
            float v = 0.f;
#pragma unroll
            for (int s = 0; s < SM; ++s)
                if (s < S) v += p[s][e];
            if (debug_z && i < F) debug_z[(size_t)t * F + i] = v;
            kf[e0 + e] = i < F ? silu(v) : 0.f;
        }
    }
}

// Token t's product rows from the up half's sums u (the select's boundary r
// and its keys kf): this thread's channels KPT tid .. + KPT-1, H in one 16-byte
// (or 8-byte) store per 8 (or 4) channels, zeros past F up to hld (a multiple of 8).
template <int KPT>
__device__ __forceinline__ void up_rows(const UpHalf &up, int F, int t, int2 r, const float (&kf)[KPT],
                                        const float (&u)[KPT])
{
    const int i0 = threadIdx.x * KPT;
    constexpr int VB = KPT % 8 == 0 ? 8 : 4;
#pragma unroll
    for (int e0 = 0; e0 < KPT; e0 += VB) {
        if (i0 + e0 >= up.hld) break;
        uint32_t hw[VB / 2];
#pragma unroll
        for (int e = 0; e < VB / 2; ++e) hw[e] = 0u;
#pragma unroll
        for (int e = 0; e < VB; ++e) {
            const int i = i0 + e0 + e;
            if (i < F) {
                const uint16_t g = topk_on(kf[e0 + e], i, r) ? f2bf(kf[e0 + e]) : (uint16_t)0;
                hw[e >> 1] |= (uint32_t)f2bf(bf2f(g) * u[e0 + e]) << (16 * (e & 1));
                if (up.usave) up.usave[(size_t)t * F + i] = u[e0 + e];
                if (t == 0) up.uidx[i] = i;
            }
        }
        uint16_t *h = up.H + (size_t)t * up.hld + i0 + e0;
        if constexpr (VB == 8) *reinterpret_cast<uint4 *>(h) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        else *reinterpret_cast<uint2 *>(h) = make_uint2(hw[0], hw[1]);
    }
    if (t == 0 && threadIdx.x == 0) *up.ucount = F;
}

// Batched Top-K and top-p of a small batch straight from the gate GEMM's
// split-K partials: token t's keys (sum_split_keys), its select, its flags
// (and with the up half, its product rows).
template <int KPT, int SM, bool MASS>
__global__ __launch_bounds__(1024) void k_sum_select_flags(const float *__restrict__ part, int S, int T, int F,
                                                           int K, float p, float *__restrict__ debug_z,
                                                           uint8_t *__restrict__ act, uint16_t *__restrict__ G,
                                                           uint32_t *__restrict__ ubits, UpHalf up)
{
    __shared__ typename std::conditional<MASS, SelectMassLds, SelectLds>::type L;
    const int t = blockIdx.x;
    float kf[KPT];
    if constexpr (!MASS) select_kth_clear(L);
    sum_split_keys<KPT, SM>(part, S, T, F, t, debug_z, kf);
    // the up half (up to kSelectUpMaxSplits splits; with more, the registers
    // would spill): its sums do not depend on the select, so their loads go
    // out before it
    constexpr bool UP = SM <= kSelectUpMaxSplits;
    float u[KPT];
    if (UP && up.part) sum_split_rows<KPT, SM>(up.part, S, T, F, t, u);
    int2 r;
    if constexpr (MASS) r = select_mass<KPT>(nullptr, F, p, L, kf);
    else r = select_kth<KPT>(nullptr, F, K, L, kf);
    write_flags<KPT>(nullptr, F, r, kf, act + (size_t)t * F, G + (size_t)t * F, ubits);
    if (UP && up.part) up_rows<KPT>(up, F, t, r, kf, u);
}

// Batched Top-K, one 256-thread workgroup per token (d_ff up to
// kTopkLdsKeys): its keys staged into LDS, the select (wg_topk_boundary, the
// same as the decode one), then its flags act[t][i], gate values G[t][i]
// (bf16 key where selected, else 0) and union bits (ORed per 32-channel word
// by one lane of the wavefront; ubits null: none).
__global__ __launch_bounds__(256) void k_topk_select_flags_wg(const float *__restrict__ keys, int F, int K,
                                                               uint8_t *__restrict__ act, uint16_t *__restrict__ G,
                                                               uint32_t *__restrict__ ubits)
{
    constexpr int U = kTopkLdsKeys / 256;
    __shared__ TopkLds L;
    __shared__ float kl[U * 256];
    const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
    const float *s = keys + (size_t)t * F;
    topk_stage_keys<U>(s, F, kl);
    wait_vm_lgkm<0>();
    __syncthreads();
    const int2 r = wg_topk_boundary<U>(s, F, K, L, kl, nullptr, nullptr, 0);
    uint8_t *a = act + (size_t)t * F;
    uint16_t *g = G + (size_t)t * F;
    for (int i0 = tid - lane; i0 < F; i0 += 256) {  // uniform per wavefront
        const int i = i0 + lane;
        bool on = false;
        if (i < F) {
            const float k = kl[i];
            on = topk_on(k, i, r);
            a[i] = on;
            g[i] = on ? f2bf(k) : (uint16_t)0;
        }
        const unsigned long long b = __ballot(on);
        const uint32_t bits = (uint32_t)(b >> (lane & 32));
        if (ubits && (lane & 31) == 0 && bits) atomicOr(&ubits[i >> 5], bits);
    }
}

// Batched top-p: the select of token t, then its flags.
template <int KPT>
__global__ __launch_bounds__(1024) void k_topp_select_flags(const float *__restrict__ keys, int F, float p,
                                                            uint8_t *__restrict__ act, uint16_t *__restrict__ G,
                                                            uint32_t *__restrict__ ubits)
{
    __shared__ SelectMassLds L;
    const int t = blockIdx.x;
    const float *s = keys + (size_t)t * F;
    float kf[KPT > 0 ? KPT : 1];
    load_keys<KPT>(s, F, kf);
    const int2 r = select_mass<KPT>(s, F, p, L, kf);
    write_flags<KPT>(s, F, r, kf, act + (size_t)t * F, G + (size_t)t * F, ubits);
}

// Batched 2:8 structured selection: block (x, y) takes channels
// [256 x, 256 x + 256) (32 whole groups of 8) of tokens [TPB y, TPB y + TPB).
// The block's keys of all its tokens are loaded first (one round trip); then
// per token the keys go through LDS, each channel is ranked within its group
// by (key descending, channel ascending) and the first 2 are kept: act[t][i],
// G[t][i] = bf16 key where kept, else 0. The union bits of the block's tokens
// are ORed in registers and added with one atomic per 32-bit word: TPB tokens
// per block keep the atomics on each bitmap word at T / TPB. With part set (a
// small batch whose gate GEMM split K), a key is the sum of the S split-K
// partials [S][T][F] in split order, then SiLU (as the split-K sum kernel
// computes it; the sums also into debug_z when it is set), and with the up
// half the product rows follow from the same channel's up partials.
template <int TPB>
__global__ __launch_bounds__(256) void k_nm_flags(const float *__restrict__ keys, int T, int F,
                                                  uint8_t *__restrict__ act, uint16_t *__restrict__ G,
                                                  uint32_t *__restrict__ ubits, const float *__restrict__ part,
                                                  int S, float *__restrict__ debug_z, UpHalf up)
{
    constexpr int GROUP = 8, KEEP = 2;
    constexpr int SC = 16 / TPB > 1 ? 16 / TPB : 1;  // partials of a key in flight together
    __shared__ float kl[2][256];
    const int i0 = blockIdx.x * 256, tid = threadIdx.x, lane = tid & 63;
    const int i = i0 + tid;
    const int b = tid & ~(GROUP - 1);
    const int t0 = blockIdx.y * TPB;
    float kv[TPB], uv[TPB];
    if (part) {
        // the gate's partials and (with the up half) the up GEMM's, in flight together
        const bool two = up.part != nullptr;
        float v[TPB];
#pragma unroll
        for (int j = 0; j < TPB; ++j) v[j] = uv[j] = 0.f;
        for (int s0 = 0; s0 < S; s0 += SC) {
            float q[TPB][SC], q2[TPB][SC];
#pragma unroll
            for (int j = 0; j < TPB; ++j)
#pragma unroll
                for (int c = 0; c < SC; ++c) {
                    const int t = t0 + j, sp = s0 + c;
                    const bool in = t < T && i < F && sp < S;
                    q[j][c] = in ? part[((size_t)sp * T + t) * F + i] : 0.f;
                    q2[j][c] = in && two ? up.part[((size_t)sp * T + t) * F + i] : 0.f;
                }
#pragma unroll
            for (int j = 0; j < TPB; ++j)
#pragma unroll
                for (int c = 0; c < SC; ++c)
                    if (s0 + c < S) {
                        v[j] += q[j][c];
                        uv[j] += q2[j][c];
                    }
        }
#pragma unroll
        for (int j = 0; j < TPB; ++j) {
            const int t = t0 + j;
            if (debug_z && t < T && i < F) debug_z[(size_t)t * F + i] = v[j];
            kv[j] = silu(v[j]);
        }
    } else {
#pragma unroll
        for (int j = 0; j < TPB; ++j) {
            const int t = t0 + j;
            kv[j] = t < T && i < F ? keys[(size_t)t * F + i] : 0.f;
        }
    }
    uint32_t acc_bits = 0;
#pragma unroll
    for (int j = 0; j < TPB; ++j) {
        const int t = t0 + j;
        if (t >= T) break;  // the same in every thread of the block
        float *k2 = kl[j & 1];  // two buffers: one barrier per token
        const float k = kv[j];
        k2[tid] = k;
        __syncthreads();
        int rank = 0;
#pragma unroll
        for (int e = 0; e < GROUP; ++e) {
            const float o = k2[b + e];
            rank += i0 + b + e < F && (o > k || (o == k && b + e < tid));
        }
        const bool on = i < F && rank < KEEP;
        if (i < F) {
            const size_t o = (size_t)t * F + i;
            const uint16_t g = on ? f2bf(k) : (uint16_t)0;
            act[o] = on;
            G[o] = g;
            if (up.part) {
                up.H[(size_t)t * up.hld + i] = f2bf(bf2f(g) * uv[j]);
                if (up.usave) up.usave[o] = uv[j];
                if (t == 0) up.uidx[i] = i;
            }
        } else if (up.part && i < up.hld) {
            up.H[(size_t)t * up.hld + i] = 0;
        }
        const unsigned long long m = __ballot(on);
        acc_bits |= (uint32_t)(m >> (lane & 32));
    }
    if ((lane & 31) == 0 && acc_bits) atomicOr(&ubits[i >> 5], acc_bits);
    if (up.part && i == 0 && t0 == 0) *up.ucount = F;
}

// The union bitmap from the flags of T tokens: channel i (one thread) is in
// it when some act[t][i] is set; the scan stops at the first such token. Each
// wavefront writes its 64 channels' two words (one writer per word).
__global__ __launch_bounds__(256) void k_union_flags(const uint8_t *__restrict__ act, int T, int F,
                                                     uint32_t *__restrict__ ubits)
{
    const int i = blockIdx.x * 256 + threadIdx.x, lane = threadIdx.x & 63;
    bool on = false;
    if (i < F)
        for (int t = 0; t < T && !on; ++t) on = act[(size_t)t * F + i] != 0;
    const unsigned long long b = __ballot(on);
    const int w = (i - lane) / 32, words = (F + 31) / 32;
    if (lane == 0 && w < words) ubits[w] = (uint32_t)b;
    if (lane == 32 && w + 1 < words) ubits[w + 1] = (uint32_t)(b >> 32);
}

hipError_t launch_union_flags(const uint8_t *act, int T, int F, uint32_t *ubits, hipStream_t st)
{
    hipLaunchKernelGGL(k_union_flags, dim3((F + 255) / 256), dim3(256), 0, st, act, T, F, ubits);
    return hipGetLastError();
}

hipError_t launch_nm_flags(const float *keys, int T, int F, uint8_t *act, uint16_t *G, uint32_t *ubits,
                           hipStream_t st, const float *part, int S, float *debug_z, const UpHalf &up)
{
    // one token per block up to 16 tokens (enough blocks to fill the GPU),
    // 4 up to 255, then 16: at most T / 4 atomics per bitmap word, and a
    // block's key loads in flight together
    const dim3 block(256);
    const int gx = (F + 255) / 256;
    if (T <= 16)
        hipLaunchKernelGGL(k_nm_flags<1>, dim3(gx, T), block, 0, st, keys, T, F, act, G, ubits, part, S, debug_z, up);
    else if (T < 256)
        hipLaunchKernelGGL(k_nm_flags<4>, dim3(gx, (T + 3) / 4), block, 0, st, keys, T, F, act, G, ubits, part, S,
                           debug_z, up);
    else
        hipLaunchKernelGGL(k_nm_flags<16>, dim3(gx, (T + 15) / 16), block, 0, st, keys, T, F, act, G, ubits, part, S,
                           debug_z, up);
    return hipGetLastError();
}

hipError_t launch_topp_select_flags(const float *keys, int T, int F, float p, uint8_t *act, uint16_t *G,
                                   uint32_t *ubits, hipStream_t st)
{
    const dim3 grid(T), block(1024);
    if (F <= 1024 * 4) hipLaunchKernelGGL(k_topp_select_flags<4>, grid, block, 0, st, keys, F, p, act, G, ubits);
    else if (F <= 1024 * 8) hipLaunchKernelGGL(k_topp_select_flags<8>, grid, block, 0, st, keys, F, p, act, G, ubits);
    else if (F <= 1024 * 16)
        hipLaunchKernelGGL(k_topp_select_flags<16>, grid, block, 0, st, keys, F, p, act, G, ubits);
    else hipLaunchKernelGGL(k_topp_select_flags<0>, grid, block, 0, st, keys, F, p, act, G, ubits);
    return hipGetLastError();
}

bool sum_select_fits(int F, int S) { return F <= 1024 * 16 && S >= 2 && S <= 16; }

hipError_t launch_sum_select_flags(const float *part, int S, int T, int F, int mode, int K, float p, float *debug_z,
                                   uint8_t *act, uint16_t *G, uint32_t *ubits, hipStream_t st, const UpHalf &up)
{
    const dim3 grid(T), block(1024);
    auto go_sm = [&](auto kpt, auto mass) {
        constexpr int KPT = decltype(kpt)::value;
        constexpr bool MASS = decltype(mass)::value;
#define SFFN_SS(SMV) \
    hipLaunchKernelGGL((k_sum_select_flags<KPT, SMV, MASS>), grid, block, 0, st, part, S, T, F, K, p, debug_z, act, G, \
                       ubits, up)
        if (S <= 2) SFFN_SS(2);
        else if (S <= 4) SFFN_SS(4);
        else if (S <= 8) SFFN_SS(8);
        else SFFN_SS(16);
#undef SFFN_SS
    };
    auto go = [&](auto mass) {
        if (F <= 1024 * 4) go_sm(std::integral_constant<int, 4>{}, mass);
        else if (F <= 1024 * 8) go_sm(std::integral_constant<int, 8>{}, mass);
        else go_sm(std::integral_constant<int, 16>{}, mass);
    };
    if (mode == SFFN_TOPP) go(std::true_type{});
    else go(std::false_type{});
    return hipGetLastError();
}

hipError_t launch_topk_select_flags(const float *keys, int T, int F, int K, uint8_t *act, uint16_t *G,
                                   uint32_t *ubits, hipStream_t st)
{
    const dim3 grid(T), block(1024);
    // many tokens: the 256-thread workgroups pack onto the CUs four at a time
    // (2048 tokens of the MoC layer: the training step 1257 us instead of
    // 1286); a few: one 1024-thread select per token is faster (64 tokens:
    // 62.6 us per forward instead of 72)
    if (F <= kTopkLdsKeys && T >= 256) {
        hipLaunchKernelGGL(k_topk_select_flags_wg, grid, dim3(256), 0, st, keys, F, K, act, G, ubits);
        return hipGetLastError();
    }
    if (F <= 1024 * 4) hipLaunchKernelGGL(k_topk_select_flags<4>, grid, block, 0, st, keys, F, K, act, G, ubits);
    else if (F <= 1024 * 8) hipLaunchKernelGGL(k_topk_select_flags<8>, grid, block, 0, st, keys, F, K, act, G, ubits);
    else if (F <= 1024 * 16)
        hipLaunchKernelGGL(k_topk_select_flags<16>, grid, block, 0, st, keys, F, K, act, G, ubits);
    else hipLaunchKernelGGL(k_topk_select_flags<0>, grid, block, 0, st, keys, F, K, act, G, ubits);
    return hipGetLastError();
}

}  // namespace sffn
