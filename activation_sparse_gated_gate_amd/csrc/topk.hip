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
    load_keys<KPT>(s, F, kf);
    const int2 r = select_kth<KPT>(s, F, K, L, kf);
    write_flags<KPT>(s, F, r, kf, act + (size_t)t * F, G + (size_t)t * F, ubits);
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
// [256 x, 256 x + 256) (32 whole groups of 8) of tokens [tpb y, tpb y + tpb).
// Per token the keys go through LDS; each channel is ranked within its group
// by (key descending, channel ascending) and the first 2 are kept: act[t][i],
// G[t][i] = bf16 key where kept, else 0. The union bits of the block's tokens
// are ORed in registers and added with one atomic per 32-bit word: tpb
// tokens per block keep the atomics on each bitmap word at T / tpb.
__global__ __launch_bounds__(256) void k_nm_flags(const float *__restrict__ keys, int T, int F, int tpb,
                                                  uint8_t *__restrict__ act, uint16_t *__restrict__ G,
                                                  uint32_t *__restrict__ ubits)
{
    constexpr int GROUP = 8, KEEP = 2;
    __shared__ float kl[2][256];
    const int i0 = blockIdx.x * 256, tid = threadIdx.x, lane = tid & 63;
    const int i = i0 + tid;
    const int b = tid & ~(GROUP - 1);
    uint32_t acc_bits = 0;
    const int t0 = blockIdx.y * tpb, t1 = min(T, t0 + tpb);
    for (int t = t0; t < t1; ++t) {
        float *k2 = kl[t & 1];  // two buffers: one barrier per token
        const size_t o = (size_t)t * F + i;
        const float k = i < F ? keys[o] : 0.f;
        k2[tid] = k;
        __syncthreads();
        int rank = 0;
#pragma unroll
        for (int e = 0; e < GROUP; ++e) {
            const float v = k2[b + e];
            rank += i0 + b + e < F && (v > k || (v == k && b + e < tid));
        }
        const bool on = i < F && rank < KEEP;
        if (i < F) {
            act[o] = on;
            G[o] = on ? f2bf(k) : (uint16_t)0;
        }
        const unsigned long long m = __ballot(on);
        acc_bits |= (uint32_t)(m >> (lane & 32));
    }
    if ((lane & 31) == 0 && acc_bits) atomicOr(&ubits[i >> 5], acc_bits);
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
                           hipStream_t st)
{
    // one token per block up to 255 tokens (enough blocks to fill the
    // GPU), then up to 16, at most 128 atomics per word
    const int tpb = T < 256 ? 1 : std::min(16, T / 128);
    hipLaunchKernelGGL(k_nm_flags, dim3((F + 255) / 256, (T + tpb - 1) / tpb), dim3(256), 0, st, keys, T, F, tpb,
                       act, G, ubits);
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
