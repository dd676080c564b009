// Per-token Top-K selection over the SiLU gate keys, shared by the decode and
// batched regimes ("Mixture-of-Channels" blog summary, "Dentro il 'mixture'":
// each token keeps its K channels of largest SiLU(gate)).
//
// k_topk_thr finds, per token, the K-th largest key and a tie cutoff; it
// writes no per-channel output. Channel i of token t is then selected iff
//   key > kth  or  (key == kth and i <= cut)
// (topk_on), so ties at the K-th value go to the lower channel indices and
// exactly K channels are selected. The consumer applies that rule where it
// reads the keys anyway: the decode up kernel, or k_topk_flags for a batch
// (which also writes the batch's gate values and union bitmap).
#include "select.h"
#include "sffn_internal.h"

namespace sffn {

// One workgroup (1024 threads) per token; the select itself is select_kth
// (select.h).
template <int KPT>
__global__ __launch_bounds__(1024) void k_topk_thr(const float *__restrict__ keys, int F, int K,
                                                   int2 *__restrict__ thr)
{
    __shared__ SelectLds L;
    const int t = blockIdx.x;
    const int2 r = select_kth<KPT>(keys + (size_t)t * F, F, K, L);
    if (threadIdx.x == 0) thr[t] = r;
}

// Batched: act[t][i] from the thresholds, the gate values the up GEMM reads
// (G[t][i] = bf16 key where selected, else 0), and the union bitmap. Block
// (x, y) takes 256 channels and 8 tokens; the union words are ORed in (the
// bitmap is all zero on entry: the down GEMM clears it after use).
__global__ __launch_bounds__(256) void k_topk_flags(const float *__restrict__ keys, int T, int F,
                                                    const int2 *__restrict__ thr, uint8_t *__restrict__ act,
                                                    uint16_t *__restrict__ G, int W, uint32_t *__restrict__ ubits)
{
    const int i = blockIdx.x * 256 + threadIdx.x, lane = threadIdx.x & 63;
    const int t0 = blockIdx.y * 8, t1 = min(T, t0 + 8);
    bool any = false;
    if (i < F)
        for (int t = t0; t < t1; ++t) {
            const size_t o = (size_t)t * F + i;
            const float k = keys[o];
            const bool on = topk_on(k, i, thr[t]);
            act[o] = on;
            G[o] = on ? f2bf(k) : (uint16_t)0;
            any |= on;
        }
    const unsigned long long m = __ballot(any);
    const int w = i >> 5;
    const uint32_t bits = (uint32_t)(m >> (lane & 32));
    if ((lane & 31) == 0 && w < W && bits) atomicOr(&ubits[w], bits);
}

hipError_t launch_topk_thr(const float *keys, int T, int F, int K, int2 *thr, hipStream_t st)
{
    const dim3 grid(T), block(1024);
    if (F <= 1024 * 4) hipLaunchKernelGGL(k_topk_thr<4>, grid, block, 0, st, keys, F, K, thr);
    else if (F <= 1024 * 8) hipLaunchKernelGGL(k_topk_thr<8>, grid, block, 0, st, keys, F, K, thr);
    else if (F <= 1024 * 16) hipLaunchKernelGGL(k_topk_thr<16>, grid, block, 0, st, keys, F, K, thr);
    else hipLaunchKernelGGL(k_topk_thr<0>, grid, block, 0, st, keys, F, K, thr);
    return hipGetLastError();
}

hipError_t launch_topk_flags(const float *keys, int T, int F, const int2 *thr, uint8_t *act, uint16_t *G, int W,
                             uint32_t *ubits, hipStream_t st)
{
    hipLaunchKernelGGL(k_topk_flags, dim3((F + 255) / 256, (T + 7) / 8), dim3(256), 0, st, keys, T, F, thr, act, G, W,
                       ubits);
    return hipGetLastError();
}

}  // namespace sffn
