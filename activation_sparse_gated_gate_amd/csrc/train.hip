// Training side of the layer: the stored activations of a forward and the
// set-up of the backward over them.
//
// "Mixture-of-Channels" blog summary, "Dentro il 'mixture'": in training only
// the masked parts of the FFN activations are kept for the backward, and the
// rest is rebuilt when it is needed. Here a training forward keeps, per
// token, its active channels (ascending) with their gate pre-activation z and
// up value u = x . W_up[i]: cap slots per token instead of d_ff. The backward
// rebuilds g(z), g'(z) and h = g(z) u from them. The GEMMs of the backward
// run on the union path's MFMA kernel (batched.hip); the kernels here move
// the stored rows in and out of the layouts those GEMMs read.
#include <algorithm>

#include "compact.h"
#include "device_common.h"
#include "sffn_internal.h"

namespace sffn {

// Token t (one block): the channels the mode keeps, from the forward's dense
// z (the same fp32 value the gate's select compared), its up values and its
// flags; the first cap of them are stored, cnt[t] = how many there are.
__global__ __launch_bounds__(256) void k_save(const float *__restrict__ zd, const float *__restrict__ ud,
                                              const uint8_t *__restrict__ act, int F, int mode, float tau, int cap,
                                              int32_t *__restrict__ cnt, int32_t *__restrict__ idx,
                                              float *__restrict__ zo, float *__restrict__ uo)
{
    __shared__ int scratch[5];
    const int t = blockIdx.x;
    const float *zt = zd + (size_t)t * F, *ut = ud + (size_t)t * F;
    const uint8_t *at = act + (size_t)t * F;
    const bool flags = mode == SFFN_TOPK || mode == SFFN_TOPK_2_8 || mode == SFFN_TOPP;
    const bool all = mode == SFFN_DENSE_SILU;
    auto on8 = [&](int i0, bool f[8]) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int i = i0 + e;
            f[e] = i < F && (all || (flags ? at[i] != 0 : zt[i] > tau));
        }
    };
    int32_t *io = idx + (size_t)t * cap;
    float *zt_o = zo + (size_t)t * cap, *ut_o = uo + (size_t)t * cap;
    const int c = emit_ordered_fn(
        F, on8,
        [&](int pos, int i) {
            if (pos < cap) {
                io[pos] = i;
                zt_o[pos] = zt[i];
                ut_o[pos] = ut[i];
            }
        },
        scratch);
    if (threadIdx.x == 0) cnt[t] = c;
}

hipError_t launch_save(const float *zd, const float *ud, const uint8_t *act, int T, int F, int mode, float tau,
                       const Saved &sv, hipStream_t st)
{
    hipLaunchKernelGGL(k_save, dim3(T), dim3(256), 0, st, zd, ud, act, F, mode, tau, sv.cap, sv.cnt, sv.idx, sv.z,
                       sv.u);
    return hipGetLastError();
}

// ZU = (NaN, 0) everywhere (every channel off), and token columns [T, tp) of
// the first F rows of the transposed buffers zeroed (the weight-gradient
// products read whole 8-token chunks).
__global__ __launch_bounds__(256) void k_bwd_clear(float2 *__restrict__ ZU, size_t TF, uint16_t *__restrict__ dut,
                                                   uint16_t *__restrict__ dzt, uint16_t *__restrict__ ht, int F, int T,
                                                   int tp)
{
    const size_t g = (size_t)blockIdx.x * blockDim.x + threadIdx.x, stride = (size_t)gridDim.x * blockDim.x;
    const float2 off = make_float2(__uint_as_float(0x7fc00000u), 0.f);
    for (size_t e = g; e < TF; e += stride) ZU[e] = off;
    const int padw = tp - T;
    if (padw > 0)
        for (size_t e = g; e < (size_t)F * padw; e += stride) {
            const size_t o = (e / padw) * tp + T + e % padw;
            dut[o] = 0;
            dzt[o] = 0;
            ht[o] = 0;
        }
}

// Token t (one block): its stored (z, u) into ZU[t][i]. Channel indices
// outside [0, F) are skipped.
__global__ __launch_bounds__(256) void k_bwd_scatter(const int32_t *__restrict__ cnt, const int32_t *__restrict__ idx,
                                                     const float *__restrict__ z, const float *__restrict__ u, int cap,
                                                     int F, float2 *__restrict__ ZU)
{
    const int t = blockIdx.x;
    const int c = min(cnt[t], cap);
    for (int s = threadIdx.x; s < c; s += 256) {
        const size_t o = (size_t)t * cap + s;
        const int i = idx[o];
        if (i < 0 || i >= F) continue;
        ZU[(size_t)t * F + i] = make_float2(z[o], u[o]);
    }
}

// Token t (one block): its whole row of ZU at once, (NaN, 0) for every
// channel and the stored (z, u) where it has them, built in LDS and written
// with coalesced stores (one pass over ZU instead of a clear and a scatter;
// d_ff up to kFillMax). Stored channel indices are unique (ascending, as
// k_save writes them); indices outside [0, F) are skipped.
constexpr int kFillMax = 6144;
__global__ __launch_bounds__(256) void k_bwd_fill(const int32_t *__restrict__ cnt, const int32_t *__restrict__ idx,
                                                  const float *__restrict__ z, const float *__restrict__ u, int cap,
                                                  int F, float2 *__restrict__ ZU)
{
    __shared__ float2 row[kFillMax];
    const int t = blockIdx.x, tid = threadIdx.x;
    const float2 off = make_float2(__uint_as_float(0x7fc00000u), 0.f);
    for (int i = tid; i < F; i += 256) row[i] = off;
    __syncthreads();
    const int c = min(cnt[t], cap);
    for (int s = tid; s < c; s += 256) {
        const size_t o = (size_t)t * cap + s;
        const int i = idx[o];
        if (i >= 0 && i < F) row[i] = make_float2(z[o], u[o]);
    }
    __syncthreads();
    float2 *dst = ZU + (size_t)t * F;
    for (int i = tid; i < F; i += 256) dst[i] = row[i];
}

// The union bitmap: channel i (one thread) is in it when some token stored
// it, i.e. some ZU[t][i].x is not NaN; the scan stops at the first such
// token. Each wavefront writes its 64 channels' two words (no atomics: every
// word has one writer).
__global__ __launch_bounds__(256) void k_bwd_union(const float2 *__restrict__ ZU, int T, int F, int words,
                                                   uint32_t *__restrict__ ubits)
{
    const int i = blockIdx.x * 256 + threadIdx.x, lane = threadIdx.x & 63;
    bool on = false;
    if (i < F) {
        const float *zc = reinterpret_cast<const float *>(ZU) + 2 * (size_t)i;
        for (int t = 0; t < T && !on; ++t) {
            const float v = zc[2 * (size_t)t * F];
            on = v == v;
        }
    }
    const unsigned long long b = __ballot(on);
    const int w = (i - lane) / 32;
    if (lane == 0 && w < words) ubits[w] = (uint32_t)b;
    if (lane == 32 && w + 1 < words) ubits[w + 1] = (uint32_t)(b >> 32);
}

// The ascending union list from the bitmap: one block of 1024 threads, each
// owning a contiguous run of words (at most 8 for d_ff <= 2^18).
__global__ __launch_bounds__(1024) void k_bwd_list(const uint32_t *__restrict__ ubits, int words,
                                                   int32_t *__restrict__ uidx, int *__restrict__ ucount)
{
    __shared__ int scratch[16];
    const int wpt = (words + 1023) / 1024;
    const int w0 = threadIdx.x * wpt;
    int c = 0;
    for (int q = 0; q < wpt; ++q)
        if (w0 + q < words) c += __popc(ubits[w0 + q]);
    const int incl = block_incl_scan(c, scratch);
    int pos = incl - c;
    for (int q = 0; q < wpt && w0 + q < words; ++q) {
        uint32_t v = ubits[w0 + q];
        while (v) {
            const int b = __ffs(v) - 1;
            v &= v - 1;
            uidx[pos++] = (w0 + q) * 32 + b;
        }
    }
    if (threadIdx.x == 1023) *ucount = incl;
}

// x and dy [T][d] -> [d][tp] (z = 0: x, 1: dy), zero for tokens past T;
// 64 x 64 tiles through LDS.
__global__ __launch_bounds__(256) void k_transpose_pad(const uint16_t *__restrict__ x, const uint16_t *__restrict__ dy,
                                                       uint16_t *__restrict__ xt, uint16_t *__restrict__ dyt, int T,
                                                       int d, int tp)
{
    __shared__ uint16_t tile[64][66];
    const uint16_t *src = blockIdx.z ? dy : x;
    uint16_t *dst = blockIdx.z ? dyt : xt;
    const int t0 = blockIdx.x * 64, k0 = blockIdx.y * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    for (int r = ty; r < 64; r += 4) {
        const int t = t0 + r, k = k0 + tx;
        tile[r][tx] = (t < T && k < d) ? src[(size_t)t * d + k] : (uint16_t)0;
    }
    __syncthreads();
    for (int r = ty; r < 64; r += 4) {
        const int k = k0 + r, t = t0 + tx;
        if (k < d && t < tp) dst[(size_t)k * tp + t] = tile[tx][r];
    }
}

hipError_t launch_bwd_setup(const Saved &sv, int T, int F, int d, int tp, float2 *ZU, uint32_t *ubits,
                            int32_t *uidx, int *ucount, uint16_t *dut, uint16_t *dzt, uint16_t *ht,
                            const uint16_t *x, const uint16_t *dy, uint16_t *xt, uint16_t *dyt, hipStream_t st)
{
    const int words = (F + 31) / 32;
    const size_t TF = (size_t)T * F;
    const int blocks = (int)std::min<size_t>(4096, (TF + 255) / 256 + 1);
    if (F <= kFillMax) {
        // one pass over ZU; the clear kernel only zeroes the padding (if any)
        if (tp > T) hipLaunchKernelGGL(k_bwd_clear, dim3(blocks), dim3(256), 0, st, ZU, 0, dut, dzt, ht, F, T, tp);
        hipLaunchKernelGGL(k_bwd_fill, dim3(T), dim3(256), 0, st, sv.cnt, sv.idx, sv.z, sv.u, sv.cap, F, ZU);
    } else {
        hipLaunchKernelGGL(k_bwd_clear, dim3(blocks), dim3(256), 0, st, ZU, TF, dut, dzt, ht, F, T, tp);
        hipLaunchKernelGGL(k_bwd_scatter, dim3(T), dim3(256), 0, st, sv.cnt, sv.idx, sv.z, sv.u, sv.cap, F, ZU);
    }
    hipLaunchKernelGGL(k_bwd_union, dim3((F + 255) / 256), dim3(256), 0, st, ZU, T, F, words, ubits);
    hipLaunchKernelGGL(k_bwd_list, dim3(1), dim3(1024), 0, st, ubits, words, uidx, ucount);
    hipLaunchKernelGGL(k_transpose_pad, dim3((tp + 63) / 64, (d + 63) / 64, 2), dim3(256), 0, st, x, dy, xt, dyt, T,
                       d, tp);
    return hipGetLastError();
}

}  // namespace sffn
