// Token grouping for large batches: tokens that keep similar channels are
// put in the same group, and each group runs the up and down products over
// the union of its own tokens' channels, instead of every token over the
// union of the whole batch. The Hugging Face "Daily Papers" listing (query
// "FFN modules"), SPT abstract: a routed FFN batches tokens by the model
// parameters they activate. How tokens are grouped is not given there; here
// it is k-means on the tokens' 0/1 channel masks (Lloyd iterations; the
// centroid of a group is its per-channel frequency), seeded with evenly
// spaced tokens.
//
// With c[g][i] = tokens of group g keeping channel i, n_g = |group g| and
// Q_g = sum_i c[g][i]^2, the squared distance from token t (mask m_t) to the
// centroid c[g] / n_g is |m_t| - (2 S_g n_g - Q_g) / n_g^2 with
// S_g = sum over the channels t keeps of c[g][i], so a token joins the group
// of largest (2 S_g n_g - Q_g) / n_g^2 (ties to the lower group). Counts are
// integers, the scores fp64 from exact integers: the grouping is
// deterministic. Any grouping gives the same outputs: a token's y uses only
// its own channels, whose gate values are zero elsewhere.
#include "device_common.h"
#include "sffn_internal.h"

namespace sffn {

// Mb[t][w]: bit b set when token t keeps channel 32 w + b (G[t][i] != 0).
__global__ __launch_bounds__(256) void k_grp_bits(const uint16_t *__restrict__ G, int T, int F, int W,
                                                  uint32_t *__restrict__ Mb)
{
    const int t = blockIdx.x;
    const uint16_t *g = G + (size_t)t * F;
    for (int w = threadIdx.x; w < W; w += blockDim.x) {
        uint32_t bits = 0;
        const int i0 = 32 * w;
#pragma unroll 8
        for (int b = 0; b < 32; ++b)
            if (i0 + b < F && g[i0 + b] != 0) bits |= 1u << b;
        Mb[(size_t)t * W + w] = bits;
    }
}

// Seeds: token (2 g + 1) T / (2 ng) starts group g; the others join none yet.
__global__ void k_grp_seed(int T, int ng, int *__restrict__ grp)
{
    for (int t = blockIdx.x * blockDim.x + threadIdx.x; t < T; t += gridDim.x * blockDim.x) {
        int g = -1;
        for (int q = 0; q < ng; ++q)
            if (t == (int)(((2LL * q + 1) * T) / (2 * ng))) g = q;
        grp[t] = g;
    }
}

__global__ void k_grp_zero(int *__restrict__ p, size_t count)
{
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < count; i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0;
}

// cnt[g][i] += tokens of group g keeping channel i, for word w of the masks
// and 256 tokens per block (wavefront ballots, then one atomic per counter
// and block).
__global__ __launch_bounds__(256) void k_grp_counts(const uint32_t *__restrict__ Mb, const int *__restrict__ grp,
                                                    int T, int W, int F, int ng, int *__restrict__ cnt)
{
    __shared__ int lc[kMaxTokenGroups][32];
    const int w = blockIdx.x, t = blockIdx.y * 256 + threadIdx.x, lane = threadIdx.x & 63;
    for (int e = threadIdx.x; e < kMaxTokenGroups * 32; e += 256) (&lc[0][0])[e] = 0;
    __syncthreads();
    const uint32_t bits = t < T ? Mb[(size_t)t * W + w] : 0u;
    const int g = t < T ? grp[t] : -1;
    for (int q = 0; q < ng; ++q) {
        const uint32_t mine = g == q ? bits : 0u;
        if (__ballot(mine != 0) == 0) continue;
        for (int b = 0; b < 32; ++b) {
            const int c = __popcll(__ballot((mine >> b) & 1u));
            if (lane == 0 && c) atomicAdd(&lc[q][b], c);
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < ng * 32; e += 256) {
        const int q = e >> 5, b = e & 31, i = 32 * w + b;
        if (i < F && lc[q][b]) atomicAdd(&cnt[(size_t)q * F + i], lc[q][b]);
    }
}

// n[g] += tokens in group g, Q[g] += sum_i cnt[g][i]^2 over block y's slices
// of the tokens and channels (exact integer sums, so the order of the
// atomics does not matter; cnt <= 65536 and F <= 262144 keep Q in 64 bits);
// both start at zero.
__global__ __launch_bounds__(256) void k_grp_stats(const int *__restrict__ grp, const int *__restrict__ cnt, int T,
                                                   int F, int *__restrict__ nsz, long long *__restrict__ Q)
{
    __shared__ long long red[2][4];
    const int g = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int stride = 256 * gridDim.y, first = 256 * blockIdx.y + threadIdx.x;
    long long n = 0, q = 0;
    for (int t = first; t < T; t += stride) n += grp[t] == g;
    for (int i = first; i < F; i += stride) {
        const long long c = cnt[(size_t)g * F + i];
        q += c * c;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        n += __shfl_xor(n, o, 64);
        q += __shfl_xor(q, o, 64);
    }
    if (lane == 0) {
        red[0][wave] = n;
        red[1][wave] = q;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const long long bn = ((red[0][0] + red[0][1]) + red[0][2]) + red[0][3];
        const long long bq = ((red[1][0] + red[1][1]) + red[1][2]) + red[1][3];
        if (bn) atomicAdd(&nsz[g], (int)bn);
        if (bq) atomicAdd(reinterpret_cast<unsigned long long *>(&Q[g]), (unsigned long long)bq);
    }
}

// The assignment step: token t (one block) joins the group of largest
// (2 S_g n_g - Q_g) / n_g^2 among the non-empty groups, ties to the lower g.
__global__ __launch_bounds__(256) void k_grp_assign(const uint32_t *__restrict__ Mb, const int *__restrict__ cnt,
                                                    const int *__restrict__ nsz, const long long *__restrict__ Q,
                                                    int T, int W, int F, int ng, int *__restrict__ grp)
{
    __shared__ long long red[4][kMaxTokenGroups];
    const int t = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    long long S[kMaxTokenGroups];
#pragma unroll
    for (int q = 0; q < kMaxTokenGroups; ++q) S[q] = 0;
    for (int w = threadIdx.x; w < W; w += 256) {
        uint32_t bits = Mb[(size_t)t * W + w];
        while (bits) {
            const int i = 32 * w + __ffs(bits) - 1;
            bits &= bits - 1;
#pragma unroll
            for (int q = 0; q < kMaxTokenGroups; ++q)
                if (q < ng) S[q] += cnt[(size_t)q * F + i];
        }
    }
#pragma unroll
    for (int q = 0; q < kMaxTokenGroups; ++q) {
        long long v = S[q];
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
        if (lane == 0) red[wave][q] = v;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int best = -1;
        double bscore = 0.0;
        for (int q = 0; q < ng; ++q) {
            const long long n = nsz[q];
            if (n <= 0) continue;
            const long long s = ((red[0][q] + red[1][q]) + red[2][q]) + red[3][q];
            const double score = (2.0 * (double)(s * n) - (double)Q[q]) / ((double)n * (double)n);
            if (best < 0 || score > bscore) {
                best = q;
                bscore = score;
            }
        }
        grp[t] = best < 0 ? 0 : best;
    }
}

// Union bitmap of each group: word w of group g has the bits of the
// channels some token of g keeps (cnt > 0).
__global__ void k_grp_union(const int *__restrict__ cnt, int F, int W, int ng, uint32_t *__restrict__ gub)
{
    for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < ng * W; e += gridDim.x * blockDim.x) {
        const int g = e / W, w = e - g * W;
        uint32_t bits = 0;
        for (int b = 0; b < 32 && 32 * w + b < F; ++b) bits |= (uint32_t)(cnt[(size_t)g * F + 32 * w + b] > 0) << b;
        gub[e] = bits;
    }
}

// tmap[s_g + r] = the r-th token of group g in token order (s_g = the sizes
// of the groups before g); one block of 1024 threads per group.
__global__ __launch_bounds__(1024) void k_grp_perm(const int *__restrict__ grp, const int *__restrict__ nsz, int T,
                                                   int *__restrict__ tmap)
{
    __shared__ int scratch[16];
    __shared__ int total;
    const int g = blockIdx.x;
    int s = 0;
    for (int q = 0; q < g; ++q) s += nsz[q];
    int base = 0;
    for (int c0 = 0; c0 < T; c0 += 1024) {
        const int t = c0 + (int)threadIdx.x;
        const int f = t < T && grp[t] == g;
        const int incl = block_incl_scan(f, scratch);
        if (f) tmap[s + base + incl - 1] = t;
        if (threadIdx.x == 1023) total = incl;
        __syncthreads();
        base += total;
        __syncthreads();
    }
}

// xp[p] = x[tmap[p]] (rows of d bf16, d a multiple of 8).
__global__ void k_grp_gather(const uint16_t *__restrict__ x, const int *__restrict__ tmap, int T, int d,
                             uint16_t *__restrict__ xp)
{
    const int c8 = d / 8;
    for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < (size_t)T * c8;
         e += (size_t)gridDim.x * blockDim.x) {
        const int p = (int)(e / c8), c = (int)(e - (size_t)p * c8);
        reinterpret_cast<uint4 *>(xp + (size_t)p * d)[c] = reinterpret_cast<const uint4 *>(x + (size_t)tmap[p] * d)[c];
    }
}

// The batch's union size (into *ncount), then the bitmap cleared for the next
// forward (the grouped products use the groups' bitmaps instead).
__global__ __launch_bounds__(256) void k_union_count_clear(uint32_t *__restrict__ ubits, int W, int *__restrict__ ncount)
{
    __shared__ int red[4];
    int c = 0;
    for (int w = threadIdx.x; w < W; w += 256) c += __popc(ubits[w]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o, 64);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = c;
    __syncthreads();
    if (threadIdx.x == 0) *ncount = ((red[0] + red[1]) + red[2]) + red[3];
    for (int w = threadIdx.x; w < W; w += 256) ubits[w] = 0;
}

hipError_t launch_token_groups(const GroupArgs &a, int *n_host)
{
    const int T = a.T, F = a.F, W = (F + 31) / 32, ng = a.ng;
    hipStream_t st = a.stream;
    hipLaunchKernelGGL(k_union_count_clear, dim3(1), dim3(256), 0, st, a.ubits, W, a.ncount);
    hipLaunchKernelGGL(k_grp_bits, dim3(T), dim3(256), 0, st, a.G, T, F, W, a.Mb);
    hipLaunchKernelGGL(k_grp_seed, dim3((T + 255) / 256), dim3(256), 0, st, T, ng, a.grp);
    const dim3 cgrid(W, (T + 255) / 256);
    for (int it = 0; it <= kTokenGroupIters; ++it) {
        hipLaunchKernelGGL(k_grp_zero, dim3(256), dim3(256), 0, st, a.cnt, (size_t)ng * F);
        hipLaunchKernelGGL(k_grp_zero, dim3(1), dim3(256), 0, st, a.nsz, (size_t)3 * kMaxTokenGroups);
        hipLaunchKernelGGL(k_grp_counts, cgrid, dim3(256), 0, st, a.Mb, a.grp, T, W, F, ng, a.cnt);
        hipLaunchKernelGGL(k_grp_stats, dim3(ng, 32), dim3(256), 0, st, a.grp, a.cnt, T, F, a.nsz, a.Q);
        if (it == kTokenGroupIters) break;
        hipLaunchKernelGGL(k_grp_assign, dim3(T), dim3(256), 0, st, a.Mb, a.cnt, a.nsz, a.Q, T, W, F, ng, a.grp);
    }
    hipLaunchKernelGGL(k_grp_union, dim3((ng * W + 255) / 256), dim3(256), 0, st, a.cnt, F, W, ng, a.gub);
    hipLaunchKernelGGL(k_grp_perm, dim3(ng), dim3(1024), 0, st, a.grp, a.nsz, T, a.tmap);
    hipLaunchKernelGGL(k_grp_gather, dim3(1024), dim3(256), 0, st, a.x, a.tmap, T, a.d, a.xp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // the group sizes size the groups' launches: the one synchronisation
    if ((e = hipMemcpyAsync(n_host, a.nsz, sizeof(int) * ng, hipMemcpyDeviceToHost, st)) != hipSuccess) return e;
    return hipStreamSynchronize(st);
}

}  // namespace sffn
