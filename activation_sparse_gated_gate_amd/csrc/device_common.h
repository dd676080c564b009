// Device helpers shared by the HIP kernels: 128-bit loads of 8 elements,
// bf16 widening, wavefront reductions and scans, Top-K key encoding.
#pragma once

#include <type_traits>

#include <hip/hip_runtime.h>

#include <cstdint>

namespace sffn {

typedef uint16_t bf16_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

// bf16 is the upper half of an IEEE binary32: widening is a shift.
__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Eight consecutive elements: one 128-bit load for bf16, two for fp32.
template <typename T>
struct Ld8;

template <>
struct Ld8<bf16_t> {
    struct raw {
        uint4 q;
    };
    static __device__ __forceinline__ raw load(const bf16_t *p)
    {
        raw r;
        r.q = *reinterpret_cast<const uint4 *>(p);
        return r;
    }
    // Streaming load for weights read once per forward (non-temporal hint).
    static __device__ __forceinline__ raw load_nt(const bf16_t *p)
    {
        const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
        raw r;
        r.q = make_uint4(v.x, v.y, v.z, v.w);
        return r;
    }
    static __device__ __forceinline__ raw zero()
    {
        raw r;
        r.q = make_uint4(0, 0, 0, 0);
        return r;
    }
    static __device__ __forceinline__ void store(bf16_t *p, const raw &r)
    {
        *reinterpret_cast<uint4 *>(p) = r.q;
    }
    static __device__ __forceinline__ void cvt(const raw &r, float v[8])
    {
        v[0] = bf_lo(r.q.x); v[1] = bf_hi(r.q.x);
        v[2] = bf_lo(r.q.y); v[3] = bf_hi(r.q.y);
        v[4] = bf_lo(r.q.z); v[5] = bf_hi(r.q.z);
        v[6] = bf_lo(r.q.w); v[7] = bf_hi(r.q.w);
    }
};

template <>
struct Ld8<float> {
    struct raw {
        float4 a, b;
    };
    static __device__ __forceinline__ raw load(const float *p)
    {
        raw r;
        r.a = reinterpret_cast<const float4 *>(p)[0];
        r.b = reinterpret_cast<const float4 *>(p)[1];
        return r;
    }
    static __device__ __forceinline__ raw load_nt(const float *p)
    {
        const f32x4_t a = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(p));
        const f32x4_t b = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(p) + 1);
        raw r;
        r.a = make_float4(a.x, a.y, a.z, a.w);
        r.b = make_float4(b.x, b.y, b.z, b.w);
        return r;
    }
    static __device__ __forceinline__ void add(raw &r, const raw &o)
    {
        r.a.x += o.a.x; r.a.y += o.a.y; r.a.z += o.a.z; r.a.w += o.a.w;
        r.b.x += o.b.x; r.b.y += o.b.y; r.b.z += o.b.z; r.b.w += o.b.w;
    }
    static __device__ __forceinline__ raw zero()
    {
        raw r;
        r.a = make_float4(0.f, 0.f, 0.f, 0.f);
        r.b = r.a;
        return r;
    }
    static __device__ __forceinline__ void store(float *p, const raw &r)
    {
        reinterpret_cast<float4 *>(p)[0] = r.a;
        reinterpret_cast<float4 *>(p)[1] = r.b;
    }
    static __device__ __forceinline__ void cvt(const raw &r, float v[8])
    {
        v[0] = r.a.x; v[1] = r.a.y; v[2] = r.a.z; v[3] = r.a.w;
        v[4] = r.b.x; v[5] = r.b.y; v[6] = r.b.z; v[7] = r.b.w;
    }
};

// c + sum of the 8 products w[e] * x[e], accumulated in fp32. For bf16 x bf16
// this is four packed v_dot2_f32_bf16 (bf16 products are exact in fp32).
template <typename TW, typename TX>
__device__ __forceinline__ float dot8(const typename Ld8<TW>::raw &w, const typename Ld8<TX>::raw &x, float c)
{
    if constexpr (sizeof(TW) == 2 && sizeof(TX) == 2) {
        c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.q.x), __builtin_bit_cast(bf16x2_t, x.q.x), c, false);
        c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.q.y), __builtin_bit_cast(bf16x2_t, x.q.y), c, false);
        c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.q.z), __builtin_bit_cast(bf16x2_t, x.q.z), c, false);
        c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.q.w), __builtin_bit_cast(bf16x2_t, x.q.w), c, false);
        return c;
    } else {
        float wv[8], xv[8];
        Ld8<TW>::cvt(w, wv);
        Ld8<TX>::cvt(x, xv);
#pragma unroll
        for (int e = 0; e < 8; ++e) c = fmaf(wv[e], xv[e], c);
        return c;
    }
}

// Sum over aligned groups of G lanes (G a power of two <= 64). Every lane of a
// group ends with the same bits: each butterfly step adds the same two
// operands on both partner lanes, and fp32 addition commutes exactly.
template <int G>
__device__ __forceinline__ float group_sum(float v)
{
    static_assert(G == 1 || G == 2 || G == 4 || G == 8 || G == 16 || G == 32 || G == 64, "power of two <= 64");
    // within 16 lanes by DPP moves (every lane ends with its group's sum):
    // pairs, quads, the two quads of 8 lanes (half-row mirror), the two
    // halves of 16 (row mirror); then shuffles across rows
#define SFFN_DPP_F(x, ctrl) __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), ctrl, 0xf, 0xf, false))
    if constexpr (G >= 2) v += SFFN_DPP_F(v, 0xb1);   // quad_perm [1,0,3,2]
    if constexpr (G >= 4) v += SFFN_DPP_F(v, 0x4e);   // quad_perm [2,3,0,1]
    if constexpr (G >= 8) v += SFFN_DPP_F(v, 0x141);  // row_half_mirror
    if constexpr (G >= 16) v += SFFN_DPP_F(v, 0x140); // row_mirror
#undef SFFN_DPP_F
    if constexpr (G >= 32) v += __shfl_xor(v, 16, 64);
    if constexpr (G >= 64) v += __shfl_xor(v, 32, 64);
    return v;
}

// Inclusive prefix sum across one 64-lane wavefront, in registers with DPP
// moves: shifts by 1, 2, 4 and 8 within each row of 16 lanes (a lane with no
// source adds 0), then lane 15 of rows 0 and 2 into rows 1 and 3, then lane
// 31 into rows 2 and 3. Every lane must be active.
__device__ __forceinline__ int wave_incl_scan(int v)
{
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);  // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);  // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);  // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);  // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
    return v;
}

// Inclusive prefix sum across the whole workgroup (blockDim.x a multiple of
// 64, at most 1024). `scratch` holds one int per wavefront. Contains
// barriers: every thread of the block must call it.
__device__ __forceinline__ int block_incl_scan(int v, int *scratch)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nw = blockDim.x >> 6;
    v = wave_incl_scan(v);
    if (lane == 63) scratch[wave] = v;
    __syncthreads();
    int add = 0;
    for (int w = 0; w < wave; ++w) add += scratch[w];
    (void)nw;
    __syncthreads();
    return v + add;
}

// Order-preserving map from fp32 to uint32 (larger float -> larger key).
// -0 is folded onto +0 so that equal values get equal keys.
__device__ __forceinline__ uint32_t f2key(float f)
{
    uint32_t u = __float_as_uint(f == 0.f ? 0.f : f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// The same for 64-bit values: the DPP moves of wave_incl_scan on the two
// 32-bit halves, then one 64-bit add per step (exact: integer sums).
__device__ __forceinline__ unsigned long long wave_incl_scan_u64(unsigned long long v)
{
    auto step = [&v](auto ctrl, auto row_mask, auto bound) {
        const uint32_t lo = __builtin_amdgcn_update_dpp(0u, (uint32_t)v, decltype(ctrl)::value,
                                                        decltype(row_mask)::value, 0xf, decltype(bound)::value);
        const uint32_t hi = __builtin_amdgcn_update_dpp(0u, (uint32_t)(v >> 32), decltype(ctrl)::value,
                                                        decltype(row_mask)::value, 0xf, decltype(bound)::value);
        v += ((unsigned long long)hi << 32) | lo;
    };
    step(std::integral_constant<int, 0x111>{}, std::integral_constant<int, 0xf>{}, std::true_type{});   // row_shr:1
    step(std::integral_constant<int, 0x112>{}, std::integral_constant<int, 0xf>{}, std::true_type{});   // row_shr:2
    step(std::integral_constant<int, 0x114>{}, std::integral_constant<int, 0xf>{}, std::true_type{});   // row_shr:4
    step(std::integral_constant<int, 0x118>{}, std::integral_constant<int, 0xf>{}, std::true_type{});   // row_shr:8
    step(std::integral_constant<int, 0x142>{}, std::integral_constant<int, 0xa>{}, std::false_type{});  // row_bcast:15
    step(std::integral_constant<int, 0x143>{}, std::integral_constant<int, 0xc>{}, std::false_type{});  // row_bcast:31
    return v;
}

// inverse of f2key (for the keys f2key produces)
__device__ __forceinline__ float key2f(uint32_t k)
{
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Top-p masses (select_mass and the workgroup top-p select): the fixed-point
// weight of key v against the token's largest key top, round(exp(v - top)
// 2^44) with exp in fp32 (24 significant bits), so every sum of them is exact
// and independent of order; and the target mass ceil(p Z) of a total Z,
// clamped to [1, Z].
__device__ __forceinline__ unsigned long long topp_mass(float v, float top)
{
    return (unsigned long long)(expf(v - top) * 17592186044416.0f + 0.5f);  // 2^44
}

__device__ __forceinline__ unsigned long long topp_target(float p, unsigned long long Z)
{
    const unsigned long long T = (unsigned long long)ceil((double)p * (double)Z);
    return T < 1ull ? 1ull : T > Z ? Z : T;
}

// Operand types of __builtin_amdgcn_global_load_lds (global source, LDS
// destination: each lane's bytes land at the destination + lane * size).
typedef __attribute__((address_space(1))) const void gmem_t;
typedef __attribute__((address_space(3))) void lmem_t;

// s_waitcnt: at most N vector-memory operations of this wavefront in flight,
// and every LDS operation done.
template <int N>
__device__ __forceinline__ void wait_vm_lgkm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
}

// Top-K membership of channel i from its token's threshold: thr.x is the
// K-th largest key (f2key encoding), thr.y the last channel index kept among
// the keys equal to it.
__device__ __forceinline__ bool topk_on(float g, int i, int2 thr)
{
    const uint32_t k = f2key(g), kth = (uint32_t)thr.x;
    return k > kth || (k == kth && i <= thr.y);
}

__device__ __forceinline__ float silu(float z) { return z / (1.f + expf(-z)); }

// fp32 -> bf16, round to nearest even (finite inputs), and back.
__device__ __forceinline__ uint16_t f2bf(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

}  // namespace sffn
