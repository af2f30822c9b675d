// Device building blocks shared by the gfx950 kernels: 16-byte element
// formats (fp32, bf16 with round-to-nearest-even packing), row loads and
// stores (optionally nontemporal) and wavefront reductions without LDS.
//
// Page names used in comments:
//   [Ovis]   vllm-omni pull request "[Kernel][Ovis-Image] Fuse text/image QK
//            RMSNorm + cat + RoPE into one Triton launch"
#pragma once

#include <cfloat>

#include "qkr_internal.hpp"

namespace qkr {
namespace {

constexpr int kWaves = kThreads / 64;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// Element formats.  A 16-byte vector holds VE elements.
// ---------------------------------------------------------------------------
struct F32 {
    static constexpr int VE = 4;
    __device__ __forceinline__ static uint4 add(const uint4& x, const uint4& r)
    {
        return make_uint4(__float_as_uint(__uint_as_float(x.x) + __uint_as_float(r.x)),
                          __float_as_uint(__uint_as_float(x.y) + __uint_as_float(r.y)),
                          __float_as_uint(__uint_as_float(x.z) + __uint_as_float(r.z)),
                          __float_as_uint(__uint_as_float(x.w) + __uint_as_float(r.w)));
    }
    __device__ __forceinline__ static void unpack(const uint4& v, float* x)
    {
        x[0] = __uint_as_float(v.x); x[1] = __uint_as_float(v.y);
        x[2] = __uint_as_float(v.z); x[3] = __uint_as_float(v.w);
    }
    __device__ __forceinline__ static uint4 pack(const float* x)
    {
        return make_uint4(__float_as_uint(x[0]), __float_as_uint(x[1]),
                          __float_as_uint(x[2]), __float_as_uint(x[3]));
    }
    // fp32 outputs keep the normalised value unrounded.
    __device__ __forceinline__ static void round_trip(float*) {}
    // A table value in the activation type: fp32 already.
    __device__ __forceinline__ static void round_pair(float&, float&) {}
    __device__ __forceinline__ static float sumsq(const uint4& v, float acc)
    {
        acc = fmaf(__uint_as_float(v.x), __uint_as_float(v.x), acc);
        acc = fmaf(__uint_as_float(v.y), __uint_as_float(v.y), acc);
        acc = fmaf(__uint_as_float(v.z), __uint_as_float(v.z), acc);
        return fmaf(__uint_as_float(v.w), __uint_as_float(v.w), acc);
    }
};

struct BF16 {
    static constexpr int VE = 8;
    // The sum of two bf16 vectors rounded once to bf16 (the fp32 sum of two
    // bf16 values is exact unless their exponents differ by more than 15, and
    // then the smaller one is far below half a bf16 step: one rounding either way).
    __device__ __forceinline__ static uint4 add(const uint4& x, const uint4& r);
    __device__ __forceinline__ static void unpack(const uint4& v, float* x)
    {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = __uint_as_float(w[i] << 16);
            x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
    // Round to nearest even (v_cvt_pk_bf16_f32), two values per instruction.
    __device__ __forceinline__ static uint32_t pack2(float lo, float hi)
    {
        const float2_t f = {lo, hi};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
    }
    __device__ __forceinline__ static uint4 pack(const float* x)
    {
        return make_uint4(pack2(x[0], x[1]), pack2(x[2], x[3]), pack2(x[4], x[5]), pack2(x[6], x[7]));
    }
    // Contract rounding: the normalised value is rounded to bf16 before the
    // rotation ([Ovis] kernel review: one documented rounding contract).  One
    // conversion per value with the value in the high half and +0 in the low
    // half gives the rounded value's fp32 bits directly (a packed conversion
    // of two values would need two more instructions to unpack them).
    __device__ __forceinline__ static void round_trip(float* x)
    {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            x[i] = __uint_as_float(pack2(0.0f, x[i]));
    }
    // Two fp32 values rounded to bf16 (a cos/sin table stored in bf16).
    __device__ __forceinline__ static void round_pair(float& a, float& b)
    {
        const uint32_t w = pack2(a, b);
        a = __uint_as_float(w << 16);
        b = __uint_as_float(w & 0xffff0000u);
    }
    // Sum of squares straight from the packed pairs (v_dot2c_f32_bf16: the
    // bf16 products are exact in fp32, accumulation in fp32), so no unpacked
    // copy of the row has to stay live until it is normalised.
    __device__ __forceinline__ static float sumsq(const uint4& v, float acc)
    {
        acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v.x), as_bf16x2(v.x), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v.y), as_bf16x2(v.y), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v.z), as_bf16x2(v.z), acc, false);
        return __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v.w), as_bf16x2(v.w), acc, false);
    }
    __device__ __forceinline__ static bf16x2_t as_bf16x2(uint32_t w) { return __builtin_bit_cast(bf16x2_t, w); }
};

__device__ __forceinline__ uint4 BF16::add(const uint4& x, const uint4& r)
{
    float a[8], b[8];
    unpack(x, a);
    unpack(r, b);
#pragma unroll
    for (int i = 0; i < 8; ++i)
        a[i] += b[i];
    return pack(a);
}

// y / scale rounded to nearest fp32 from the reciprocal inv = 1 / scale
// (computed once, correctly rounded): q = y * inv, the remainder y - scale * q
// exactly by one FMA, and one correction q + r * inv (a reciprocal-based
// division with one Newton-style correction step; the tests compare it with
// the correctly rounded quotient bit for bit).  |y / scale| must stay below
// the fp32 overflow threshold.
__device__ __forceinline__ float div_by_scale(float y, float scale, float inv)
{
    const float q = y * inv;
    const float r = fmaf(-scale, q, y);
    return fmaf(r, inv, q);
}

// Four OCP FP8 E4M3 codes (lowest byte first) of finite fp32 values: clamp to
// +-448 (saturation), then gfx950's packed conversion, which rounds half to
// even on the E4M3 grid and keeps subnormals (checked against the oracle's
// encoder on every tie and its neighbours).
__device__ __forceinline__ uint32_t fp8_e4m3_pack4(float a, float b, float c, float d)
{
    const auto clamp = [](float v) { return fminf(fmaxf(v, -448.0f), 448.0f); };
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(clamp(a), clamp(b), 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(clamp(c), clamp(d), lo, true);
}

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load16(const char* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void store16(char* p, const uint4& v) { *reinterpret_cast<uint4*>(p) = v; }

// Row data is read once and written once: with NT the accesses carry the
// nontemporal hint (streaming, evict-first) so they do not displace the
// small reused operands (weights, positions, planes) from the caches.
template <bool NT>
__device__ __forceinline__ uint4 load_row16(const char* p)
{
    if constexpr (NT) {
        const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
        return make_uint4(v.x, v.y, v.z, v.w);
    } else {
        return load16(p);
    }
}

template <bool NT>
__device__ __forceinline__ void store_row16(char* p, const uint4& v)
{
    if constexpr (NT) {
        const u32x4_t w = {v.x, v.y, v.z, v.w};
        __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(p));
    } else {
        store16(p, v);
    }
}

// 16 bytes per lane from global memory straight into LDS (gfx950's
// global_load_lds_dwordx4): lane i's bytes land at lds + 16 i, lds being
// wave-uniform; no vector registers hold the data.  The write to LDS is
// counted by vmcnt like a load, so readers wait for vmcnt(0) first.  With NT
// the access carries the nontemporal hint.
template <bool NT>
__device__ __forceinline__ void lds_dma16(const char* p, uint4* lds)
{
    __builtin_amdgcn_global_load_lds((const void*)p, (__attribute__((address_space(3))) void*)lds, 16, 0, NT ? 2 : 0);
}

// Raw buffer access (stride 0) through a wave-uniform resource over `bytes`
// bytes at p: the hardware's range check makes a load at an offset >= bytes
// read zeros and drops a store there, so a slot past the end of a row needs
// no branch.  The third descriptor word is the gfx9-family data format.
// NT sets the nontemporal cache policy (as the global forms above).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

template <bool NT>
__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, NT ? 2 : 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}

template <bool NT>
__device__ __forceinline__ void buffer_store16(const uint4& v, __amdgpu_buffer_rsrc_t r, uint32_t off)
{
    const u32x4_t w = {v.x, v.y, v.z, v.w};
    __builtin_amdgcn_raw_buffer_store_b128(w, r, off, 0, NT ? 2 : 0);
}

template <bool NT>
__device__ __forceinline__ void buffer_store8(uint32_t lo, uint32_t hi, __amdgpu_buffer_rsrc_t r, uint32_t off)
{
    typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
    const u32x2_t w = {lo, hi};
    __builtin_amdgcn_raw_buffer_store_b64(w, r, off, 0, NT ? 2 : 0);
}

template <bool NT>
__device__ __forceinline__ void buffer_store4(uint32_t v, __amdgpu_buffer_rsrc_t r, uint32_t off)
{
    __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, NT ? 2 : 0);
}

// ---------------------------------------------------------------------------
// Wavefront reductions without LDS.  DPP moves inside rows of 16 lanes:
// quad_perm xor 1 and xor 2, then row_half_mirror (lane i <- 7 - i within 8
// lanes) and row_mirror (lane i <- 15 - i within 16 lanes); each step adds a
// disjoint partner group, so after log2(L) steps every lane of an L-lane
// group holds the group's sum.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

template <int L>
__device__ __forceinline__ float group_sum(float v)
{
    static_assert((L & (L - 1)) == 0, "groups of a power-of-two number of lanes");
    if constexpr (L >= 2) v += dpp_f32<0xB1>(v);   // quad_perm [1,0,3,2]
    if constexpr (L >= 4) v += dpp_f32<0x4E>(v);   // quad_perm [2,3,0,1]
    if constexpr (L >= 8) v += dpp_f32<0x141>(v);  // row_half_mirror
    if constexpr (L >= 16) v += dpp_f32<0x140>(v); // row_mirror
    if constexpr (L >= 32) v += __shfl_xor(v, 16);
    if constexpr (L >= 64) v += __shfl_xor(v, 32);
    return v;
}

// Whole-wave sum, returned wave-uniform: 16-lane DPP sums, then the four
// row totals read with v_readlane.
__device__ __forceinline__ float wave_sum(float v)
{
    const int iv = __float_as_int(group_sum<16>(v));
    return (__int_as_float(__builtin_amdgcn_readlane(iv, 0)) +
            __int_as_float(__builtin_amdgcn_readlane(iv, 16))) +
           (__int_as_float(__builtin_amdgcn_readlane(iv, 32)) +
            __int_as_float(__builtin_amdgcn_readlane(iv, 48)));
}

__device__ __forceinline__ float bperm(int src_lane, float v)
{
    return __int_as_float(__builtin_amdgcn_ds_bpermute(src_lane << 2, __float_as_int(v)));
}

// Lane src_lane's 16-byte vector.
__device__ __forceinline__ uint4 bperm16(int src_lane, const uint4& v)
{
    const int a = src_lane << 2;
    return make_uint4((uint32_t)__builtin_amdgcn_ds_bpermute(a, (int)v.x), (uint32_t)__builtin_amdgcn_ds_bpermute(a, (int)v.y),
                      (uint32_t)__builtin_amdgcn_ds_bpermute(a, (int)v.z), (uint32_t)__builtin_amdgcn_ds_bpermute(a, (int)v.w));
}

// A wave-uniform value held in a scalar register.  Selecting among such
// values per lane stays a chain of selects: the compiler cannot turn it back
// into a per-lane indexed load from the kernel arguments (a vector memory
// access that would queue behind the row loads).
__device__ __forceinline__ uint32_t uniform(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

template <class T>
__device__ __forceinline__ const T* uniform(const T* ptr)
{
    // readfirstlane yields a signed int: widen each half through uint32_t,
    // or a low word with bit 31 set would sign-extend into the high word.
    const uint64_t v = reinterpret_cast<uint64_t>(ptr);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<const T*>((uint64_t)lo | ((uint64_t)hi << 32));
}

// Axis of pair p (p < kMaxPairs) from the host-built table of 2-bit fields.
// The table is read whole, as two 16-byte vectors, before the per-lane
// selection: a select whose operand is a lone load of one word is turned
// into a branch around that load, one scalar-memory wait per word.
__device__ __forceinline__ int32_t axis_of(const uint32_t (&bits)[kMaxPairs / 16], int32_t p)
{
    static_assert(kMaxPairs / 16 == 8, "the table is two 16-byte vectors");
    const uint4 lo = *reinterpret_cast<const uint4*>(&bits[0]);
    const uint4 hi = *reinterpret_cast<const uint4*>(&bits[4]);
    const uint32_t word[8] = {uniform(lo.x), uniform(lo.y), uniform(lo.z), uniform(lo.w),
                              uniform(hi.x), uniform(hi.y), uniform(hi.z), uniform(hi.w)};
    const int32_t w = p >> 4;
    uint32_t v = word[0];
#pragma unroll
    for (int k = 1; k < 8; ++k)
        v = w == k ? word[k] : v;
    return (int32_t)((v >> ((p & 15) << 1)) & 3u);
}

// 1 / sqrt(v) for v = mean square + eps.  The library routine is the
// hardware reciprocal square root plus a rescaling that matters only for
// subnormal arguments; when eps is a normal number v cannot be subnormal and
// the bare instruction returns the same bits.  `eps_normal` is wave-uniform.
__device__ __forceinline__ float rms_rsqrt(float v, bool eps_normal)
{
    if (eps_normal)
        return __builtin_amdgcn_rsqf(v);
    return rsqrtf(v);
}

// A 4-byte load from global memory through a pointer the compiler cannot
// trace back to a kernel argument (rebuilt by readfirstlane, or selected per
// lane among several): without the address space it becomes a flat load, and
// the wait for a flat load also waits for every vector load issued after it.
__device__ __forceinline__ float load_global(const float* p)
{
    return *(const __attribute__((address_space(1))) float*)p;
}

// The rotation of one pair with every product and sum rounded to fp32 on
// its own: no fused multiply-add (the eager numerics; [Ovis] "Supplemental
// eager bitwise measurements": the preset that reproduced an eager chain
// turned floating-point fusion off).
__device__ __forceinline__ void rotate_unfused(float& a, float& b, float c, float s)
{
#pragma clang fp contract(off)
    const float ac = a * c, bs = b * s, bc = b * c, as = a * s;
    a = ac - bs;
    b = bc + as;
}

// Orders one wave's LDS writes before its later LDS reads of other lanes'
// data (and those reads before the next writes).  LDS executes a wave's
// operations in order, so this only keeps the compiler from moving them.
__device__ __forceinline__ void wave_lds_order()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace
}  // namespace qkr
