// gfx950 kernels: per-head QK RMSNorm + RoPE, plain row RMSNorm, ViT cos/sin
// setup.  All of them are HBM-bound streams: rows move as 128-bit vectors,
// reductions stay inside a wavefront (DPP), cos/sin are computed in registers
// once per (token, pair) and shared by every head of the token.  No LDS tree,
// no atomics, no MFMA (there is no dense contraction in this path).
//
// Page names used in comments:
//   [Ovis]   vllm-omni pull request "[Kernel][Ovis-Image] Fuse text/image QK
//            RMSNorm + cat + RoPE into one Triton launch"
//   [Vulkan] vllm.cpp pull request "perf(vulkan): decode RmsNorm ran on ONE
//            workgroup -- 7.85 -> 1.59 ms/token"
//   [IMROPE] llama.cpp fork pull request "hrx: the multi-section rotation of
//            Qwen3-VL runs on the device, not on the CPU"
//   [ViT]    vLLM API page "vllm.model_executor.layers.rotary_embedding.
//            mrope_vit_setup"
//   [VecRMS] vLLM pull request "Vectorize RMS norm variance using
//            vectorize_read_with_alignment"
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
    // rotation ([Ovis] kernel review: one documented rounding contract).
    __device__ __forceinline__ static void round_trip(float* x)
    {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t w = pack2(x[2 * i], x[2 * i + 1]);
            x[2 * i] = __uint_as_float(w << 16);
            x[2 * i + 1] = __uint_as_float(w & 0xffff0000u);
        }
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

__device__ __forceinline__ float bperm(int src_lane, float v);

template <int L>
__device__ __forceinline__ float group_sum(float v)
{
    if constexpr ((L & (L - 1)) != 0) {
        // Groups of L consecutive lanes, L not a power of two (rows that are
        // not a power-of-two number of vector pairs, e.g. head_dim 80 bf16):
        // every lane adds the group's values in the same lane order, so all
        // lanes of a group hold the identical sum.
        const int base = ((int)(threadIdx.x & 63) / L) * L;
        float s = 0.0f;
#pragma unroll
        for (int k = 0; k < L; ++k)
            s += bperm(base + k, v);
        return s;
    }
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

// ---------------------------------------------------------------------------
// Rotation operands of one (token, pair), fetched before the row data so that
// cos/sin are ready while the rows are still in flight.
//   ROPE 1: the token's positions, one per plane (wave-uniform scalar loads,
//           counted apart from the vector loads), and inv_freq[p].
//   ROPE 2: the cos/sin the setup wrote for the pair's axis.
// ---------------------------------------------------------------------------
// The token's position on each plane (wave-uniform).
struct TokenPositions {
    int32_t t, h, w, e;
};

struct PairOperand {
    float inv_or_c;   // inv_freq[p] (ROPE 1) or cos (ROPE 2)
    float s;          // sin (ROPE 2)
    int32_t axis;
};

template <int ROPE>
__device__ __forceinline__ PairOperand fetch_pair(const RopeArgs& r, const VitGridArgs& v, int64_t t, int32_t p)
{
    PairOperand o;
    if constexpr (ROPE == 3) {
        // ViT: contiguous t/h/w sections of the pairs, one inverse-frequency
        // ladder per axis.
        o.axis = pair_axis(kPosAxes, r.sec, p);
        const float* inv = o.axis == 0 ? v.inv[0] : (o.axis == 1 ? v.inv[1] : v.inv[2]);
        const int32_t off = o.axis == 0 ? 0 : (o.axis == 1 ? r.sec[0] : r.sec[0] + r.sec[1]);
        o.inv_or_c = inv[p - off];
        o.s = 0.0f;
        return o;
    }
    o.axis = pair_axis(r.mode, r.sec, p);
    if constexpr (ROPE == 2) {
        const int64_t idx = ((int64_t)o.axis * r.planes_tokens + t) * r.half + p;
        o.inv_or_c = r.cos_planes[idx];
        o.s = r.sin_planes[idx];
    } else {
        o.inv_or_c = r.inv_freq[p];
        o.s = 0.0f;
    }
    return o;
}

// (t, h, w) of ViT token `tok` for the fused mode, wave-uniform: the grid is
// the last one whose first token has been reached (a select loop, scalar),
// then frame, spatial-merge block and cell ([ViT] setup kernel's token
// order), with the host's divisors instead of hardware divides.
__device__ __forceinline__ TokenPositions vit_token_positions(const VitGridArgs& v, uint32_t tok)
{
    // Scalar fields only: selecting whole structs out of the kernel-argument
    // table would make the compiler copy the table to private memory.
    uint32_t start = (uint32_t)v.cu[0];
    uint32_t a_d = v.div_area[0].d, a_m = v.div_area[0].m, a_l = v.div_area[0].l;
    uint32_t w_d = v.div_mw[0].d, w_m = v.div_mw[0].m, w_l = v.div_mw[0].l;
    for (int k = 1; k < v.num_grids; ++k) {
        const bool in_k = tok >= (uint32_t)v.cu[k];
        start = in_k ? (uint32_t)v.cu[k] : start;
        a_d = in_k ? v.div_area[k].d : a_d;
        a_m = in_k ? v.div_area[k].m : a_m;
        a_l = in_k ? v.div_area[k].l : a_l;
        w_d = in_k ? v.div_mw[k].d : w_d;
        w_m = in_k ? v.div_mw[k].m : w_m;
        w_l = in_k ? v.div_mw[k].l : w_l;
    }
    const FastDiv da{a_d, a_m, a_l}, dmw{w_d, w_m, w_l};
    const uint32_t local = tok - start;
    const uint32_t t = fast_div(local, da);
    const uint32_t rem = local - t * da.d;
    const uint32_t bh = fast_div(rem, dmw);
    const uint32_t r = rem - bh * dmw.d;
    const uint32_t bw = fast_div(r, v.div_mm);
    const uint32_t r2 = r - bw * v.div_mm.d;
    const uint32_t mh = fast_div(r2, v.div_m);
    TokenPositions p;
    p.t = (int32_t)t;
    p.h = (int32_t)(bh * v.div_m.d + mh);
    p.w = (int32_t)(bw * v.div_m.d + (r2 - mh * v.div_m.d));
    p.e = 0;
    return p;
}

// The angle is the fp32 product of the fp32 position and inv_freq[p] ([ViT]
// setup kernel); sincosf is the accurate device-library routine (its argument
// reduction holds far past the 8191 rad these workloads reach).
template <int ROPE>
__device__ __forceinline__ void pair_cos_sin(const PairOperand& o, const TokenPositions& pos, float& c, float& s)
{
    if constexpr (ROPE == 2) {
        c = o.inv_or_c;
        s = o.s;
    } else {
        const int32_t q = o.axis == 0 ? pos.t : (o.axis == 1 ? pos.h : (o.axis == 2 ? pos.w : pos.e));
        const float theta = (float)q * o.inv_or_c;
        sincosf(theta, &s, &c);
    }
}

// Row addressing of one tensor at one (batch, token): address of head 0 and
// the head stride, for the input view of the token's stream and for the
// joint output.  Pointers stay derived from the kernel-argument pointers so
// the accesses are global (not flat) memory operations.
struct TensorRows {
    const char* in;
    char* out;
    int64_t in_sh, out_sh;
};

__device__ __forceinline__ TensorRows tensor_rows(const TensorArgs& t, bool s1, int32_t b, int32_t tok,
                                                  int32_t ltok)
{
    TensorRows r;
    const char* in = s1 ? t.in[1] : t.in[0];
    r.in = in + (int64_t)b * (s1 ? t.in_sb[1] : t.in_sb[0]) + (int64_t)ltok * (s1 ? t.in_st[1] : t.in_st[0]);
    r.in_sh = s1 ? t.in_sh[1] : t.in_sh[0];
    r.out = t.out + (int64_t)b * t.out_sb + (int64_t)tok * t.out_st;
    r.out_sh = t.out_sh;
    return r;
}

// ---------------------------------------------------------------------------
// Per-(token, head) RMSNorm + RoPE.
//
// Work unit (tile): one wavefront takes NP passes over RPP = 64 / LPR rows of
// one token; LPR lanes share a row and every lane owns two 16-byte vectors of
// it.  With the NeoX pairing a lane owns vectors j and j + R/(2 VE), so every
// rotated pair (p, p + R/2) is lane-local; with the adjacent pairing the pairs
// sit inside one vector.
//
// Order of work in a wave:
//   1. the rotation operands (the token's positions by scalar loads, the
//      lane's inv_freq or planes entry), then the weights, then every row
//      load of the tile.  All vector loads are unconditional (lanes without
//      a vector of their own re-read one of their row, a cache hit), so the
//      compiler can count them and wait only for the operands;
//   2. cos/sin of the token's pairs (lane i: pair i) while the rows are in
//      flight, handed to the lanes that need them with ds_bpermute;
//   3. per row: DPP sum of squares over the row's LPR lanes, normalise, round
//      per the contract, rotate, store (stores only for owned vectors).
//
// ROPE: 0 norm only, 1 positions + inv_freq (1D / AXES / IMROPE chosen at run
// time), 2 cos/sin planes, 3 ViT positions computed from the grid table.
// ---------------------------------------------------------------------------
template <class E, int LPR, int NP, int ROPE, int PAIRING, bool NT>
__global__ __launch_bounds__(kThreads) void norm_rope_kernel(const NormRopeArgs a)
{
    constexpr int VE = E::VE;
    constexpr int RPP = 64 / LPR;
    constexpr int RPW = RPP * NP;
    constexpr bool ROT = ROPE != 0;

    const int lane = threadIdx.x & 63;
    // Tile coordinates are wave-uniform and stay in scalar registers:
    // tile = ((batch * tokens) + token) * blocks_per_token + block.
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t tile = blockIdx.x * kWaves + wave;
    if (tile >= a.ntiles)
        return;   // wave-uniform
    const uint32_t bt = fast_div(tile, a.div_bpt);
    const int32_t blk = (int32_t)(tile - bt * a.div_bpt.d);
    const uint32_t bq = fast_div(bt, a.div_tokens);
    const int32_t tok = (int32_t)(bt - bq * a.div_tokens.d);
    const int32_t b = (int32_t)bq;
    const bool s1 = tok >= a.tokens0;              // token of stream 1 (image)
    const int32_t ltok = s1 ? tok - a.tokens0 : tok;

    // Named per-tensor values, not arrays: a per-lane choice among them must
    // stay a select, never an indexed memory access.
    const TensorRows R0 = tensor_rows(a.t[0], s1, b, tok, ltok);
    const TensorRows R1 = tensor_rows(a.t[1], s1, b, tok, ltok);
    const TensorRows R2 = tensor_rows(a.t[2], s1, b, tok, ltok);
    const int h0 = a.t[0].heads, h01 = a.t[0].heads + a.t[1].heads;

    // Lanes past RPP * LPR (64 is not a multiple of a non-power-of-two LPR)
    // own nothing.
    const bool lane_ok = lane < RPP * LPR;
    const int g = lane_ok ? lane / LPR : 0;
    const int j = lane_ok ? lane % LPR : LPR;
    const int nv = a.head_dim / VE;

    // The two vectors this lane owns in every row.
    int v0, v1;
    bool rot_lane = false;
    if (PAIRING == kNeox && ROT) {
        const int nr = a.rotary_dim / (2 * VE);   // vector pairs that rotate
        if (j < nr) {
            v0 = j;
            v1 = j + nr;
            rot_lane = true;
        } else {                                  // pass-through vectors past R
            v0 = 2 * nr + 2 * (j - nr);
            v1 = v0 + 1;
        }
    } else {
        const int hv = (nv + 1) >> 1;
        v0 = j < hv ? j : nv;
        v1 = j < hv ? j + hv : nv;
    }
    if (!lane_ok) {
        v0 = v1 = nv;
        rot_lane = false;
    }
    const bool own0 = v0 < nv, own1 = v1 < nv;
    const int64_t off0 = (int64_t)(own0 ? v0 : 0) * 16, off1 = (int64_t)(own1 ? v1 : 0) * 16;

    // Row r of the token (clamped to a real row for the load) -> tensor, head.
    auto locate = [&](int r, int& ti, int& h) {
        ti = r < h0 ? 0 : (r < h01 ? 1 : 2);
        h = r - (ti == 0 ? 0 : (ti == 1 ? h0 : h01));
    };

    const bool tile_norms = blk * RPW < a.rope_rows;   // wave-uniform
    const RopeArgs& rp = a.rope;
    const int half = rp.half;
    const int64_t tabs = rp.token_base + tok;          // token inside the position planes

    // 1a) Rotation operands: positions (scalar), then the lane's pair operands.
    TokenPositions pos{0, 0, 0, 0};
    PairOperand op0{}, op1{};
    if constexpr (ROT) {
        if constexpr (ROPE == 1) {
            const int nplanes = rp.mode == kPosImrope ? 4 : (rp.mode == kPos1D ? 1 : 3);
            pos.t = rp.positions[tabs];
            if (nplanes > 1) {
                pos.h = rp.positions[rp.pos_stride + tabs];
                pos.w = rp.positions[2 * rp.pos_stride + tabs];
            }
            if (nplanes > 3)
                pos.e = rp.positions[3 * rp.pos_stride + tabs];
        }
        if constexpr (ROPE == 3)
            pos = vit_token_positions(a.vit, (uint32_t)tabs);
        op0 = fetch_pair<ROPE>(rp, a.vit, tabs, lane < half ? lane : half - 1);
        op1 = fetch_pair<ROPE>(rp, a.vit, tabs, lane + 64 < half ? lane + 64 : half - 1);
    }

    // 1b) Weights of Q and K for this stream (tiny, cached).  A tensor without
    //     heads has no weight; the other one's stands in (never used).
    const char* wq = s1 ? a.t[0].weight[1] : a.t[0].weight[0];
    const char* wk = s1 ? a.t[1].weight[1] : a.t[1].weight[0];
    wq = wq != nullptr ? wq : wk;
    wk = wk != nullptr ? wk : wq;
    uint4 wq0 = make_uint4(0, 0, 0, 0), wq1 = wq0, wk0 = wq0, wk1 = wq0;
    if (wq != nullptr) {   // wave-uniform; null only for a copy-only call
        wq0 = load16(wq + off0);
        wq1 = load16(wq + off1);
        wk0 = load16(wk + off0);
        wk1 = load16(wk + off1);
    }

    // 1c) Every row load of the tile.
    uint4 d[NP][2];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        int r = blk * RPW + p * RPP + g;
        r = r < a.rows_per_token ? r : a.rows_per_token - 1;
        int ti, h;
        locate(r, ti, h);
        const char* base = ti == 0 ? R0.in : (ti == 1 ? R1.in : R2.in);
        const int64_t sh = ti == 0 ? R0.in_sh : (ti == 1 ? R1.in_sh : R2.in_sh);
        const char* row = base + (int64_t)h * sh;
        d[p][0] = load_row16<NT>(row + off0);
        d[p][1] = load_row16<NT>(row + off1);
    }

    // 2) cos/sin of the lane's VE pairs, computed once per token while the
    //    rows are in flight.
    float cs_c[VE], cs_s[VE];
#pragma unroll
    for (int e = 0; e < VE; ++e) {
        cs_c[e] = 1.0f;
        cs_s[e] = 0.0f;
    }
    if constexpr (ROT) {
        if (tile_norms) {
            const bool wide = half > 64;   // wave-uniform
            float c0, s0, c1 = 1.0f, s1v = 0.0f;
            pair_cos_sin<ROPE>(op0, pos, c0, s0);
            if (wide)
                pair_cos_sin<ROPE>(op1, pos, c1, s1v);
#pragma unroll
            for (int e = 0; e < VE; ++e) {
                int p;
                if constexpr (PAIRING == kNeox)
                    p = j * VE + e;
                else
                    p = (e < VE / 2 ? v0 : v1) * (VE / 2) + (e % (VE / 2));
                p = p < half ? p : half - 1;
                const int src = p & 63;
                float c = bperm(src, c0), sn = bperm(src, s0);
                if (wide) {
                    const float c_hi = bperm(src, c1), s_hi = bperm(src, s1v);
                    c = p >= 64 ? c_hi : c;
                    sn = p >= 64 ? s_hi : sn;
                }
                cs_c[e] = c;
                cs_s[e] = sn;
            }
        }
    }

    // 3) Row sums of squares; every lane takes part in every DPP step.
    float ssq[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        // A slot the lane does not own holds a re-read of another vector
        // (the loads are unconditional): it must not count.
        const float s0 = E::sumsq(d[p][0], 0.0f);
        const float part = (own0 ? s0 : 0.0f) + (own1 ? E::sumsq(d[p][1], 0.0f) : 0.0f);
        ssq[p] = group_sum<LPR>(part);
    }

    // 4) Per row: normalise, round, rotate, store.
    const float eps = a.eps, inv_d = a.inv_d;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const int r = blk * RPW + p * RPP + g;
        if (r >= a.rows_per_token)
            continue;
        int ti, h;
        locate(r, ti, h);
        char* obase = ti == 0 ? R0.out : (ti == 1 ? R1.out : R2.out);
        const int64_t osh = ti == 0 ? R0.out_sh : (ti == 1 ? R1.out_sh : R2.out_sh);
        char* orow = obase + (int64_t)h * osh;
        if (r >= a.rope_rows) {   // routed tensor (V): bit copy
            if (own0) store_row16<NT>(orow + off0, d[p][0]);
            if (own1) store_row16<NT>(orow + off1, d[p][1]);
            continue;
        }
        float x0[VE], x1[VE];
        E::unpack(d[p][0], x0);
        E::unpack(d[p][1], x1);
        const float rrms = rsqrtf(ssq[p] * inv_d + eps);
        float w0[VE], w1[VE];
        E::unpack(ti == 0 ? wq0 : wk0, w0);
        E::unpack(ti == 0 ? wq1 : wk1, w1);
#pragma unroll
        for (int e = 0; e < VE; ++e) {
            x0[e] = x0[e] * rrms * w0[e];
            x1[e] = x1[e] * rrms * w1[e];
        }
        E::round_trip(x0);
        E::round_trip(x1);
        if constexpr (ROT) {
            if constexpr (PAIRING == kNeox) {
                if (rot_lane) {
#pragma unroll
                    for (int e = 0; e < VE; ++e) {
                        const float xa = x0[e], xb = x1[e];
                        x0[e] = xa * cs_c[e] - xb * cs_s[e];
                        x1[e] = xb * cs_c[e] + xa * cs_s[e];
                    }
                }
            } else {
#pragma unroll
                for (int k = 0; k < VE / 2; ++k) {
                    if (v0 * (VE / 2) + k < half) {
                        const float xa = x0[2 * k], xb = x0[2 * k + 1];
                        x0[2 * k] = xa * cs_c[k] - xb * cs_s[k];
                        x0[2 * k + 1] = xb * cs_c[k] + xa * cs_s[k];
                    }
                    if (v1 * (VE / 2) + k < half) {
                        const float xa = x1[2 * k], xb = x1[2 * k + 1];
                        x1[2 * k] = xa * cs_c[VE / 2 + k] - xb * cs_s[VE / 2 + k];
                        x1[2 * k + 1] = xb * cs_c[VE / 2 + k] + xa * cs_s[VE / 2 + k];
                    }
                }
            }
        }
        if (own0) store_row16<NT>(orow + off0, E::pack(x0));
        if (own1) store_row16<NT>(orow + off1, E::pack(x1));
    }
}

// ---------------------------------------------------------------------------
// Plain row RMSNorm.
//   KIND 0 rows : one wavefront per row, 4 rows per workgroup.
//   KIND 1 split: `splits` wavefronts per row, each on its own workgroup (so
//                 on different compute units); each reads the whole row for
//                 the sum of squares (the repeats come from L2) and writes
//                 only its slice: one launch, no atomics, no cross-workgroup
//                 hand-off.  For the few-row decode case ([Vulkan]: one row
//                 on one workgroup leaves the GPU idle).
//   KIND 2 wide : one workgroup of 4 wavefronts per row, one LDS exchange.
// Every lane holds VPL 16-byte vectors of the row, all loaded up front
// ([VecRMS]: 16-byte vectorized reads of the row).
// ---------------------------------------------------------------------------
template <class E, int VPL, int KIND, bool NT>
__global__ __launch_bounds__(kThreads) void rms_kernel(const RmsArgs a)
{
    constexpr int VE = E::VE;
    const int lane = threadIdx.x & 63;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int64_t row;
    int split = 0;
    int first, step;   // vector index of the lane's slot 0, distance between slots
    if constexpr (KIND == 0) {
        row = blockIdx.x * kWaves + wave;
        first = lane;
        step = 64;
    } else if constexpr (KIND == 1) {
        const uint32_t item = blockIdx.x * kWaves + wave;
        const uint32_t r = fast_div(item, a.div_splits);
        row = r;
        split = (int)(item - r * a.div_splits.d);
        first = lane;
        step = 64;
    } else {
        row = blockIdx.x;
        first = threadIdx.x;
        step = kThreads;
    }
    if (row >= a.rows)
        return;   // wave-uniform (workgroup-uniform for KIND 2)

    const char* x = a.x + row * a.x_stride;
    uint4 d[VPL];
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        const int v = first + k * step;
        d[k] = v < a.nvec ? load_row16<NT>(x + (int64_t)v * 16) : make_uint4(0, 0, 0, 0);
    }
    float ss = 0.0f;
#pragma unroll
    for (int k = 0; k < VPL; ++k)
        ss = E::sumsq(d[k], ss);
    ss = wave_sum(ss);
    if constexpr (KIND == 2) {
        __shared__ float part[kWaves];
        if (lane == 0)
            part[wave] = ss;
        __syncthreads();
        ss = part[0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w)
            ss += part[w];
    }
    const float rrms = rsqrtf(ss * a.inv_width + a.eps);

    int lo = 0, hi = a.nvec;
    if constexpr (KIND == 1) {
        lo = split * a.split_len;
        hi = min(a.nvec, lo + a.split_len);
    }
    char* y = a.y + row * a.y_stride;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        const int v = first + k * step;
        if (v >= lo && v < hi) {
            float xv[VE], wv[VE];
            E::unpack(d[k], xv);
            E::unpack(load16(a.w + (int64_t)v * 16), wv);
#pragma unroll
            for (int e = 0; e < VE; ++e)
                xv[e] = xv[e] * rrms * wv[e];
            store_row16<NT>(y + (int64_t)v * 16, E::pack(xv));
        }
    }
}

// ---------------------------------------------------------------------------
// ViT cos/sin planes ([ViT] setup kernel): one thread per (token, column).
// Column c belongs to axis a (t, h, w contiguous); plane a receives
// cos/sin(fl32(pos_a) * inv_a[c - off_a]) at [a][token][c].
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void vit_setup_kernel(const VitArgs a)
{
    const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (idx >= a.tok_count * a.half_rot)
        return;
    const int64_t tok = a.tok_begin + idx / a.half_rot;
    const int32_t col = (int32_t)(idx % a.half_rot);
    int32_t pos[3];
    vit_position(a.cu, a.hw, a.num_grids, a.merge, tok, &pos[0], &pos[1], &pos[2]);
    const int axis = col < a.off[1] ? 0 : (col < a.off[2] ? 1 : 2);
    const float* inv = axis == 0 ? a.inv[0] : (axis == 1 ? a.inv[1] : a.inv[2]);
    const int32_t off = axis == 0 ? a.off[0] : (axis == 1 ? a.off[1] : a.off[2]);
    const int32_t p = axis == 0 ? pos[0] : (axis == 1 ? pos[1] : pos[2]);
    const float theta = (float)p * inv[col - off];
    float s, c;
    sincosf(theta, &s, &c);
    const int64_t o = ((int64_t)axis * a.n_tokens + tok) * a.half_rot + col;
    a.cos_out[o] = c;
    a.sin_out[o] = s;
}

__global__ void debug_axis_kernel(int32_t mode, int32_t s0, int32_t s1, int32_t s2, int32_t s3,
                                  int32_t n_pairs, int32_t* out)
{
    const int p = blockIdx.x * blockDim.x + threadIdx.x;
    if (p >= n_pairs)
        return;
    const int32_t sec[4] = {s0, s1, s2, s3};
    out[p] = pair_axis(mode, sec, p);
}

__global__ __launch_bounds__(kThreads) void debug_vit_kernel(const VitArgs a, int32_t* out)
{
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= a.tok_count)
        return;
    const int64_t tok = a.tok_begin + i;
    int32_t t, h, w;
    vit_position(a.cu, a.hw, a.num_grids, a.merge, tok, &t, &h, &w);
    out[tok] = t;
    out[a.n_tokens + tok] = h;
    out[2 * a.n_tokens + tok] = w;
}

// ---------------------------------------------------------------------------
// Dispatch tables
// ---------------------------------------------------------------------------
using NormRopeFn = void (*)(NormRopeArgs);

template <class E, int LPR, int ROPE, int PAIRING, bool NT>
NormRopeFn pick_np(int np)
{
    switch (np) {
    case 1: return norm_rope_kernel<E, LPR, 1, ROPE, PAIRING, NT>;
    case 2: return norm_rope_kernel<E, LPR, 2, ROPE, PAIRING, NT>;
    case 3: return norm_rope_kernel<E, LPR, 3, ROPE, PAIRING, NT>;
    default: return norm_rope_kernel<E, LPR, 4, ROPE, PAIRING, NT>;
    }
}

template <class E, int LPR, int ROPE, int PAIRING>
NormRopeFn pick_nt(bool nt, int np)
{
    return nt ? pick_np<E, LPR, ROPE, PAIRING, true>(np) : pick_np<E, LPR, ROPE, PAIRING, false>(np);
}

template <class E, int LPR, int ROPE>
NormRopeFn pick_pairing(int pairing, bool nt, int np)
{
    return pairing == kNeox ? pick_nt<E, LPR, ROPE, kNeox>(nt, np) : pick_nt<E, LPR, ROPE, kAdjacent>(nt, np);
}

template <class E, int LPR>
NormRopeFn pick_rope(int rope, int pairing, bool nt, int np)
{
    switch (rope) {
    case 0: return pick_pairing<E, LPR, 0>(pairing, nt, np);
    case 1: return pick_pairing<E, LPR, 1>(pairing, nt, np);
    case 2: return pick_pairing<E, LPR, 2>(pairing, nt, np);
    default: return pick_pairing<E, LPR, 3>(pairing, nt, np);
    }
}

template <class E>
NormRopeFn pick_lpr(int lpr, int rope, int pairing, bool nt, int np)
{
    switch (lpr) {
    case 1: return pick_rope<E, 1>(rope, pairing, nt, np);
    case 2: return pick_rope<E, 2>(rope, pairing, nt, np);
    case 4: return pick_rope<E, 4>(rope, pairing, nt, np);
    case 5: return pick_rope<E, 5>(rope, pairing, nt, np);
    case 8: return pick_rope<E, 8>(rope, pairing, nt, np);
    case 16: return pick_rope<E, 16>(rope, pairing, nt, np);
    default: return pick_rope<E, 32>(rope, pairing, nt, np);
    }
}

using RmsFn = void (*)(RmsArgs);

template <class E, int KIND, bool NT>
RmsFn pick_vpl(int vpl)
{
    switch (vpl) {
    case 1: return rms_kernel<E, 1, KIND, NT>;
    case 2: return rms_kernel<E, 2, KIND, NT>;
    case 3: return rms_kernel<E, 3, KIND, NT>;
    case 4: return rms_kernel<E, 4, KIND, NT>;
    case 5: return rms_kernel<E, 5, KIND, NT>;
    case 6: return rms_kernel<E, 6, KIND, NT>;
    case 8: return rms_kernel<E, 8, KIND, NT>;
    case 10: return rms_kernel<E, 10, KIND, NT>;
    case 12: return rms_kernel<E, 12, KIND, NT>;
    default: return rms_kernel<E, 16, KIND, NT>;
    }
}

template <class E, int KIND>
RmsFn pick_rms_nt(bool nt, int vpl)
{
    return nt ? pick_vpl<E, KIND, true>(vpl) : pick_vpl<E, KIND, false>(vpl);
}

int round_vpl(int need)
{
    static const int sizes[] = {1, 2, 3, 4, 5, 6, 8, 10, 12, 16};
    for (int s : sizes)
        if (need <= s)
            return s;
    return -1;
}

thread_local char g_variant[96];

}  // namespace

hipError_t launch_norm_rope(const NormRopeArgs& a_in, int32_t dtype, int32_t pairing, int np, int nt,
                            hipStream_t stream, const char** variant)
{
    NormRopeArgs a = a_in;
    const int ve = dtype == kBF16 ? 8 : 4;
    const int nv = a.head_dim / ve;
    // Lanes per row: enough for two vectors per lane; a power of two, or 5
    // (rows of 5 vector pairs, e.g. head_dim 80 bf16: 12 rows per pass in 60
    // lanes instead of 8 rows in 64 lanes of which 24 idle).
    int lpr = 1;
    while (2 * lpr < nv)
        lpr *= 2;
    if ((nv + 1) / 2 == 5)
        lpr = 5;
    const int rpp = 64 / lpr;
    if (np <= 0) {
        // A token of up to three passes goes to one wavefront (its cos/sin
        // computed once); longer tokens are cut into two-pass tiles, which
        // keeps registers low enough for 5-7 waves per SIMD.  Measured on
        // MI355X: 24 rows/token (16 Q + 8 K) fastest at 3 passes, 72 rows
        // (joint Q, K, V of 24 heads) and 32 rows (16 + 16) at 2 passes.
        const int passes = (a.rows_per_token + rpp - 1) / rpp;
        np = passes <= 3 ? (passes < 1 ? 1 : passes) : 2;
    }
    const int rope = a.rope.mode == kPosNone ? 0
                     : (a.rope.mode == kPosPlanes ? 2 : (a.rope.mode == kPosVit ? 3 : 1));
    const int rpw = rpp * np;
    const uint32_t bpt = (uint32_t)((a.rows_per_token + rpw - 1) / rpw);
    const int64_t tiles = (int64_t)a.batch * a.tokens * bpt;
    if (tiles == 0)
        return hipSuccess;
    if (tiles >= ((int64_t)1 << 31))
        return hipErrorInvalidValue;   // the host layer refuses such calls first
    a.ntiles = (uint32_t)tiles;
    a.div_bpt = make_fastdiv(bpt);
    a.div_tokens = make_fastdiv((uint32_t)a.tokens);
    const int64_t blocks = (tiles + kWaves - 1) / kWaves;
    const bool use_nt = nt != 0;
    NormRopeFn fn = dtype == kBF16 ? pick_lpr<BF16>(lpr, rope, pairing, use_nt, np)
                                   : pick_lpr<F32>(lpr, rope, pairing, use_nt, np);
    hipLaunchKernelGGL(fn, dim3((uint32_t)blocks), dim3(kThreads), 0, stream, a);
    snprintf(g_variant, sizeof(g_variant), "rope:np%d:nt%d:lpr%d:%s:%s:%s", np, (int)use_nt, lpr,
             dtype == kBF16 ? "bf16" : "f32",
             rope == 0 ? "none" : (rope == 1 ? "pos" : (rope == 2 ? "planes" : "vit")),
             pairing == kNeox ? "neox" : "adjacent");
    *variant = g_variant;
    return hipGetLastError();
}

hipError_t launch_rms_norm(RmsArgs a, int32_t dtype, int kind, int nt, hipStream_t stream, const char** variant)
{
    if (a.rows == 0)
        return hipSuccess;
    if (kind < 0) {
        // Few rows: spread each row over several compute units.
        kind = a.rows < 256 ? 1 : 0;
    }
    int vpl = round_vpl(kind == 2 ? (a.nvec + kThreads - 1) / kThreads : (a.nvec + 63) / 64);
    if (vpl < 0 && kind != 2) {
        kind = 2;
        vpl = round_vpl((a.nvec + kThreads - 1) / kThreads);
    }
    if (vpl < 0)
        return hipErrorInvalidValue;
    int64_t blocks;
    if (kind == 0) {
        blocks = (a.rows + kWaves - 1) / kWaves;
    } else if (kind == 1) {
        // one slice of 64 vectors per wave (each lane stores one vector)
        a.split_len = 64;
        a.splits = (a.nvec + a.split_len - 1) / a.split_len;
        a.div_splits = make_fastdiv((uint32_t)a.splits);
        blocks = (a.rows * a.splits + kWaves - 1) / kWaves;
    } else {
        blocks = a.rows;
    }
    const bool use_nt = nt != 0;
    RmsFn fn;
    if (dtype == kBF16)
        fn = kind == 0 ? pick_rms_nt<BF16, 0>(use_nt, vpl)
                       : (kind == 1 ? pick_rms_nt<BF16, 1>(use_nt, vpl) : pick_rms_nt<BF16, 2>(use_nt, vpl));
    else
        fn = kind == 0 ? pick_rms_nt<F32, 0>(use_nt, vpl)
                       : (kind == 1 ? pick_rms_nt<F32, 1>(use_nt, vpl) : pick_rms_nt<F32, 2>(use_nt, vpl));
    hipLaunchKernelGGL(fn, dim3((uint32_t)blocks), dim3(kThreads), 0, stream, a);
    snprintf(g_variant, sizeof(g_variant), "rms:%s:nt%d:vpl%d:%s",
             kind == 0 ? "rows" : (kind == 1 ? "split" : "wide"), (int)use_nt, vpl, dtype == kBF16 ? "bf16" : "f32");
    *variant = g_variant;
    return hipGetLastError();
}

hipError_t launch_vit_setup(const VitArgs& a, hipStream_t stream)
{
    const int64_t n = a.tok_count * a.half_rot;
    if (n == 0)
        return hipSuccess;
    hipLaunchKernelGGL(vit_setup_kernel, dim3((uint32_t)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                       stream, a);
    return hipGetLastError();
}

hipError_t launch_debug_axis_map(int32_t mode, const int32_t* sec, int32_t n_pairs, int32_t* out,
                                 hipStream_t stream)
{
    if (n_pairs == 0)
        return hipSuccess;
    hipLaunchKernelGGL(debug_axis_kernel, dim3((n_pairs + 63) / 64), dim3(64), 0, stream, mode, sec[0], sec[1],
                       sec[2], sec[3], n_pairs, out);
    return hipGetLastError();
}

hipError_t launch_debug_vit_positions(const VitArgs& a, int32_t* out, hipStream_t stream)
{
    if (a.tok_count == 0)
        return hipSuccess;
    hipLaunchKernelGGL(debug_vit_kernel, dim3((uint32_t)((a.tok_count + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, stream, a, out);
    return hipGetLastError();
}

}  // namespace qkr
