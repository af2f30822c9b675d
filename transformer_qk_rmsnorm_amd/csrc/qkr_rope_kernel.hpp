// Per-head QK RMSNorm + RoPE kernel template and its dispatch tables.  One
// translation unit per lanes-per-row value instantiates it (qkr_rope_part.hip).
//
// Page names used in comments:
//   [Ovis]   vllm-omni pull request "[Kernel][Ovis-Image] Fuse text/image QK
//            RMSNorm + cat + RoPE into one Triton launch"
//   [IMROPE] llama.cpp fork pull request "hrx: the multi-section rotation of
//            Qwen3-VL runs on the device, not on the CPU"
//   [ViT]    vLLM API page "vllm.model_executor.layers.rotary_embedding.
//            mrope_vit_setup"
#pragma once

#include "qkr_device.hpp"

namespace qkr {
namespace {

// The token's position on each plane (wave-uniform).
struct TokenPositions {
    int32_t t, h, w, e;
};

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

// Angle of one pair: the fp32 product of the fp32 position on the pair's
// axis and the pair's inverse frequency ([ViT] setup kernel).  sincosf is the
// accurate device-library routine (its argument reduction holds far past the
// 8191 rad these workloads reach).
__device__ __forceinline__ void pair_cos_sin(int32_t axis, const TokenPositions& pos, float inv, float& c, float& s)
{
    const int32_t q = axis == 0 ? pos.t : (axis == 1 ? pos.h : (axis == 2 ? pos.w : pos.e));
    sincosf((float)q * inv, &s, &c);
}

// One of three wave-uniform values, by selects (an indexed access into the
// kernel-argument table would make the compiler copy it to private memory).
template <class T>
__device__ __forceinline__ T sel3(int i, T v0, T v1, T v2)
{
    return i == 0 ? v0 : (i == 1 ? v1 : v2);
}

// ---------------------------------------------------------------------------
// Per-(token, head) RMSNorm + RoPE.
//
// Work unit (tile): one wavefront takes NP passes over RPP = 64 / LPR heads of
// ONE tensor (Q, K or V) of one token, so every base address, stride and
// weight vector of the tile is wave-uniform.  LPR lanes share a row and every
// lane owns two 16-byte vectors of it: with the NeoX pairing vectors j and
// j + R/(2 VE), so every rotated pair (p, p + R/2) is lane-local; otherwise
// vectors j and j + ceil(nv/2), and adjacent pairs sit inside one vector.
//
// Order of work in a wave:
//   0. the tile decode and the tensor descriptor: kernel-argument reads with
//      no branch between them (padding waves past the tile count run the
//      last tile with every store off instead of leaving early), so they
//      arrive in few batches;
//   1. vector loads, which complete in order: the lane's pair operands
//      (inverse frequency, planes entry or ladder value), then every row of
//      the tile, then the tensor's weight vectors.  All are unconditional
//      (rows past the tensor re-read its last head, a cache hit, never
//      stored), so the compiler counts them and each wait below covers only
//      what it needs.  The token's positions follow as scalar loads;
//   2. cos/sin of the token's pairs (lane i: pair i, axis from a host-built
//      table) while the rows are in flight, handed to the lanes that need
//      them with ds_bpermute; the weights unpacked once;
//   3. per pass: DPP sum of squares over the row's LPR lanes, normalise,
//      round per the contract, rotate, store.
// A routed tensor (V) tile only loads its rows and stores them.
//
// STAGE: where half a row is not a whole number of 128-byte lines (e.g.
// head_dim 80 bf16: 80-byte halves), a store instruction of the lane-local
// layout would cover every line it touches only in part, and partial-line
// writes cost HBM efficiency.  The pass's results then go through a per-wave
// LDS slice indexed by (row, vector) and leave as vectors lane and 64 + lane
// of the pass, i.e. contiguous 1 KB runs when a token's heads are adjacent.
//
// ROPE: 0 norm only, 1 positions + inv_freq (1D / AXES / IMROPE: the axis
// table carries the difference), 2 cos/sin planes, 3 ViT positions computed
// from the grid table.
// ---------------------------------------------------------------------------
template <class E, int LPR, int NP, int ROPE, int PAIRING, bool NT, bool STAGE>
__global__ __launch_bounds__(kThreads) void norm_rope_kernel(const NormRopeArgs a)
{
    constexpr int VE = E::VE;
    constexpr int RPP = 64 / LPR;
    constexpr bool ROT = ROPE != 0;
    static_assert((LPR & (LPR - 1)) == 0 && LPR <= 32, "lanes per row: a power of two up to 32");

    const int lane = threadIdx.x & 63;
    // Tile coordinates are wave-uniform and stay in scalar registers:
    // tile = (batch * tokens + token) * tiles_per_token + k, where tiles
    // [tile_first[i], tile_first[i + 1]) of a token belong to tensor i.
    // Padding waves of the last workgroup (index >= ntiles) redo the loads
    // of the last tile and store nothing: with no early exit, no branch
    // splits the kernel-argument reads of the prologue into separate waits.
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t tile_raw = blockIdx.x * kWaves + wave;
    const bool pad = tile_raw >= a.ntiles;         // wave-uniform
    const uint32_t tile = pad ? a.ntiles - 1 : tile_raw;
    const uint32_t bt = fast_div(tile, a.div_tpt);
    const int32_t k = (int32_t)(tile - bt * a.div_tpt.d);
    const int ti = k >= a.tile_first[2] ? 2 : (k >= a.tile_first[1] ? 1 : 0);
    const int32_t blk = k - sel3(ti, 0, a.tile_first[1], a.tile_first[2]);
    const uint32_t bq = fast_div(bt, a.div_tokens);
    const int32_t tok = (int32_t)(bt - bq * a.div_tokens.d);
    const int32_t b = (int32_t)bq;
    const bool s1 = tok >= a.tokens0;              // token of stream 1 (image)
    const int32_t ltok = s1 ? tok - a.tokens0 : tok;

    const TensorArgs& T = a.t[ti];
    const int si = s1 ? 1 : 0;
    const char* const in = T.in[si];
    const int64_t in_sb = T.in_sb[si], in_st = T.in_st[si], in_sh = T.in_sh[si];
    const char* const wt = T.weight[si];
    char* const out = T.out;
    const int64_t out_sb = T.out_sb, out_st = T.out_st, out_sh = T.out_sh;
    const int32_t heads = T.heads;
    const int64_t* const slots = T.slots;
    const int64_t nslots = T.nslots;

    // Heads [h0, h0 + hrem) of the tensor are left from this tile on.
    const int32_t h0 = blk * RPP * NP;
    const int32_t hrem = heads - h0;
    const char* const in_t = in + (int64_t)b * in_sb + (int64_t)ltok * in_st + (int64_t)h0 * in_sh;

    // The two vectors this lane owns in every row.
    const int g = lane / LPR, j = lane % LPR;
    const int nv = a.head_dim / VE;
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
    const bool own0 = v0 < nv, own1 = v1 < nv;
    const int32_t off0 = (own0 ? v0 : 0) * 16, off1 = (own1 ? v1 : 0) * 16;

    // Loads of pass p: head p * RPP + g of the tile, clamped into the tensor.
    const int64_t lane_in0 = (int64_t)g * in_sh + off0;
    auto load_pass = [&](int p, uint4& x0, uint4& x1) {
        const int lim = hrem - 1 - p * RPP;    // last valid g of the pass (may be < 0)
        const char* base = in_t + (int64_t)(p * RPP) * in_sh;
        const int64_t o0 = (p + 1) * RPP <= hrem ? lane_in0 : (int64_t)(g < lim ? g : lim) * in_sh + off0;
        x0 = load_row16<NT>(base + o0);
        x1 = load_row16<NT>(base + o0 + (off1 - off0));
    };

    // The output row of the token: the token itself, or the cache row its
    // slot picks ([IMROPE]: the rotation's set_rows twin).  A slot outside
    // the cache writes nothing, so the tile ends there (wave-uniform).  The
    // slot is read once the tile's row loads are issued; those are in range
    // and are simply dropped.
    auto out_base = [&](char*& out_t) {
        int64_t orow = tok;
        if (slots != nullptr) {
            orow = slots[tok];
            if (orow < 0 || orow >= nslots)
                return false;
        }
        out_t = out + (int64_t)b * out_sb + orow * out_st + (int64_t)h0 * out_sh;
        return true;
    };

    // Stores of pass p (heads past the tensor are skipped).  Every per-lane
    // address is formed once from the tile's output base; a pass adds the
    // uniform offset of its heads.
    __shared__ uint4 stage_all[STAGE ? kWaves * 128 : 1];
    uint4* const stage = stage_all + (STAGE ? wave * 128 : 0);   // RPP * nv <= 2 * 64 vectors
    struct Dst {
        char* lane_out;      // direct: this lane's row of pass 0
        int slot_row[2];     // staged: row of each vector slot of a pass (1 << 30: none)
        char* slot_out[2];
    };
    auto dst_of = [&](char* out_t) {
        Dst t;
        t.lane_out = out_t + (int64_t)g * out_sh;
        if constexpr (STAGE) {
#pragma unroll
            for (int sl = 0; sl < 2; ++sl) {
                const int f = sl * 64 + lane;                               // vector of the pass
                const int fr = (int)(((uint32_t)f * a.nv_recip) >> 16);     // its row in the pass
                const int fv = f - fr * nv;
                t.slot_row[sl] = fr < RPP ? fr : (1 << 30);
                t.slot_out[sl] = out_t + (int64_t)fr * out_sh + (int64_t)fv * 16;
            }
        }
        return t;
    };
    auto store_pass = [&](const Dst& t, int p, const uint4& o0, const uint4& o1) {
        const int64_t pass_off = (int64_t)(p * RPP) * out_sh;           // wave-uniform
        const int live = pad ? 0 : hrem - p * RPP;                       // rows of the pass to store
        if constexpr (STAGE) {
            if (g < live) {
                if (own0) stage[g * nv + v0] = o0;
                if (own1) stage[g * nv + v1] = o1;
            }
            wave_lds_order();
#pragma unroll
            for (int sl = 0; sl < 2; ++sl)
                if (t.slot_row[sl] < live)
                    store_row16<NT>(t.slot_out[sl] + pass_off, stage[sl * 64 + lane]);
            wave_lds_order();
        } else {
            if (g < live) {
                char* const dst = t.lane_out + pass_off;
                if (own0) store_row16<NT>(dst + off0, o0);
                if (own1) store_row16<NT>(dst + off1, o1);
            }
        }
    };

    // The rotation's scalar parameters are read before the V branch, in the
    // descriptor's batch of kernel-argument loads.
    const RopeArgs& rp = a.rope;
    const int half = (int)uniform((uint32_t)rp.half);
    const int64_t tabs = rp.token_base + tok;      // token inside the position planes
    const float* const inv_freq = uniform(rp.inv_freq);
    const int p0 = lane < half ? lane : half - 1;
    const int p1 = lane + 64 < half ? lane + 64 : half - 1;

    uint4 d[NP][2];
    if (wt == nullptr) {   // wave-uniform: a routed tensor (V), bit copy
#pragma unroll
        for (int p = 0; p < NP; ++p)
            load_pass(p, d[p][0], d[p][1]);
        char* out_t;
        if (!out_base(out_t))
            return;
        const Dst t = dst_of(out_t);
#pragma unroll
        for (int p = 0; p < NP; ++p)
            if (p * RPP < hrem)   // wave-uniform: a pass past the tensor has nothing to store
                store_pass(t, p, d[p][0], d[p][1]);
        return;
    }

    // 1) Loads of a normed tile, in this order: the lane's pair operands
    //    (inverse frequency, planes entries or ladder values; tiny, cached,
    //    and first in the in-order vector queue, so the trig waits for them
    //    alone), every row, the tensor's weight vectors (the first pass
    //    waits for every row either way).  The token's positions are scalar
    //    loads, counted apart from the vector loads, read after the rows.
    TokenPositions pos{0, 0, 0, 0};
    int32_t ax0 = 0, ax1 = 0;
    float op0 = 0.0f, op1 = 0.0f, os0 = 0.0f, os1 = 0.0f;   // inv_freq or cos, and sin
    if constexpr (ROPE == 1) {
        op0 = load_global(inv_freq + p0);
        op1 = load_global(inv_freq + p1);
    }
    if constexpr (ROPE == 2) {
        ax0 = axis_of(rp.axis_bits, p0);
        ax1 = axis_of(rp.axis_bits, p1);
        const int64_t i0 = ((int64_t)ax0 * rp.planes_tokens + tabs) * half + p0;
        const int64_t i1 = ((int64_t)ax1 * rp.planes_tokens + tabs) * half + p1;
        op0 = rp.cos_planes[i0];
        os0 = rp.sin_planes[i0];
        op1 = rp.cos_planes[i1];
        os1 = rp.sin_planes[i1];
    }
    if constexpr (ROPE == 3) {
        // ViT: contiguous t/h/w sections, one inverse-frequency ladder per
        // axis.  The token's (t, h, w) is found after the row loads are out.
        ax0 = axis_of(rp.axis_bits, p0);
        ax1 = axis_of(rp.axis_bits, p1);
        const int32_t o_h = rp.sec[0], o_w = rp.sec[0] + rp.sec[1];
        const float* const it = uniform(a.vit.inv[0]);
        const float* const ih = uniform(a.vit.inv[1]);
        const float* const iw = uniform(a.vit.inv[2]);
        const float* const l0 = sel3(ax0, it, ih, iw);
        const float* const l1 = sel3(ax1, it, ih, iw);
        op0 = load_global(l0 + (p0 - sel3(ax0, 0, o_h, o_w)));
        op1 = load_global(l1 + (p1 - sel3(ax1, 0, o_h, o_w)));
    }
#pragma unroll
    for (int p = 0; p < NP; ++p)
        load_pass(p, d[p][0], d[p][1]);
    const uint4 wv0 = load16(wt + off0), wv1 = load16(wt + off1);

    char* out_t;
    if (!out_base(out_t))
        return;
    const Dst dst = dst_of(out_t);
    if constexpr (ROPE == 1) {
        // Held as scalar values: a per-lane choice among four loads would
        // otherwise become one per-lane load from a chosen address, queued
        // behind the rows.
        pos.t = (int32_t)uniform((uint32_t)rp.positions[rp.plane_off[0] + tabs]);
        pos.h = (int32_t)uniform((uint32_t)rp.positions[rp.plane_off[1] + tabs]);
        pos.w = (int32_t)uniform((uint32_t)rp.positions[rp.plane_off[2] + tabs]);
        pos.e = (int32_t)uniform((uint32_t)rp.positions[rp.plane_off[3] + tabs]);
    }
    if constexpr (ROPE == 3)
        pos = vit_token_positions(a.vit, (uint32_t)tabs);   // scalar work, rows in flight

    // 2) cos/sin of the lane's VE pairs while the rows are in flight.
    float cs_c[VE], cs_s[VE];
#pragma unroll
    for (int e = 0; e < VE; ++e) {
        cs_c[e] = 1.0f;
        cs_s[e] = 0.0f;
    }
    if constexpr (ROT) {
        const bool wide = half > 64;   // wave-uniform
        float c0, s0, c1 = 1.0f, s1v = 0.0f;
        if constexpr (ROPE == 2) {
            c0 = op0;
            s0 = os0;
            c1 = op1;
            s1v = os1;
        } else {
            if constexpr (ROPE == 1)
                ax0 = axis_of(rp.axis_bits, p0);
            pair_cos_sin(ax0, pos, op0, c0, s0);
            if (wide) {
                if constexpr (ROPE == 1)
                    ax1 = axis_of(rp.axis_bits, p1);
                pair_cos_sin(ax1, pos, op1, c1, s1v);
            }
        }
        // Pair p's values sit on lane p mod 64 (ds_bpermute takes the lane
        // from address bits 7..2, so the address needs no mask).  Pairs at or
        // past `half` are never rotated: whatever such a lane receives goes
        // unused.
#pragma unroll
        for (int e = 0; e < VE; ++e) {
            int p;
            if constexpr (PAIRING == kNeox)
                p = j * VE + e;
            else
                p = (e < VE / 2 ? v0 : v1) * (VE / 2) + (e % (VE / 2));
            float c = bperm(p, c0), sn = bperm(p, s0);
            if (wide) {
                const float c_hi = bperm(p, c1), s_hi = bperm(p, s1v);
                c = p >= 64 ? c_hi : c;
                sn = p >= 64 ? s_hi : sn;
            }
            cs_c[e] = c;
            cs_s[e] = sn;
        }
    }
    float w0[VE], w1[VE];
    E::unpack(wv0, w0);
    E::unpack(wv1, w1);

    // 3) Per pass: sum of squares over the row's lanes (a slot the lane does
    //    not own holds a re-read of another vector and must not count),
    //    normalise, round, rotate, store.
    const float eps = a.eps, inv_d = a.inv_d;
    const bool eps_normal = eps >= FLT_MIN;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        // A pass wholly past the tensor (its loads re-read the last head) has
        // no row to normalise: wave-uniform skip; the load count is unchanged.
        if (p * RPP >= hrem)
            break;
        const float s0 = E::sumsq(d[p][0], 0.0f);
        const float part = (own0 ? s0 : 0.0f) + (own1 ? E::sumsq(d[p][1], 0.0f) : 0.0f);
        const float rrms = rms_rsqrt(group_sum<LPR>(part) * inv_d + eps, eps_normal);
        float x0[VE], x1[VE];
        E::unpack(d[p][0], x0);
        E::unpack(d[p][1], x1);
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
                for (int q = 0; q < VE / 2; ++q) {
                    if (v0 * (VE / 2) + q < half) {
                        const float xa = x0[2 * q], xb = x0[2 * q + 1];
                        x0[2 * q] = xa * cs_c[q] - xb * cs_s[q];
                        x0[2 * q + 1] = xb * cs_c[q] + xa * cs_s[q];
                    }
                    if (v1 * (VE / 2) + q < half) {
                        const float xa = x1[2 * q], xb = x1[2 * q + 1];
                        x1[2 * q] = xa * cs_c[VE / 2 + q] - xb * cs_s[VE / 2 + q];
                        x1[2 * q + 1] = xb * cs_c[VE / 2 + q] + xa * cs_s[VE / 2 + q];
                    }
                }
            }
        }
        store_pass(dst, p, E::pack(x0), E::pack(x1));
    }
}

template <class E, int LPR, int ROPE, int PAIRING, bool NT, bool STAGE>
NormRopeFn pick_np(int np)
{
    switch (np) {
    case 1: return norm_rope_kernel<E, LPR, 1, ROPE, PAIRING, NT, STAGE>;
    case 2: return norm_rope_kernel<E, LPR, 2, ROPE, PAIRING, NT, STAGE>;
    case 3: return norm_rope_kernel<E, LPR, 3, ROPE, PAIRING, NT, STAGE>;
    default: return norm_rope_kernel<E, LPR, 4, ROPE, PAIRING, NT, STAGE>;
    }
}

// Staged stores exist for 2..8 lanes per row (rows up to 16 vectors, the
// only ones whose halves can miss 128-byte lines).
template <class E, int LPR, int ROPE, int PAIRING>
NormRopeFn pick_nt(bool nt, bool stage, int np)
{
    constexpr bool kCanStage = LPR >= 2 && LPR <= 8;
    if (kCanStage && stage)
        return nt ? pick_np<E, LPR, ROPE, PAIRING, true, kCanStage>(np)
                  : pick_np<E, LPR, ROPE, PAIRING, false, kCanStage>(np);
    return nt ? pick_np<E, LPR, ROPE, PAIRING, true, false>(np) : pick_np<E, LPR, ROPE, PAIRING, false, false>(np);
}

template <class E, int LPR, int ROPE>
NormRopeFn pick_pairing(int pairing, bool nt, bool stage, int np)
{
    return pairing == kNeox ? pick_nt<E, LPR, ROPE, kNeox>(nt, stage, np)
                            : pick_nt<E, LPR, ROPE, kAdjacent>(nt, stage, np);
}

template <class E, int LPR>
NormRopeFn pick_rope(int rope, int pairing, bool nt, bool stage, int np)
{
    switch (rope) {
    case 0: return pick_pairing<E, LPR, 0>(pairing, nt, stage, np);
    case 1: return pick_pairing<E, LPR, 1>(pairing, nt, stage, np);
    case 2: return pick_pairing<E, LPR, 2>(pairing, nt, stage, np);
    default: return pick_pairing<E, LPR, 3>(pairing, nt, stage, np);
    }
}

}  // namespace
}  // namespace qkr
