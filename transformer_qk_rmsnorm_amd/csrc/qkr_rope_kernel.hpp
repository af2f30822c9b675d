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
// the last one whose first token has been reached (a select loop, scalar);
// then frame, merge block (raster order over the block grid) and cell, as in
// vit_position ([ViT] setup kernel's token order), with the host's divisors
// instead of hardware divides.
__device__ __forceinline__ TokenPositions vit_token_positions(const VitGridArgs& v, uint32_t tok)
{
    // Scalar fields only: selecting whole structs out of the kernel-argument
    // table would make the compiler copy the table to private memory.
    uint32_t start = (uint32_t)v.cu[0];
    uint32_t a_d = v.div_area[0].d, a_m = v.div_area[0].m, a_l = v.div_area[0].sh;
    uint32_t b_d = v.div_bcols[0].d, b_m = v.div_bcols[0].m, b_l = v.div_bcols[0].sh;
    for (int k = 1; k < v.num_grids; ++k) {
        // Grid k's fields are all read before the choice (an empty asm takes
        // them): a choice between a field and the value so far would
        // otherwise become a branch around that field's load, one wait each.
        uint32_t ck = (uint32_t)v.cu[k], ad = v.div_area[k].d, am = v.div_area[k].m, as = v.div_area[k].sh;
        uint32_t bd = v.div_bcols[k].d, bm = v.div_bcols[k].m, bs = v.div_bcols[k].sh;
        asm("" : "+s"(ck), "+s"(ad), "+s"(am), "+s"(as), "+s"(bd), "+s"(bm), "+s"(bs));
        const bool in_k = tok >= ck;
        start = in_k ? ck : start;
        a_d = in_k ? ad : a_d;
        a_m = in_k ? am : a_m;
        a_l = in_k ? as : a_l;
        b_d = in_k ? bd : b_d;
        b_m = in_k ? bm : b_m;
        b_l = in_k ? bs : b_l;
    }
    const FastDiv d_frame{a_d, a_m, a_l}, d_bcols{b_d, b_m, b_l};
    const uint32_t local = tok - start;
    const uint32_t t = fast_div(local, d_frame);
    const uint32_t in_frame = local - t * d_frame.d;
    const uint32_t block = fast_div(in_frame, v.div_mm);
    const uint32_t cell = in_frame - block * v.div_mm.d;
    const uint32_t brow = fast_div(block, d_bcols);
    const uint32_t bcol = block - brow * d_bcols.d;
    const uint32_t crow = fast_div(cell, v.div_m);
    TokenPositions p;
    p.t = (int32_t)t;
    p.h = (int32_t)(brow * v.div_m.d + crow);
    p.w = (int32_t)(bcol * v.div_m.d + (cell - crow * v.div_m.d));
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
// In the planes mode the rows also arrive that way and reach the lane-local
// layout through the same slice.  That costs registers (NeoX variants 80 ->
// 82 VGPRs, 6 -> 5 waves per SIMD): measured a gain where cos/sin come from
// memory and a loss where the wave computes them, so only the planes mode
// stages its loads.
//
// ROPE: 0 norm only, 1 positions + inv_freq (1D / AXES / IMROPE: the axis
// table carries the difference), 2 cos/sin planes, 3 ViT positions computed
// from the grid table.
//
// EAGER: the rounding points of an eager RMSNorm + RoPE chain instead of the
// contract: (act)((act)(x * rrms) * w) ([VecRMS] review thread: the RMSNorm
// kernel's output expression), cos and sin rounded to the activation type
// (the chain's RoPE table), and no fused multiply-add in the rotation.
// ---------------------------------------------------------------------------
template <class E, int LPR, int NP, int ROPE, int PAIRING, bool NT, bool STAGE, bool EAGER>
__global__ __launch_bounds__(kThreads) void norm_rope_kernel(const NormRopeArgs a)
{
    constexpr int VE = E::VE;
    constexpr int RPP = 64 / LPR;
    constexpr bool ROT = ROPE != 0;
    constexpr bool STAGE_LD = STAGE && ROPE == 2;   // staged loads as well as stores
    static_assert((LPR & (LPR - 1)) == 0 && LPR <= 32, "lanes per row: a power of two up to 32");

    const int lane = threadIdx.x & 63;
    // The rotation's scalar parameters depend on no tile coordinate: read
    // with the first batch of kernel-argument loads.
    const RopeArgs& rp = a.rope;
    const int half = (int)uniform((uint32_t)rp.half);
    const float* const inv_freq = uniform(rp.inv_freq);
    const int p0 = lane < half ? lane : half - 1;
    const int p1 = lane + 64 < half ? lane + 64 : half - 1;
    // Tile coordinates are wave-uniform and stay in scalar registers:
    // tile = (batch * tokens + token) * tiles_per_token + k, where tiles
    // [tile_first[i], tile_first[i + 1]) of a token belong to tensor i.
    // Padding waves of the last workgroup (index >= ntiles) redo the loads
    // of the last tile and store nothing: with no early exit, no branch
    // splits the kernel-argument reads of the prologue into separate waits.
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t tile_raw = a.tile_base + blockIdx.x * kWaves + wave;
    const bool pad = tile_raw >= a.ntiles;         // wave-uniform
    const uint32_t tile = pad ? a.ntiles - 1 : tile_raw;
    const uint32_t bt = fast_div(tile, a.div_tpt);
    const int32_t k = (int32_t)(tile - bt * a.div_tpt.d);
    // Tensor and stream indices from sign bits (x >= y is the sign of
    // y - 1 - x for these small non-negative values): plain scalar
    // arithmetic, where comparisons would be widened to integers through
    // vector selects, and an index the compiler cannot split into selects,
    // so a stream's fields come from one computed kernel-argument address.
    const int ti = (int)(((uint32_t)(a.tile_first[1] - 1 - k) >> 31) + ((uint32_t)(a.tile_first[2] - 1 - k) >> 31));
    const int32_t blk = k - sel3(ti, 0, a.tile_first[1], a.tile_first[2]);
    const uint32_t bq = fast_div(bt, a.div_tokens);
    const int32_t tok = (int32_t)(bt - bq * a.div_tokens.d);
    const int32_t b = (int32_t)bq;
    const int si = (int)((uint32_t)(a.tokens0 - 1 - tok) >> 31);   // 1: a token of stream 1 (image)
    const int32_t ltok = tok - si * a.tokens0;

    const TensorArgs& T = a.t[ti];
    const StreamView& S = T.s[si];
    const char* const in = S.in;
    const int64_t in_sb = S.sb, in_st = S.st, in_sh = S.sh;
    const char* const wt = S.weight;
    char* const out = T.out;
    const int64_t out_sb = T.out_sb, out_st = T.out_st, out_sh = T.out_sh;
    const int32_t heads = T.heads;
    const int64_t* const slots = T.slots;
    const int64_t nslots = T.nslots;

    // Heads [h0, h0 + hrem) of the tensor are left from this tile on.
    const int32_t h0 = blk * RPP * NP;
    const int32_t hrem = heads - h0;
    // b, ltok and h0 are non-negative: zero-extended, each product takes one
    // multiply fewer than a signed widening.
    const char* const in_t = in + (int64_t)(uint32_t)b * in_sb + (int64_t)(uint32_t)ltok * in_st +
                             (int64_t)(uint32_t)h0 * in_sh;

    // The two vectors this lane owns in every row.
    const int g = lane / LPR, j = lane % LPR;
    const int nv = (int)((uint32_t)a.head_dim / VE);
    int v0, v1;
    bool rot_lane = false;
    if (PAIRING == kNeox && ROT) {
        const int nr = (int)((uint32_t)a.rotary_dim / (2 * VE));   // vector pairs that rotate
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
    // Staged loads: the pass's vectors in (row, vector) order instead, vector
    // sl * 64 + lane in slot sl (past the pass's last vector: a re-read of
    // it), handed to the lane-local layout through LDS (unstage below).
    const int64_t lane_in0 = (int64_t)g * in_sh + off0;
    int ld_row[2] = {0, 0}, ld_col[2] = {0, 0};
    if constexpr (STAGE_LD) {
#pragma unroll
        for (int sl = 0; sl < 2; ++sl) {
            const int f = sl * 64 + lane < RPP * nv ? sl * 64 + lane : RPP * nv - 1;
            const int fr = (int)(((uint32_t)f * a.nv_recip) >> 16);
            ld_row[sl] = fr;
            ld_col[sl] = (f - fr * nv) * 16;
        }
    }
    auto load_pass = [&](int p, uint4& x0, uint4& x1) {
        const int lim = hrem - 1 - p * RPP;    // last valid row of the pass (may be < 0)
        const char* base = in_t + (int64_t)(p * RPP) * in_sh;
        if constexpr (STAGE_LD) {
            x0 = load_row16<NT>(base + (int64_t)(ld_row[0] < lim ? ld_row[0] : lim) * in_sh + ld_col[0]);
            x1 = load_row16<NT>(base + (int64_t)(ld_row[1] < lim ? ld_row[1] : lim) * in_sh + ld_col[1]);
        } else {
            const int64_t o0 = (p + 1) * RPP <= hrem ? lane_in0 : (int64_t)(g < lim ? g : lim) * in_sh + off0;
            x0 = load_row16<NT>(base + o0);
            x1 = load_row16<NT>(base + o0 + (off1 - off0));
        }
    };

    // The output row of the token: the token itself, or the cache row its
    // slot picks ([IMROPE]: the rotation's set_rows twin).  A slot outside
    // the cache writes nothing, so the tile ends there (wave-uniform).  The
    // slot is read once the tile's row loads are issued; those are in range
    // and are simply dropped.
    auto out_base = [&](char*& out_t) {
        int64_t orow = tok;
        if (slots != nullptr) {
            // A load through the constant address space is a scalar load for
            // a uniform address: V tiles would otherwise read the slot with a
            // vector load queued behind their rows.
            orow = *(const __attribute__((address_space(4))) int64_t*)(slots + tok);
            if (orow < 0 || orow >= nslots)
                return false;
        }
        out_t = out + (int64_t)(uint32_t)b * out_sb + orow * out_st + (int64_t)(uint32_t)h0 * out_sh;
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
    // Staged: the pass's flat vectors (slots as loaded) to the lane-local
    // layout: vectors v0, v1 of row g (a vector the lane does not own: the
    // row's first, which the sum of squares skips).
    auto unstage = [&](uint4& x0, uint4& x1) {
        stage[lane] = x0;
        stage[64 + lane] = x1;     // slots past the pass's vectors are never read
        wave_lds_order();
        x0 = stage[g * nv + (own0 ? v0 : 0)];
        x1 = stage[g * nv + (own1 ? v1 : 0)];
        wave_lds_order();
    };
    // Staged stores of flat vectors (a routed tile's loads as they came).
    auto store_flat = [&](const Dst& t, int p, const uint4& f0, const uint4& f1) {
        const int64_t pass_off = (int64_t)(p * RPP) * out_sh;
        const int live = pad ? 0 : hrem - p * RPP;
        if (t.slot_row[0] < live)
            store_row16<NT>(t.slot_out[0] + pass_off, f0);
        if (t.slot_row[1] < live)
            store_row16<NT>(t.slot_out[1] + pass_off, f1);
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
            store_flat(t, p, stage[lane], stage[64 + lane]);
            wave_lds_order();
        } else {
            if (g < live) {
                char* const dst = t.lane_out + pass_off;
                if (own0) store_row16<NT>(dst + off0, o0);
                if (own1) store_row16<NT>(dst + off1, o1);
            }
        }
    };

    const int64_t tabs = rp.token_base + tok;      // token inside the position planes

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
        for (int p = 0; p < NP; ++p) {
            if (p * RPP < hrem) {   // wave-uniform: a pass past the tensor has nothing to store
                if constexpr (STAGE_LD)
                    store_flat(t, p, d[p][0], d[p][1]);
                else
                    store_pass(t, p, d[p][0], d[p][1]);
            }
        }
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
        if constexpr (EAGER) {
            E::round_pair(c0, s0);
            E::round_pair(c1, s1v);
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
        if constexpr (STAGE_LD)
            unstage(d[p][0], d[p][1]);
        const float s0 = E::sumsq(d[p][0], 0.0f);
        const float part = (own0 ? s0 : 0.0f) + (own1 ? E::sumsq(d[p][1], 0.0f) : 0.0f);
        const float rrms = rms_rsqrt(group_sum<LPR>(part) * inv_d + eps, eps_normal);
        float x0[VE], x1[VE];
        E::unpack(d[p][0], x0);
        E::unpack(d[p][1], x1);
        if constexpr (EAGER) {
            // (act)((act)(x * rrms) * w)
#pragma unroll
            for (int e = 0; e < VE; ++e) {
                x0[e] = x0[e] * rrms;
                x1[e] = x1[e] * rrms;
            }
            E::round_trip(x0);
            E::round_trip(x1);
#pragma unroll
            for (int e = 0; e < VE; ++e) {
                x0[e] = x0[e] * w0[e];
                x1[e] = x1[e] * w1[e];
            }
        } else {
#pragma unroll
            for (int e = 0; e < VE; ++e) {
                x0[e] = x0[e] * rrms * w0[e];
                x1[e] = x1[e] * rrms * w1[e];
            }
        }
        E::round_trip(x0);
        E::round_trip(x1);
        // One pair: a' = a c - b s, b' = b c + a s (unfused for EAGER).
        auto rot = [](float& xa, float& xb, float c, float sn) {
            if constexpr (EAGER) {
                rotate_unfused(xa, xb, c, sn);
            } else {
                const float a0 = xa, b0 = xb;
                xa = a0 * c - b0 * sn;
                xb = b0 * c + a0 * sn;
            }
        };
        if constexpr (ROT) {
            if constexpr (PAIRING == kNeox) {
                if (rot_lane) {
#pragma unroll
                    for (int e = 0; e < VE; ++e)
                        rot(x0[e], x1[e], cs_c[e], cs_s[e]);
                }
            } else {
#pragma unroll
                for (int q = 0; q < VE / 2; ++q) {
                    if (v0 * (VE / 2) + q < half)
                        rot(x0[2 * q], x0[2 * q + 1], cs_c[q], cs_s[q]);
                    if (v1 * (VE / 2) + q < half)
                        rot(x1[2 * q], x1[2 * q + 1], cs_c[VE / 2 + q], cs_s[VE / 2 + q]);
                }
            }
        }
        store_pass(dst, p, E::pack(x0), E::pack(x1));
    }
}

template <class E, int LPR, int ROPE, int PAIRING, bool NT, bool STAGE, bool EAGER>
NormRopeFn pick_np(int np)
{
    switch (np) {
    case 1: return norm_rope_kernel<E, LPR, 1, ROPE, PAIRING, NT, STAGE, EAGER>;
    case 2: return norm_rope_kernel<E, LPR, 2, ROPE, PAIRING, NT, STAGE, EAGER>;
    case 3: return norm_rope_kernel<E, LPR, 3, ROPE, PAIRING, NT, STAGE, EAGER>;
    default: return norm_rope_kernel<E, LPR, 4, ROPE, PAIRING, NT, STAGE, EAGER>;
    }
}

// Staged stores exist for 2..8 lanes per row (rows up to 16 vectors, the
// only ones whose halves can miss 128-byte lines).
template <class E, int LPR, int ROPE, int PAIRING, bool EAGER>
NormRopeFn pick_nt(bool nt, bool stage, int np)
{
    constexpr bool kCanStage = LPR >= 2 && LPR <= 8;
    if (kCanStage && stage)
        return nt ? pick_np<E, LPR, ROPE, PAIRING, true, kCanStage, EAGER>(np)
                  : pick_np<E, LPR, ROPE, PAIRING, false, kCanStage, EAGER>(np);
    return nt ? pick_np<E, LPR, ROPE, PAIRING, true, false, EAGER>(np)
              : pick_np<E, LPR, ROPE, PAIRING, false, false, EAGER>(np);
}

template <class E, int LPR, int ROPE, bool EAGER>
NormRopeFn pick_pairing(int pairing, bool nt, bool stage, int np)
{
    return pairing == kNeox ? pick_nt<E, LPR, ROPE, kNeox, EAGER>(nt, stage, np)
                            : pick_nt<E, LPR, ROPE, kAdjacent, EAGER>(nt, stage, np);
}

template <class E, int LPR, bool EAGER>
NormRopeFn pick_rope(int rope, int pairing, bool nt, bool stage, int np)
{
    switch (rope) {
    case 0: return pick_pairing<E, LPR, 0, EAGER>(pairing, nt, stage, np);
    case 1: return pick_pairing<E, LPR, 1, EAGER>(pairing, nt, stage, np);
    case 2: return pick_pairing<E, LPR, 2, EAGER>(pairing, nt, stage, np);
    default: return pick_pairing<E, LPR, 3, EAGER>(pairing, nt, stage, np);
    }
}

// ---------------------------------------------------------------------------
// Token tiles: one wavefront takes every Q and K row of one token.
//
// Rows of nv vectors need L = ceil(nv / 2) lanes (a lane owns two vectors, as
// in the tile kernel above).  Where L is not a power of two (3, 5, 6, 7: bf16
// head_dim 48, 80, 96, 112) the tile kernel's row groups of 4 or 8 lanes leave
// lanes idle (3 of 8 for head_dim 80); here rows take L lanes each, 64 / L
// rows per pass, Q rows first, then K rows.  The token's rows (at most
// kTokenVecs 16-byte vectors: its Q vectors, then its K vectors) sit in the
// wave's LDS slice; each lane reads its two vectors of a row from there, the
// results go back, and the token leaves as flat stores: slot s of a tensor is
// its vectors 64 s + lane (contiguous when the tensor's heads are), Q slots
// first, so every store has a wave-uniform base and a 32-bit lane offset (the
// host keeps a tensor's rows of one token within 2^31 bytes).  A row's sum of
// squares is gathered from its L lanes by ds_bpermute in one fixed order, so
// every lane of the row gets the same total.  cos/sin are computed once per
// token instead of once per tensor.
//
// The rows reach the slice in one of two ways (token_dma):
//   - LDS DMA (gfx950's global_load_lds_dwordx4): memory to LDS with no
//     vector registers in between, flat over the token's vectors (slot s =
//     vectors 64 s + lane; lanes past the last vector re-read it into the
//     slice's unused tail), every lane loading, so no load sits behind a
//     branch.  The weight vectors stay in the registers of lanes 0 .. 2 nv - 1
//     and reach a row's lanes by ds_bpermute, so the slice is 20 KB per
//     workgroup of four waves and eight workgroups fit a compute unit.
//   - Register loads per tensor slot, written to the slice once the trig is
//     done, the weight vectors beside them in the slice (22 KB, seven
//     workgroups).  The compiler counts LDS DMA apart from plain loads and
//     makes the first wait after one a wait for every outstanding load, so
//     with DMA the angle computation, which needs the lane's inverse
//     frequency, would start only once every row had arrived: where the
//     angles come from positions that costs more than the DMA saves.  NeoX
//     rows of 7 lanes need 73 registers with DMA (six waves per SIMD).
// Measured (8192 tokens, bf16, token-tile time with DMA / with register
// loads): head_dim 80, 16 + 16 heads: norm only 0.84, cos/sin planes 0.95,
// 1-D or t/h/w positions 1.00 to 1.06; ViT grid positions (7952 tokens) 0.90;
// head_dim 96 (12 + 12 heads) planes 0.93, positions 1.06 to 1.09; 112
// (11 + 11) planes 1.07, positions 1.17; 48 (26 + 26) planes 0.87.
// ---------------------------------------------------------------------------
constexpr int kTokenVecs = kTokenTileVecs;   // row vectors of one token held in LDS (5 per lane)
constexpr int kTokenWeightVecs = 32;          // weight vectors in the slice (register loads): two rows of at most 16

// Rows by LDS DMA: norm only always; cos/sin from planes or ViT grids up to 6
// lanes per row; never where the angles come from positions.
template <int ROPE, int L>
constexpr bool token_dma() { return ROPE == 0 || (ROPE != 1 && L <= 6); }

template <class E, int L, int ROPE, int PAIRING, bool NT, bool EAGER>
__global__ __launch_bounds__(kThreads) void norm_rope_token_kernel(const NormRopeArgs a)
{
    constexpr int VE = E::VE;
    constexpr int RP = 64 / L;                         // rows per pass
    constexpr bool ROT = ROPE != 0;
    constexpr int kSlots = kTokenVecs / 64;           // slots of 64 vectors in the slice
    static_assert(kTokenVecs % 64 == 0, "the slice holds whole slots");
    static_assert(L >= 3 && L <= 7 && (L & (L - 1)) != 0, "token tiles serve 3, 5, 6 or 7 lanes per row");
    constexpr bool DMA = token_dma<ROPE, L>();
    constexpr int kSlice = kTokenVecs + (DMA ? 0 : kTokenWeightVecs);
    static_assert(!DMA || kWaves * kSlice * 16 <= 160 * 1024 / 8, "eight DMA workgroups per compute unit");
    __shared__ uint4 lds_all[kWaves * kSlice];

    const int lane = threadIdx.x & 63;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    uint4* const st = lds_all + wave * kSlice;
    uint4* const wst = st + kTokenVecs;   // weight vectors in the slice: register loads only

    const TensorArgs& TQ = a.t[0];
    const TensorArgs& TK = a.t[1];
    const RopeArgs& rp = a.rope;
    // Every kernel-argument field that the row loads and the lane's pair
    // operand depend on, read in one batch: an empty asm takes them all, so
    // the compiler issues every load before the first wait instead of
    // spreading them over several scalar round trips.
    uint32_t tile_base = a.tile_base, ntiles = a.ntiles, td = a.div_tokens.d, tm = a.div_tokens.m,
             tsh = a.div_tokens.sh, nv_recip = a.nv_recip;
    int32_t head_dim = a.head_dim, rotary_dim = a.rotary_dim, hq = TQ.heads, hk = TK.heads, half = rp.half;
    const char* qbase = TQ.s[0].in;
    const char* kbase = TK.s[0].in;
    int64_t qsb = TQ.s[0].sb, qst = TQ.s[0].st, ksb = TK.s[0].sb, kst = TK.s[0].st, token_base = rp.token_base;
    int32_t shq = (int32_t)TQ.s[0].sh, shk = (int32_t)TK.s[0].sh;
    asm("" : "+s"(tile_base), "+s"(ntiles), "+s"(td), "+s"(tm), "+s"(tsh), "+s"(nv_recip), "+s"(head_dim),
             "+s"(rotary_dim), "+s"(hq), "+s"(hk), "+s"(half), "+s"(qbase), "+s"(kbase), "+s"(qsb), "+s"(qst),
             "+s"(ksb), "+s"(kst), "+s"(token_base), "+s"(shq), "+s"(shk));

    // Tile = batch * tokens + token.  Padding waves of the last workgroup redo
    // the last tile and store nothing.
    const uint32_t tile_raw = tile_base + blockIdx.x * kWaves + wave;
    const bool pad = tile_raw >= ntiles;
    const uint32_t tile = pad ? ntiles - 1 : tile_raw;
    const FastDiv div_tokens{td, tm, tsh};
    const uint32_t bq = fast_div(tile, div_tokens);
    const int32_t tok = (int32_t)(tile - bq * td);
    const int32_t b = (int32_t)bq;

    const int nv = (int)((uint32_t)head_dim / VE);
    const int rows = hq + hk;
    const int nq = hq * nv, nk = hk * nv;              // nq + nk <= kTokenVecs (the planner's condition)
    const int ntot = nq + nk;
    const char* const qin = qbase + (int64_t)(uint32_t)b * qsb + (int64_t)(uint32_t)tok * qst;
    const char* const kin = kbase + (int64_t)(uint32_t)b * ksb + (int64_t)(uint32_t)tok * kst;

    // Byte offset within its tensor's token of the tensor's flat vector f.
    auto flat_off = [&](int f, int32_t sh) {
        const int fr = (int)(((uint32_t)f * nv_recip) >> 16);
        return (uint32_t)(fr * sh + (f - fr * nv) * 16);
    };

    // The lane's place in a row: vectors v0 and v1, as in the tile kernel.
    const int g = lane / L, j = lane - (lane / L) * L;
    int v0, v1;
    bool rot_lane = false;
    if (PAIRING == kNeox && ROT) {
        const int nr = (int)((uint32_t)rotary_dim / (2 * VE));
        if (j < nr) {
            v0 = j;
            v1 = j + nr;
            rot_lane = true;
        } else {
            v0 = 2 * nr + 2 * (j - nr);
            v1 = v0 + 1;
        }
    } else {
        const int hv = (nv + 1) >> 1;
        v0 = j;
        v1 = j + hv;
    }
    const bool own0 = v0 < nv, own1 = v1 < nv;
    const int c0i = own0 ? v0 : 0, c1i = own1 ? v1 : 0;

    // 1) Loads: the lane's pair operand, the token's rows (into the slice by
    //    LDS DMA, or into registers), the weight vectors.
    const int64_t tabs = token_base + tok;
    const int p0 = lane < half ? lane : half - 1;
    float op0 = 0.0f, os0 = 0.0f;
    int32_t ax0 = 0;
    if constexpr (ROPE == 1)
        op0 = load_global(uniform(rp.inv_freq) + p0);
    if constexpr (ROPE == 2) {
        ax0 = axis_of(rp.axis_bits, p0);
        const int64_t i0 = ((int64_t)ax0 * rp.planes_tokens + tabs) * half + p0;
        op0 = rp.cos_planes[i0];
        os0 = rp.sin_planes[i0];
    }
    if constexpr (ROPE == 3) {
        ax0 = axis_of(rp.axis_bits, p0);
        const int32_t o_h = rp.sec[0], o_w = rp.sec[0] + rp.sec[1];
        const float* const l0 = sel3(ax0, uniform(a.vit.inv[0]), uniform(a.vit.inv[1]), uniform(a.vit.inv[2]));
        op0 = load_global(l0 + (p0 - sel3(ax0, 0, o_h, o_w)));
    }
    // Slot s of a tensor: its vectors 64 s + lane (register loads: past its
    // last vector a re-read of it), Q slots first; every base wave-uniform.
    constexpr int kRegSlots = DMA ? 1 : kSlots + 1;
    const int sq = (nq + 63) >> 6;
    auto slot_is_k = [&](int s) { return s >= sq && hk > 0; };
    auto slot_in_tensor = [&](int s) { return s >= sq ? s - sq : s; };
    uint4 fl[kRegSlots];
    if constexpr (DMA) {
#pragma unroll
        for (int s = 0; s < kSlots; ++s) {
            const int f = 64 * s + lane < ntot ? 64 * s + lane : ntot - 1;
            const bool isq = f < nq;
            lds_dma16<NT>((isq ? qin : kin) + flat_off(isq ? f : f - nq, isq ? shq : shk), st + 64 * s);
        }
    } else {
#pragma unroll
        for (int s = 0; s < kRegSlots; ++s) {
            const bool isk = slot_is_k(s);
            const int n = isk ? nk : nq;
            const int f = 64 * slot_in_tensor(s) + lane;
            fl[s] = load_row16<NT>((isk ? kin : qin) +
                                   flat_off(f < n ? f : n - 1, isk ? shk : shq));
        }
    }
    // Weight vectors: lanes [0, nv) the Q tensor's, [nv, 2 nv) the K tensor's
    // (an absent tensor's lanes read the other one's: never used).
    const char* const wq = hq > 0 ? TQ.s[0].weight : TK.s[0].weight;
    const char* const wk = hk > 0 ? TK.s[0].weight : TQ.s[0].weight;
    const int wl = lane < nv ? lane : (lane < 2 * nv ? lane - nv : 0);
    const uint4 wv = load16((lane < nv ? wq : wk) + wl * 16);

    TokenPositions pos{0, 0, 0, 0};
    if constexpr (ROPE == 1) {
        pos.t = (int32_t)uniform((uint32_t)rp.positions[rp.plane_off[0] + tabs]);
        pos.h = (int32_t)uniform((uint32_t)rp.positions[rp.plane_off[1] + tabs]);
        pos.w = (int32_t)uniform((uint32_t)rp.positions[rp.plane_off[2] + tabs]);
        pos.e = (int32_t)uniform((uint32_t)rp.positions[rp.plane_off[3] + tabs]);
    }
    if constexpr (ROPE == 3)
        pos = vit_token_positions(a.vit, (uint32_t)tabs);

    // 2) cos/sin of the lane's VE pairs, once for the token.
    float cs_c[VE], cs_s[VE];
#pragma unroll
    for (int e = 0; e < VE; ++e) {
        cs_c[e] = 1.0f;
        cs_s[e] = 0.0f;
    }
    if constexpr (ROT) {
        float c0, s0;
        if constexpr (ROPE == 2) {
            c0 = op0;
            s0 = os0;
        } else {
            if constexpr (ROPE == 1)
                ax0 = axis_of(rp.axis_bits, p0);
            pair_cos_sin(ax0, pos, op0, c0, s0);
        }
        if constexpr (EAGER)
            E::round_pair(c0, s0);
#pragma unroll
        for (int e = 0; e < VE; ++e) {
            int p;
            if constexpr (PAIRING == kNeox)
                p = j * VE + e;
            else
                p = (e < VE / 2 ? v0 : v1) * (VE / 2) + (e % (VE / 2));
            cs_c[e] = bperm(p, c0);
            cs_s[e] = bperm(p, s0);
        }
    }

    if constexpr (DMA) {
        // Every row in the slice: the LDS DMA writes complete under vmcnt.
        __builtin_amdgcn_s_waitcnt(0);
    } else {
        // The rows and the weights into the slice; re-reads are dropped.
#pragma unroll
        for (int s = 0; s < kRegSlots; ++s) {
            const bool isk = slot_is_k(s);
            const int f = 64 * slot_in_tensor(s) + lane;
            if (f < (isk ? nk : (s < sq ? nq : 0)))
                st[(isk ? nq : 0) + f] = fl[s];
        }
        if (lane < 2 * nv)
            wst[lane] = wv;
    }
    wave_lds_order();

    // 3) Per pass of RP rows: the row's two vectors of this lane, the sum of
    //    squares over the row's L lanes, normalise, round, rotate, back into
    //    the slice.
    const float eps = a.eps, inv_d = a.inv_d;
    const bool eps_normal = eps >= FLT_MIN;
    const int base = g * L;
#pragma unroll
    for (int p = 0; p < 3; ++p) {
        if (p * RP >= rows)
            break;   // wave-uniform
        const int r = p * RP + g;
        const bool valid = g < RP && r < rows;
        const int rr = valid ? r : rows - 1;
        const uint4 d0 = st[rr * nv + c0i], d1 = st[rr * nv + c1i];
        const float part = (own0 ? E::sumsq(d0, 0.0f) : 0.0f) + (own1 ? E::sumsq(d1, 0.0f) : 0.0f);
        float tot = bperm(base, part);
#pragma unroll
        for (int k = 1; k < L; ++k)
            tot += bperm(base + k, part);
        const float rrms = rms_rsqrt(tot * inv_d + eps, eps_normal);
        const int wb = rr < hq ? 0 : nv;
        float x0[VE], x1[VE], w0[VE], w1[VE];
        E::unpack(d0, x0);
        E::unpack(d1, x1);
        if constexpr (DMA) {
            E::unpack(bperm16(wb + c0i, wv), w0);
            E::unpack(bperm16(wb + c1i, wv), w1);
        } else {
            E::unpack(wst[wb + c0i], w0);
            E::unpack(wst[wb + c1i], w1);
        }
        if constexpr (EAGER) {
#pragma unroll
            for (int e = 0; e < VE; ++e) {
                x0[e] = x0[e] * rrms;
                x1[e] = x1[e] * rrms;
            }
            E::round_trip(x0);
            E::round_trip(x1);
#pragma unroll
            for (int e = 0; e < VE; ++e) {
                x0[e] = x0[e] * w0[e];
                x1[e] = x1[e] * w1[e];
            }
        } else {
#pragma unroll
            for (int e = 0; e < VE; ++e) {
                x0[e] = x0[e] * rrms * w0[e];
                x1[e] = x1[e] * rrms * w1[e];
            }
        }
        E::round_trip(x0);
        E::round_trip(x1);
        auto rot = [](float& xa, float& xb, float c, float sn) {
            if constexpr (EAGER) {
                rotate_unfused(xa, xb, c, sn);
            } else {
                const float a0 = xa, b0 = xb;
                xa = a0 * c - b0 * sn;
                xb = b0 * c + a0 * sn;
            }
        };
        if constexpr (ROT) {
            if constexpr (PAIRING == kNeox) {
                if (rot_lane) {
#pragma unroll
                    for (int e = 0; e < VE; ++e)
                        rot(x0[e], x1[e], cs_c[e], cs_s[e]);
                }
            } else {
#pragma unroll
                for (int q = 0; q < VE / 2; ++q) {
                    if (v0 * (VE / 2) + q < half)
                        rot(x0[2 * q], x0[2 * q + 1], cs_c[q], cs_s[q]);
                    if (v1 * (VE / 2) + q < half)
                        rot(x1[2 * q], x1[2 * q + 1], cs_c[VE / 2 + q], cs_s[VE / 2 + q]);
                }
            }
        }
        if (valid) {
            if (own0)
                st[rr * nv + v0] = E::pack(x0);
            if (own1)
                st[rr * nv + v1] = E::pack(x1);
        }
    }
    wave_lds_order();

    // 4) The token's results leave as flat vectors.
    if (pad)
        return;
    char* const qout = TQ.out + (int64_t)b * TQ.out_sb + (int64_t)tok * TQ.out_st;
    char* const kout = TK.out + (int64_t)b * TK.out_sb + (int64_t)tok * TK.out_st;
#pragma unroll
    for (int s = 0; s < kSlots + 1; ++s) {
        const bool isk = slot_is_k(s);
        const int f = 64 * slot_in_tensor(s) + lane;
        if (f < (isk ? nk : (s < sq ? nq : 0)))
            store_row16<NT>((isk ? kout : qout) + flat_off(f, (int32_t)(isk ? TK.out_sh : TQ.out_sh)),
                            st[(isk ? nq : 0) + f]);
    }
}

template <class E, int L, int ROPE, bool EAGER>
NormRopeFn pick_token_nt(int32_t pairing, bool nt)
{
    if (pairing == kNeox)
        return nt ? norm_rope_token_kernel<E, L, ROPE, kNeox, true, EAGER>
                  : norm_rope_token_kernel<E, L, ROPE, kNeox, false, EAGER>;
    return nt ? norm_rope_token_kernel<E, L, ROPE, kAdjacent, true, EAGER>
              : norm_rope_token_kernel<E, L, ROPE, kAdjacent, false, EAGER>;
}

template <class E, int L, bool EAGER>
NormRopeFn pick_token_rope(int rope, int32_t pairing, bool nt)
{
    switch (rope) {
    case 0: return pick_token_nt<E, L, 0, EAGER>(pairing, nt);
    case 1: return pick_token_nt<E, L, 1, EAGER>(pairing, nt);
    case 2: return pick_token_nt<E, L, 2, EAGER>(pairing, nt);
    default: return pick_token_nt<E, L, 3, EAGER>(pairing, nt);
    }
}

}  // namespace
}  // namespace qkr
