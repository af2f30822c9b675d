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
// STAGE: where half a row is not a whole number of 128-byte lines (e.g.
// head_dim 80 bf16: 80-byte halves), a store instruction of the lane-local
// layout would cover every line it touches only in part, and partial-line
// writes cost HBM efficiency.  The pass's results then go through a per-wave
// LDS slice indexed by (row, vector) and leave as vectors lane and 64 + lane
// of the pass, i.e. contiguous 1 KB runs when a token's heads are adjacent.
//
// ROPE: 0 norm only, 1 positions + inv_freq (1D / AXES / IMROPE chosen at run
// time), 2 cos/sin planes, 3 ViT positions computed from the grid table.
// ---------------------------------------------------------------------------
template <class E, int LPR, int NP, int ROPE, int PAIRING, bool NT, bool STAGE>
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
    __shared__ uint4 stage_all[STAGE ? kWaves * 128 : 1];
    uint4* const stage = stage_all + (STAGE ? wave * 128 : 0);   // RPP * nv <= 2 * 64 vectors
    const float eps = a.eps, inv_d = a.inv_d;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const int r = blk * RPW + p * RPP + g;
        const bool row_ok = r < a.rows_per_token;
        uint4 o0 = d[p][0], o1 = d[p][1];   // routed tensor (V): bit copy
        int ti, h;
        locate(r, ti, h);
        if (row_ok && r < a.rope_rows) {
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
            o0 = E::pack(x0);
            o1 = E::pack(x1);
        }
        if constexpr (STAGE) {
            if (row_ok) {
                if (own0) stage[g * nv + v0] = o0;
                if (own1) stage[g * nv + v1] = o1;
            }
            wave_lds_order();
#pragma unroll
            for (int sl = 0; sl < 2; ++sl) {
                const int f = sl * 64 + lane;                       // vector of the pass
                const int fr = (int)(((uint32_t)f * a.nv_recip) >> 16); // its row in the pass
                const int fv = f - fr * nv;
                const int rf = blk * RPW + p * RPP + fr;
                if (fr < RPP && rf < a.rows_per_token) {
                    int tf, hf;
                    locate(rf, tf, hf);
                    char* obase = tf == 0 ? R0.out : (tf == 1 ? R1.out : R2.out);
                    const int64_t osh = tf == 0 ? R0.out_sh : (tf == 1 ? R1.out_sh : R2.out_sh);
                    store_row16<NT>(obase + (int64_t)hf * osh + (int64_t)fv * 16, stage[f]);
                }
            }
            wave_lds_order();
        } else if (row_ok) {
            char* obase = ti == 0 ? R0.out : (ti == 1 ? R1.out : R2.out);
            const int64_t osh = ti == 0 ? R0.out_sh : (ti == 1 ? R1.out_sh : R2.out_sh);
            char* orow = obase + (int64_t)h * osh;
            if (own0) store_row16<NT>(orow + off0, o0);
            if (own1) store_row16<NT>(orow + off1, o1);
        }
    }
}

// ---------------------------------------------------------------------------
// Dispatch tables
// ---------------------------------------------------------------------------
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
