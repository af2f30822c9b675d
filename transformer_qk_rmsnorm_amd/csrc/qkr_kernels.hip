// gfx950 kernels: plain row RMSNorm, ViT cos/sin setup, index-map debug
// kernels, and the launchers of every kernel (the QK RMSNorm + RoPE kernel
// template lives in qkr_rope_kernel.hpp).  All of them are HBM-bound streams:
// rows move as 128-bit vectors and reductions stay inside a wavefront (DPP).
// No atomics, no MFMA (there is no dense contraction in this path).
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
#include "qkr_device.hpp"

namespace qkr {
namespace {

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
template <class E, int VPL, int KIND, bool NT, int MODE>
__global__ __launch_bounds__(kThreads) void rms_kernel(const RmsArgs a)
{
    constexpr int VE = E::VE;
    constexpr bool ADD = (MODE & 1) != 0, FP8 = (MODE & 2) != 0;
    static_assert(!(ADD && KIND == 1), "the split variant cannot update the residual in place");
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
    if constexpr (ADD) {
        // Residual add ([Vulkan] decode RmsNorm: the residual stream is held
        // bit-exactly by rounding the sum in registers): s = x + r rounded once
        // to the activation type is stored as the new residual and normalised.
        // Every lane has read all of its vectors of x and r before it writes,
        // and no other lane touches them, so s may overwrite r or x in place.
        const char* r = a.r + row * a.r_stride;
        uint4 rv[VPL];
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int v = first + k * step;
            rv[k] = v < a.nvec ? load_row16<NT>(r + (int64_t)v * 16) : make_uint4(0, 0, 0, 0);
        }
        char* sres = a.s + row * a.s_stride;
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int v = first + k * step;
            d[k] = E::add(d[k], rv[k]);   // zero + zero on lanes past the row
            if (v < a.nvec)
                store_row16<NT>(sres + (int64_t)v * 16, d[k]);
        }
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
    const float rrms = rms_rsqrt(ss * a.inv_width + a.eps, a.eps >= FLT_MIN);
    float scale = 1.0f, inv_scale = 1.0f;
    if constexpr (FP8) {
        scale = *a.scale;   // wave-uniform
        inv_scale = 1.0f / scale;
    }

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
            if constexpr (FP8) {
                // One E4M3 code per element (VE bytes per vector): the code of
                // the fp32 quotient y / scale.
                uint32_t c[VE / 4];
#pragma unroll
                for (int q = 0; q < VE / 4; ++q)
                    c[q] = fp8_e4m3_pack4(div_by_scale(xv[4 * q], scale, inv_scale),
                                          div_by_scale(xv[4 * q + 1], scale, inv_scale),
                                          div_by_scale(xv[4 * q + 2], scale, inv_scale),
                                          div_by_scale(xv[4 * q + 3], scale, inv_scale));
                char* dst = y + (int64_t)v * VE;
                if constexpr (VE == 8) {
                    typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
                    const u32x2_t pk = {c[0], c[1]};
                    if constexpr (NT)
                        __builtin_nontemporal_store(pk, reinterpret_cast<u32x2_t*>(dst));
                    else
                        *reinterpret_cast<u32x2_t*>(dst) = pk;
                } else {
                    if constexpr (NT)
                        __builtin_nontemporal_store(c[0], reinterpret_cast<uint32_t*>(dst));
                    else
                        *reinterpret_cast<uint32_t*>(dst) = c[0];
                }
            } else {
                store_row16<NT>(y + (int64_t)v * 16, E::pack(xv));
            }
        }
    }
}

// The row kernel's quotient and E4M3 encoding, element by element (tests
// compare them with the correctly rounded quotient and the oracle's encoder
// bit for bit).  scale == nullptr: the values are encoded as they are.
__global__ __launch_bounds__(kThreads) void debug_fp8_kernel(const float* x, int64_t n, const float* scale,
                                                             uint8_t* out)
{
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= n)
        return;
    float v = x[i];
    if (scale != nullptr) {
        const float sc = *scale;
        v = div_by_scale(v, sc, 1.0f / sc);
    }
    out[i] = (uint8_t)(fp8_e4m3_pack4(v, 0.0f, 0.0f, 0.0f) & 0xFFu);
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

// The axis of every pair as the rotation kernels decode it from the table.
__global__ void debug_axis_kernel(const RopeArgs r, int32_t n_pairs, int32_t* out)
{
    const int p = blockIdx.x * blockDim.x + threadIdx.x;
    if (p >= n_pairs)
        return;
    out[p] = axis_of(r.axis_bits, p);
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
using RmsFn = void (*)(RmsArgs);

template <class E, int KIND, bool NT, int MODE>
RmsFn pick_vpl(int vpl)
{
    switch (vpl) {
    case 1: return rms_kernel<E, 1, KIND, NT, MODE>;
    case 2: return rms_kernel<E, 2, KIND, NT, MODE>;
    case 3: return rms_kernel<E, 3, KIND, NT, MODE>;
    case 4: return rms_kernel<E, 4, KIND, NT, MODE>;
    case 5: return rms_kernel<E, 5, KIND, NT, MODE>;
    case 6: return rms_kernel<E, 6, KIND, NT, MODE>;
    case 8: return rms_kernel<E, 8, KIND, NT, MODE>;
    case 10: return rms_kernel<E, 10, KIND, NT, MODE>;
    case 12: return rms_kernel<E, 12, KIND, NT, MODE>;
    default: return rms_kernel<E, 16, KIND, NT, MODE>;
    }
}

// The plain norm comes with and without nontemporal accesses; the add and
// FP8 modes are nontemporal only, and the add modes skip the split variant.
template <class E, int KIND>
RmsFn pick_rms_mode(bool nt, int mode, int vpl)
{
    switch (mode) {
    case 0: return nt ? pick_vpl<E, KIND, true, 0>(vpl) : pick_vpl<E, KIND, false, 0>(vpl);
    case 2: return pick_vpl<E, KIND, true, 2>(vpl);
    default:
        if constexpr (KIND == 1)
            return nullptr;
        else
            return mode == 1 ? pick_vpl<E, KIND, true, 1>(vpl) : pick_vpl<E, KIND, true, 3>(vpl);
    }
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

hipError_t launch_norm_rope(const NormRopeArgs& a_in, int32_t dtype, int32_t pairing, int np, int lpr_req,
                            int stage_req, int nt, hipStream_t stream, const char** variant)
{
    NormRopeArgs a = a_in;
    const int ve = dtype == kBF16 ? 8 : 4;
    const int nv = a.head_dim / ve;
    // Lanes per row: the smallest power of two that gives every lane at most
    // two vectors of the row.
    int lpr = 1;
    while (2 * lpr < nv)
        lpr *= 2;
    if (lpr_req > 0 && (lpr_req & (lpr_req - 1)) == 0 && lpr_req <= 32 && 2 * lpr_req >= nv)
        lpr = lpr_req;
    const int rpp = 64 / lpr;
    int max_heads = 0;
    for (int i = 0; i < 3; ++i)
        max_heads = a.t[i].heads > max_heads ? a.t[i].heads : max_heads;
    if (np <= 0) {
        // Two passes per tile where the tensor has two or more passes of
        // heads.  Measured on MI355X with two / one / three passes: the joint
        // op (24 heads of 128) 29.7 / 30.0 / 30.3 us, fused ViT (16 + 16
        // heads of 80) 19.8 / 24.1 / 21.2 us, a 2048-token IMROPE chunk
        // (16 + 8 heads of 128) 5.94 / 6.61 / 6.15 us.
        const int passes = (max_heads + rpp - 1) / rpp;
        np = passes >= 2 ? 2 : 1;
    }
    np = np < 1 ? 1 : (np > 4 ? 4 : np);
    const int rope = a.rope.mode == kPosNone ? 0
                     : (a.rope.mode == kPosPlanes ? 2 : (a.rope.mode == kPosVit ? 3 : 1));
    const int rpw = rpp * np;
    int32_t tpt = 0;
    for (int i = 0; i < 3; ++i) {
        a.tile_first[i] = tpt;
        tpt += (a.t[i].heads + rpw - 1) / rpw;
    }
    const int64_t tiles = (int64_t)a.batch * a.tokens * tpt;
    if (tiles == 0)
        return hipSuccess;
    if (tiles >= ((int64_t)1 << 31))
        return hipErrorInvalidValue;   // the host layer refuses such calls first
    a.ntiles = (uint32_t)tiles;
    a.div_tpt = make_fastdiv((uint32_t)tpt);
    a.div_tokens = make_fastdiv((uint32_t)a.tokens);
    const int64_t blocks = (tiles + kWaves - 1) / kWaves;
    const bool use_nt = nt != 0;
    // Staged stores where a half row is not a whole number of 128-byte lines.
    bool stage = stage_req < 0 ? nv % 16 != 0 : stage_req != 0;
    stage = stage && lpr >= 2 && lpr <= 8;
    a.nv_recip = (65536u + (uint32_t)nv - 1) / (uint32_t)nv;
    NormRopeFn fn;
    switch (lpr) {
    case 1: fn = pick_norm_rope<1>(dtype, rope, pairing, use_nt, stage, np); break;
    case 2: fn = pick_norm_rope<2>(dtype, rope, pairing, use_nt, stage, np); break;
    case 4: fn = pick_norm_rope<4>(dtype, rope, pairing, use_nt, stage, np); break;
    case 8: fn = pick_norm_rope<8>(dtype, rope, pairing, use_nt, stage, np); break;
    case 16: fn = pick_norm_rope<16>(dtype, rope, pairing, use_nt, stage, np); break;
    default: fn = pick_norm_rope<32>(dtype, rope, pairing, use_nt, stage, np); break;
    }
    hipLaunchKernelGGL(fn, dim3((uint32_t)blocks), dim3(kThreads), 0, stream, a);
    snprintf(g_variant, sizeof(g_variant), "rope:np%d:nt%d:lpr%d:%s:%s:%s:stage%d", np, (int)use_nt, lpr,
             dtype == kBF16 ? "bf16" : "f32",
             rope == 0 ? "none" : (rope == 1 ? "pos" : (rope == 2 ? "planes" : "vit")),
             pairing == kNeox ? "neox" : "adjacent", (int)stage);
    *variant = g_variant;
    return hipGetLastError();
}

hipError_t launch_rms_norm(RmsArgs a, int32_t dtype, int kind, int nt, int mode, hipStream_t stream,
                           const char** variant)
{
    if (a.rows == 0)
        return hipSuccess;
    const bool add = (mode & 1) != 0;
    if (kind < 0) {
        // A workgroup per row below 2048 rows, a wavefront per row above.
        // Measured on MI355X, rows of 5120 bf16 (wide / one wave per row /
        // split): 1 row 2.16 / 3.27 / 2.23 us, 32 rows 2.82 / 4.50 / 3.31,
        // 128 rows 3.04 / 4.78 / 4.30, 1024 rows 4.95 / 5.97, 2048 rows 7.95
        // / 8.18, 4096 rows 15.6 / 13.8.  The split variant never wins; it
        // stays reachable through the variant override.
        kind = a.rows < 2048 && a.nvec >= 64 ? 2 : 0;
    }
    if (add && kind == 1)
        kind = 2;
    if (mode != 0)
        nt = 1;
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
        fn = kind == 0 ? pick_rms_mode<BF16, 0>(use_nt, mode, vpl)
                       : (kind == 1 ? pick_rms_mode<BF16, 1>(use_nt, mode, vpl)
                                    : pick_rms_mode<BF16, 2>(use_nt, mode, vpl));
    else
        fn = kind == 0 ? pick_rms_mode<F32, 0>(use_nt, mode, vpl)
                       : (kind == 1 ? pick_rms_mode<F32, 1>(use_nt, mode, vpl)
                                    : pick_rms_mode<F32, 2>(use_nt, mode, vpl));
    if (fn == nullptr)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(fn, dim3((uint32_t)blocks), dim3(kThreads), 0, stream, a);
    snprintf(g_variant, sizeof(g_variant), "rms:%s:nt%d:vpl%d:%s%s%s",
             kind == 0 ? "rows" : (kind == 1 ? "split" : "wide"), (int)use_nt, vpl, dtype == kBF16 ? "bf16" : "f32",
             add ? ":add" : "", (mode & 2) ? ":fp8" : "");
    *variant = g_variant;
    return hipGetLastError();
}

hipError_t launch_debug_fp8(const float* x, int64_t n, const float* scale, uint8_t* out, hipStream_t stream)
{
    if (n == 0)
        return hipSuccess;
    hipLaunchKernelGGL(debug_fp8_kernel, dim3((uint32_t)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                       stream, x, n, scale, out);
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

hipError_t launch_debug_axis_map(const RopeArgs& r, int32_t n_pairs, int32_t* out, hipStream_t stream)
{
    if (n_pairs == 0)
        return hipSuccess;
    hipLaunchKernelGGL(debug_axis_kernel, dim3((n_pairs + 63) / 64), dim3(64), 0, stream, r, n_pairs, out);
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
