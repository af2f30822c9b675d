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
#include <mutex>
#include <unordered_map>
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
// EAGER: y = (act)((act)(x * rrms) * w), the output expression of the eager
// RMSNorm kernel the [VecRMS] review thread quotes, instead of one rounding
// of x * rrms * w (activation-type outputs only).
// ---------------------------------------------------------------------------
template <class E, int VPL, int KIND, bool NT, int MODE, bool EAGER>
__global__ __launch_bounds__(kThreads) void rms_kernel(const RmsArgs a)
{
    constexpr int VE = E::VE;
    constexpr bool ADD = (MODE & 1) != 0, FP8 = (MODE & 2) != 0;
    static_assert(!(ADD && KIND == 1), "the split variant cannot update the residual in place");
    static_assert(!(FP8 && EAGER), "the eager numerics are defined for activation-type outputs");
    const int lane = threadIdx.x & 63;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int64_t row;
    int split = 0;
    int first, step;   // vector index of the lane's slot 0, distance between slots
    if constexpr (KIND == 0) {
        row = a.item_base + blockIdx.x * kWaves + wave;
        first = lane;
        step = 64;
    } else if constexpr (KIND == 1) {
        const uint32_t item = (uint32_t)a.item_base + blockIdx.x * kWaves + wave;
        const uint32_t r = fast_div(item, a.div_splits);
        row = r;
        split = (int)(item - r * a.div_splits.d);
        first = lane;
        step = 64;
    } else {
        row = a.item_base + blockIdx.x;
        first = threadIdx.x;
        step = kThreads;
    }
    if (row >= a.rows)
        return;   // wave-uniform (workgroup-uniform for KIND 2)

    // How the row is reached, chosen per variant by measurement (rows of
    // 5120 bf16 on MI355X):
    //  * EARLY (workgroup-per-row and split variants, the few-row launches,
    //    and the wave-per-row FP8 output): every load (weights, x, the
    //    residual) is issued before the first store and no access branches.
    //    Stores go through a buffer resource over their row, whose range
    //    check drops a store past the row.  Stores count in the same
    //    vector-memory counter as loads: a load issued after a store makes
    //    whatever waits for it wait for the store too.  Rows are read through
    //    buffer resources as well (a load past the row reads zeros, which add
    //    nothing to the sum of squares), except in the wave-per-row FP8
    //    variant, which reads them with global loads clamped into the row and
    //    zeroed past it (measured 26.15 us for 4096 rows against 26.4 through
    //    buffers and 26.5 guarded).  1 / 32 rows: 1.84 / 2.20 us against
    //    2.13 / 2.50 us guarded; one row with the residual add 2.07 against
    //    2.36 us.
    //  * guarded (wave-per-row bf16 / fp32 outputs, 2048 to 4096 rows):
    //    per-slot range tests, the weight vector read beside each output
    //    vector.  The launch is a single round of waves, and there the
    //    store-by-store pacing this gives measured faster than issuing every
    //    load first: 4096 rows 13.95 against 15.3 us, with the residual add
    //    27.4 against 28.8 us.
    constexpr bool EARLY = KIND != 0 || FP8;
    constexpr bool BUF_ROWS = KIND != 0;
    const uint32_t row_bytes = (uint32_t)a.nvec * 16;
    float scale = 1.0f;
    if constexpr (FP8)
        scale = *a.scale;   // wave-uniform
    const __amdgpu_buffer_rsrc_t wr = buffer_rsrc(a.w, row_bytes);
    uint4 wv[EARLY ? VPL : 1];
    if constexpr (EARLY) {
#pragma unroll
        for (int k = 0; k < VPL; ++k)
            wv[k] = buffer_load16<false>(wr, (uint32_t)(first + k * step) * 16);
    }
    // Slot k of a row: the lane's vector first + k * step, zero past the row.
    auto load_slot = [&](const char* rowp, const __amdgpu_buffer_rsrc_t& rr, int k) {
        const int v = first + k * step;
        if constexpr (BUF_ROWS) {
            return buffer_load16<NT>(rr, (uint32_t)v * 16);
        } else if constexpr (EARLY) {
            uint4 t = load_row16<NT>(rowp + (int64_t)min(v, a.nvec - 1) * 16);
            if (v >= a.nvec)
                t = make_uint4(0, 0, 0, 0);
            return t;
        } else {
            return v < a.nvec ? load_row16<NT>(rowp + (int64_t)v * 16) : make_uint4(0, 0, 0, 0);
        }
    };
    const char* const xrow = a.x + row * a.x_stride;
    const __amdgpu_buffer_rsrc_t xr = buffer_rsrc(xrow, row_bytes);
    uint4 d[VPL];
#pragma unroll
    for (int k = 0; k < VPL; ++k)
        d[k] = load_slot(xrow, xr, k);
    if constexpr (ADD) {
        // Residual add ([Vulkan] decode RmsNorm: the residual stream is held
        // bit-exactly by rounding the sum in registers): s = x + r rounded once
        // to the activation type is stored as the new residual and normalised.
        // Every lane has read all of its vectors of x and r before it writes,
        // and no other lane touches them, so s may overwrite r or x in place.
        const char* const rrow = a.r + row * a.r_stride;
        const __amdgpu_buffer_rsrc_t rr = buffer_rsrc(rrow, row_bytes);
        uint4 rv[VPL];
#pragma unroll
        for (int k = 0; k < VPL; ++k)
            rv[k] = load_slot(rrow, rr, k);
        char* const srow = a.s + row * a.s_stride;
        const __amdgpu_buffer_rsrc_t sr = buffer_rsrc(srow, row_bytes);
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int v = first + k * step;
            d[k] = E::add(d[k], rv[k]);   // zero + zero past the row
            if constexpr (EARLY)
                buffer_store16<NT>(d[k], sr, (uint32_t)v * 16);
            else if (v < a.nvec)
                store_row16<NT>(srow + (int64_t)v * 16, d[k]);
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
    const float inv_scale = FP8 ? 1.0f / scale : 1.0f;

    // Output vectors [lo, hi) of the row (the split variant's slice).  EARLY:
    // through a resource over just those vectors, a slot outside them sent to
    // offset `out_bytes`, which the range check drops.
    constexpr uint32_t OUT_VB = FP8 ? VE : 16;   // output bytes per vector
    int lo = 0, hi = a.nvec;
    if constexpr (KIND == 1) {
        lo = split * a.split_len;
        hi = min(a.nvec, lo + a.split_len);
    }
    const uint32_t out_bytes = (uint32_t)(hi - lo) * OUT_VB;
    char* const yrow = a.y + row * a.y_stride;
    const __amdgpu_buffer_rsrc_t yr = buffer_rsrc(yrow + (int64_t)lo * OUT_VB, out_bytes);
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        const int v = first + k * step;
        const bool in_slice = v >= lo && v < hi;
        if (!EARLY && !in_slice)
            continue;
        const uint32_t off = in_slice ? (uint32_t)(v - lo) * OUT_VB : out_bytes;
        float xv[VE], wf[VE];
        E::unpack(d[k], xv);
        if constexpr (EARLY)
            E::unpack(wv[k], wf);
        else
            E::unpack(load16(a.w + (int64_t)v * 16), wf);
        if constexpr (EAGER) {
#pragma unroll
            for (int e = 0; e < VE; ++e)
                xv[e] = xv[e] * rrms;
            E::round_trip(xv);
#pragma unroll
            for (int e = 0; e < VE; ++e)
                xv[e] = xv[e] * wf[e];
        } else {
#pragma unroll
            for (int e = 0; e < VE; ++e)
                xv[e] = xv[e] * rrms * wf[e];
        }
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
            if constexpr (EARLY) {
                if constexpr (VE == 8)
                    buffer_store8<NT>(c[0], c[1], yr, off);
                else
                    buffer_store4<NT>(c[0], yr, off);
            } else {
                char* const dst = yrow + (int64_t)v * VE;
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
            }
        } else {
            if constexpr (EARLY)
                buffer_store16<NT>(E::pack(xv), yr, off);
            else
                store_row16<NT>(yrow + (int64_t)v * 16, E::pack(xv));
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
// ViT cos/sin planes ([ViT] setup kernel): one thread per (token, group of 4
// columns).  Column c belongs to axis a (t, h, w contiguous); plane a receives
// cos/sin(fl32(pos_a) * inv_a[c - off_a]) at [a][token][c].  A group whose
// four columns lie in one plane leaves as one 16-byte store per plane when
// the host allows it (aligned planes, sections of whole groups); otherwise
// column by column.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void vit_setup_kernel(const VitArgs a)
{
    // Threads past the last group compute the last one again and store
    // nothing: no early exit, so no branch splits the kernel-argument reads.
    const uint32_t groups = a.div_groups.d;
    const uint32_t total = (uint32_t)a.tok_count * groups;
    const uint32_t idx_raw = blockIdx.x * kThreads + threadIdx.x;
    const bool live = idx_raw < total;
    const uint32_t idx = live ? idx_raw : total - 1;
    const uint32_t tl = fast_div(idx, a.div_groups);
    const int32_t c0 = 4 * (int32_t)(idx - tl * groups);
    const uint32_t tok = (uint32_t)a.tok_begin + tl;
    int32_t pos[3];
    vit_position(a, tok, &pos[0], &pos[1], &pos[2]);
    float cv[4], sv[4], iv[4];
    int axis[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int32_t col = c0 + e < a.half_rot ? c0 + e : a.half_rot - 1;
        const int ax = col < a.off[1] ? 0 : (col < a.off[2] ? 1 : 2);
        const float* inv = ax == 0 ? a.inv[0] : (ax == 1 ? a.inv[1] : a.inv[2]);
        const int32_t off = ax == 0 ? a.off[0] : (ax == 1 ? a.off[1] : a.off[2]);
        iv[e] = inv[col - off];
        axis[e] = ax;
    }
    // The four inverse frequencies are in hand before the first sincosf:
    // one wait for the four loads, where the compiler would otherwise place
    // each load (and a wait for it) just before its sincosf.
    asm("" : "+v"(iv[0]), "+v"(iv[1]), "+v"(iv[2]), "+v"(iv[3]));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int ax = axis[e];
        const int32_t p = ax == 0 ? pos[0] : (ax == 1 ? pos[1] : pos[2]);
        sincosf((float)p * iv[e], &sv[e], &cv[e]);
    }
    if (!live)
        return;
    const int64_t row = ((int64_t)axis[0] * a.n_tokens + tok) * a.half_rot + c0;
    if (a.vec_ok) {
        // groups never straddle a section and rows are whole groups
        *reinterpret_cast<float4*>(a.cos_out + row) = make_float4(cv[0], cv[1], cv[2], cv[3]);
        *reinterpret_cast<float4*>(a.sin_out + row) = make_float4(sv[0], sv[1], sv[2], sv[3]);
        return;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if (c0 + e >= a.half_rot)
            break;
        const int64_t o = ((int64_t)axis[e] * a.n_tokens + tok) * a.half_rot + c0 + e;
        a.cos_out[o] = cv[e];
        a.sin_out[o] = sv[e];
    }
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
    vit_position(a, (uint32_t)tok, &t, &h, &w);
    out[tok] = t;
    out[a.n_tokens + tok] = h;
    out[2 * a.n_tokens + tok] = w;
}

// ---------------------------------------------------------------------------
// Dispatch tables
// ---------------------------------------------------------------------------
using RmsFn = void (*)(RmsArgs);

template <class E, int KIND, bool NT, int MODE, bool EAGER>
RmsFn pick_vpl(int vpl)
{
    switch (vpl) {
    case 1: return rms_kernel<E, 1, KIND, NT, MODE, EAGER>;
    case 2: return rms_kernel<E, 2, KIND, NT, MODE, EAGER>;
    case 3: return rms_kernel<E, 3, KIND, NT, MODE, EAGER>;
    case 4: return rms_kernel<E, 4, KIND, NT, MODE, EAGER>;
    case 5: return rms_kernel<E, 5, KIND, NT, MODE, EAGER>;
    case 6: return rms_kernel<E, 6, KIND, NT, MODE, EAGER>;
    case 8: return rms_kernel<E, 8, KIND, NT, MODE, EAGER>;
    case 10: return rms_kernel<E, 10, KIND, NT, MODE, EAGER>;
    case 12: return rms_kernel<E, 12, KIND, NT, MODE, EAGER>;
    default: return rms_kernel<E, 16, KIND, NT, MODE, EAGER>;
    }
}

// Every mode comes with and without nontemporal accesses; the add modes skip
// the split variant (its workgroups read the whole row while others write
// the residual); the eager numerics exist for activation-type outputs.
template <class E, int KIND, bool NT, bool EAGER>
RmsFn pick_rms_nt(int mode, int vpl)
{
    if (mode == 0)
        return pick_vpl<E, KIND, NT, 0, EAGER>(vpl);
    if constexpr (KIND != 1) {
        if (mode == 1)
            return pick_vpl<E, KIND, NT, 1, EAGER>(vpl);
    }
    if constexpr (!EAGER) {
        if (mode == 2)
            return pick_vpl<E, KIND, NT, 2, false>(vpl);
        if constexpr (KIND != 1) {
            if (mode == 3)
                return pick_vpl<E, KIND, NT, 3, false>(vpl);
        }
    }
    return nullptr;
}

template <class E, int KIND>
RmsFn pick_rms_mode(bool nt, bool eager, int mode, int vpl)
{
    if (eager)
        return nt ? pick_rms_nt<E, KIND, true, true>(mode, vpl) : pick_rms_nt<E, KIND, false, true>(mode, vpl);
    return nt ? pick_rms_nt<E, KIND, true, false>(mode, vpl) : pick_rms_nt<E, KIND, false, false>(mode, vpl);
}

thread_local char g_variant[96];

}  // namespace

// LDS a workgroup of the tile kernel reserves so that a compute unit (160 KB
// of LDS) holds at most `cap` of them, i.e. `cap` waves per SIMD (one wave
// of each workgroup per SIMD): the dynamic part beyond the kernel's own LDS.
// Only seven is used: 22 KB per workgroup fits seven (23.4 KB each) and not
// eight (20 KB each) for every allocation granularity up to 2 KB.
static hipError_t cap_lds(NormRopeFn fn, int cap, uint32_t* dynamic)
{
    *dynamic = 0;
    if (cap <= 0)
        return hipSuccess;
    if (cap != 7)
        return hipErrorInvalidValue;
    // The kernel's own LDS, queried once per kernel.
    static std::mutex mu;
    static std::unordered_map<const void*, size_t> own;
    size_t fixed;
    {
        std::lock_guard<std::mutex> lock(mu);
        auto it = own.find(reinterpret_cast<const void*>(fn));
        if (it == own.end()) {
            hipFuncAttributes attr;
            const hipError_t e = hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(fn));
            if (e != hipSuccess)
                return e;
            it = own.emplace(reinterpret_cast<const void*>(fn), attr.sharedSizeBytes).first;
        }
        fixed = it->second;
    }
    constexpr size_t kCap7 = 22 * 1024;
    *dynamic = fixed < kCap7 ? (uint32_t)(kCap7 - fixed) : 0;
    return hipSuccess;
}

// One launch per kMaxBlocksPerLaunch workgroups of kWaves tiles, each told
// its first tile.
static hipError_t launch_tiles(NormRopeFn fn, NormRopeArgs& a, int64_t tiles, hipStream_t stream,
                               uint32_t lds_dynamic = 0)
{
    const int64_t blocks = (tiles + kWaves - 1) / kWaves;
    for (int64_t b0 = 0; b0 < blocks; b0 += kMaxBlocksPerLaunch) {
        const int64_t nb = blocks - b0 < kMaxBlocksPerLaunch ? blocks - b0 : kMaxBlocksPerLaunch;
        a.tile_base = (uint32_t)(b0 * kWaves);
        hipLaunchKernelGGL(fn, dim3((uint32_t)nb), dim3(kThreads), lds_dynamic, stream, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

static const char* rope_name(int rope)
{
    return rope == 0 ? "none" : (rope == 1 ? "pos" : (rope == 2 ? "planes" : "vit"));
}

// The token-tile kernel: one tile per (batch, token).
static hipError_t launch_norm_rope_token(NormRopeArgs a, int32_t dtype, int32_t pairing, bool eager, const RopePlan& plan,
                                  int rope, hipStream_t stream, const char** variant)
{
    const int ve = dtype == kBF16 ? 8 : 4;
    const int nv = a.head_dim / ve;
    const int64_t tiles = (int64_t)a.batch * a.tokens;
    if (tiles == 0)
        return hipSuccess;
    if (tiles >= ((int64_t)1 << 31))
        return hipErrorInvalidValue;   // the host layer refuses such calls first
    a.ntiles = (uint32_t)tiles;
    a.div_tokens = make_fastdiv((uint32_t)a.tokens);
    a.nv_recip = (65536u + (uint32_t)nv - 1) / (uint32_t)nv;
    NormRopeFn fn;
    switch (plan.token) {
    case 3: fn = eager ? pick_norm_rope_token<3, true>(dtype, rope, pairing, plan.nt)
                       : pick_norm_rope_token<3, false>(dtype, rope, pairing, plan.nt); break;
    case 5: fn = eager ? pick_norm_rope_token<5, true>(dtype, rope, pairing, plan.nt)
                       : pick_norm_rope_token<5, false>(dtype, rope, pairing, plan.nt); break;
    case 6: fn = eager ? pick_norm_rope_token<6, true>(dtype, rope, pairing, plan.nt)
                       : pick_norm_rope_token<6, false>(dtype, rope, pairing, plan.nt); break;
    default: fn = eager ? pick_norm_rope_token<7, true>(dtype, rope, pairing, plan.nt)
                        : pick_norm_rope_token<7, false>(dtype, rope, pairing, plan.nt); break;
    }
    const hipError_t e = launch_tiles(fn, a, tiles, stream);
    if (e != hipSuccess)
        return e;
    snprintf(g_variant, sizeof(g_variant), "rope:token:nt%d:lanes%d:%s:%s:%s%s", (int)plan.nt, plan.token,
             dtype == kBF16 ? "bf16" : "f32", rope_name(rope), pairing == kNeox ? "neox" : "adjacent",
             eager ? ":eager" : "");
    *variant = g_variant;
    return hipSuccess;
}

hipError_t launch_norm_rope(const NormRopeArgs& a_in, int32_t dtype, int32_t pairing, bool eager, const RopePlan& plan,
                            hipStream_t stream, const char** variant)
{
    NormRopeArgs a = a_in;
    const int ve = dtype == kBF16 ? 8 : 4;
    const int nv = a.head_dim / ve;
    const int lpr = plan.lpr, np = plan.np;
    const int rope = a.rope.mode == kPosNone ? 0
                     : (a.rope.mode == kPosPlanes ? 2 : (a.rope.mode == kPosVit ? 3 : 1));
    if (plan.token > 0)
        return launch_norm_rope_token(a, dtype, pairing, eager, plan, rope, stream, variant);
    const int rpw = (64 / lpr) * np;
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
    a.nv_recip = (65536u + (uint32_t)nv - 1) / (uint32_t)nv;
    NormRopeFn fn;
    switch (lpr) {
    case 1: fn = eager ? pick_norm_rope<1, true>(dtype, rope, pairing, plan.nt, plan.stage, np)
                       : pick_norm_rope<1, false>(dtype, rope, pairing, plan.nt, plan.stage, np); break;
    case 2: fn = eager ? pick_norm_rope<2, true>(dtype, rope, pairing, plan.nt, plan.stage, np)
                       : pick_norm_rope<2, false>(dtype, rope, pairing, plan.nt, plan.stage, np); break;
    case 4: fn = eager ? pick_norm_rope<4, true>(dtype, rope, pairing, plan.nt, plan.stage, np)
                       : pick_norm_rope<4, false>(dtype, rope, pairing, plan.nt, plan.stage, np); break;
    case 8: fn = eager ? pick_norm_rope<8, true>(dtype, rope, pairing, plan.nt, plan.stage, np)
                       : pick_norm_rope<8, false>(dtype, rope, pairing, plan.nt, plan.stage, np); break;
    case 16: fn = eager ? pick_norm_rope<16, true>(dtype, rope, pairing, plan.nt, plan.stage, np)
                        : pick_norm_rope<16, false>(dtype, rope, pairing, plan.nt, plan.stage, np); break;
    default: fn = eager ? pick_norm_rope<32, true>(dtype, rope, pairing, plan.nt, plan.stage, np)
                        : pick_norm_rope<32, false>(dtype, rope, pairing, plan.nt, plan.stage, np); break;
    }
    uint32_t lds_dynamic = 0;
    hipError_t e = cap_lds(fn, plan.waves_cap, &lds_dynamic);
    if (e != hipSuccess)
        return e;
    e = launch_tiles(fn, a, tiles, stream, lds_dynamic);
    if (e != hipSuccess)
        return e;
    snprintf(g_variant, sizeof(g_variant), "rope:np%d:nt%d:lpr%d:%s:%s:%s:stage%d%s%s", np, (int)plan.nt, lpr,
             dtype == kBF16 ? "bf16" : "f32", rope_name(rope), pairing == kNeox ? "neox" : "adjacent",
             (int)plan.stage, plan.waves_cap > 0 ? ":w7" : "", eager ? ":eager" : "");
    *variant = g_variant;
    return hipSuccess;
}

hipError_t launch_rms_norm(RmsArgs a, int32_t dtype, bool eager, const RmsPlan& plan, hipStream_t stream,
                           const char** variant)
{
    if (a.rows == 0)
        return hipSuccess;
    const int kind = plan.kind, vpl = plan.vpl, mode = plan.mode;
    int64_t items, per_block;   // work items (rows, or row slices) and items per workgroup
    if (kind == 0) {
        items = a.rows;
        per_block = kWaves;
    } else if (kind == 1) {
        // one slice of 64 vectors per wave (each lane stores one vector)
        a.split_len = 64;
        a.splits = (a.nvec + a.split_len - 1) / a.split_len;
        a.div_splits = make_fastdiv((uint32_t)a.splits);
        items = a.rows * a.splits;
        per_block = kWaves;
    } else {
        items = a.rows;
        per_block = 1;
    }
    RmsFn fn;
    if (dtype == kBF16)
        fn = kind == 0 ? pick_rms_mode<BF16, 0>(plan.nt, eager, mode, vpl)
                       : (kind == 1 ? pick_rms_mode<BF16, 1>(plan.nt, eager, mode, vpl)
                                    : pick_rms_mode<BF16, 2>(plan.nt, eager, mode, vpl));
    else
        fn = kind == 0 ? pick_rms_mode<F32, 0>(plan.nt, eager, mode, vpl)
                       : (kind == 1 ? pick_rms_mode<F32, 1>(plan.nt, eager, mode, vpl)
                                    : pick_rms_mode<F32, 2>(plan.nt, eager, mode, vpl));
    if (fn == nullptr)
        return hipErrorInvalidValue;   // plan_rms_norm refuses such calls first
    const int64_t blocks = (items + per_block - 1) / per_block;
    for (int64_t b0 = 0; b0 < blocks; b0 += kMaxBlocksPerLaunch) {
        const int64_t nb = blocks - b0 < kMaxBlocksPerLaunch ? blocks - b0 : kMaxBlocksPerLaunch;
        a.item_base = b0 * per_block;
        hipLaunchKernelGGL(fn, dim3((uint32_t)nb), dim3(kThreads), 0, stream, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    snprintf(g_variant, sizeof(g_variant), "rms:%s:nt%d:vpl%d:%s%s%s%s",
             kind == 0 ? "rows" : (kind == 1 ? "split" : "wide"), (int)plan.nt, vpl, dtype == kBF16 ? "bf16" : "f32",
             (mode & 1) ? ":add" : "", (mode & 2) ? ":fp8" : "", eager ? ":eager" : "");
    *variant = g_variant;
    return hipSuccess;
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
    const int64_t n = a.tok_count * (int64_t)a.div_groups.d;
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
