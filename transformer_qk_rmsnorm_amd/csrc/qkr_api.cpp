// C-ABI entry points of libqkrope: argument validation (pure host code, run
// before any HIP call), translation of element strides into the byte strides
// the kernels take, variant choice and launch on the caller's stream.
//
// Page names used in comments:
//   [Ovis]   vllm-omni pull request "[Kernel][Ovis-Image] Fuse text/image QK
//            RMSNorm + cat + RoPE into one Triton launch"
//   [IMROPE] llama.cpp fork pull request "hrx: the multi-section rotation of
//            Qwen3-VL runs on the device, not on the CPU"
//   [ViT]    vLLM API page "vllm.model_executor.layers.rotary_embedding.
//            mrope_vit_setup"
#include "qkrope.h"

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <climits>
#include <cstring>
#include <initializer_list>
#include <utility>
#include <vector>

#include "qkr_internal.hpp"

namespace {

using namespace qkr;

thread_local char g_error[512] = "";
thread_local char g_variant[96] = "";

// Test hook: forced variants (-1 / 0 = automatic).
std::atomic<int> g_rms_kind{-1};
std::atomic<int> g_rope_np{0};
std::atomic<int> g_nt{1};
std::atomic<int> g_rope_lpr{0};
std::atomic<int> g_rope_stage{-1};
std::atomic<int> g_rope_token{-1};

qkr_status fail(qkr_status st, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_error, sizeof(g_error), fmt, ap);
    va_end(ap);
    return st;
}

qkr_status ok()
{
    g_error[0] = '\0';
    return QKR_OK;
}

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) & (n - 1)) == 0; }

// Size arithmetic on caller-supplied counts.  Every byte offset into a real
// device buffer fits the GPU's 48-bit virtual address space, so strides and
// spans are held to it; then no offset that the host or a kernel forms
// (index * stride, summed over the dimensions) can leave 64 bits.  Rows,
// tiles and tokens of one launch stay below 2^31 (32-bit tile indices).
constexpr int64_t kAddrBytes = (int64_t)1 << 48;
constexpr int64_t kMaxRows = (int64_t)1 << 31;

// a * b for a, b >= 0, or -1 when the product exceeds `limit`; never overflows.
int64_t mul_capped(int64_t a, int64_t b, int64_t limit)
{
    if (a == 0 || b == 0)
        return 0;
    return a > limit / b ? -1 : a * b;
}

// Whether the product of non-negative factors is below `limit`.
bool product_below(std::initializer_list<int64_t> factors, int64_t limit)
{
    for (const int64_t f : factors)
        if (f == 0)
            return true;
    int64_t p = 1;
    for (const int64_t f : factors)
        if ((p = mul_capped(p, f, limit - 1)) < 0)
            return false;
    return true;
}

qkr_status hip_status(hipError_t e, const char* what)
{
    if (e != hipSuccess)
        return fail(QKR_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

// The dtype argument: QKR_F32 or QKR_BF16, optionally OR-ed with
// QKR_NUMERICS_EAGER.  On return dtype holds the element type alone.
qkr_status check_dtype(int32_t& dtype, int& esize, bool& eager)
{
    const int32_t numerics = dtype & ~(int32_t)0xFF;
    if (numerics != QKR_NUMERICS_CONTRACT && numerics != QKR_NUMERICS_EAGER)
        return fail(QKR_ERR_INVALID_ARGUMENT, "dtype %d carries unknown numerics bits", dtype);
    eager = numerics == QKR_NUMERICS_EAGER;
    dtype &= 0xFF;
    if (dtype == QKR_F32) {
        esize = 4;
        return QKR_OK;
    }
    if (dtype == QKR_BF16) {
        esize = 2;
        return QKR_OK;
    }
    return fail(QKR_ERR_INVALID_ARGUMENT, "dtype %d is neither QKR_F32 nor QKR_BF16", dtype);
}

qkr_status check_eps(float eps)
{
    if (!std::isfinite(eps) || eps < 0.0f)
        return fail(QKR_ERR_INVALID_ARGUMENT, "eps must be finite and >= 0");
    return QKR_OK;
}

// Rows of head_dim elements move as 16-byte vectors.
qkr_status check_head_dim(int32_t head_dim, int esize)
{
    if (head_dim <= 0 || head_dim > 256)
        return fail(QKR_ERR_INVALID_ARGUMENT, "head_dim %d outside [1, 256]", head_dim);
    if ((head_dim * esize) % 16 != 0)
        return fail(QKR_ERR_MISALIGNED, "head_dim %d is not a whole number of 16-byte vectors", head_dim);
    return QKR_OK;
}

// A [batch, tokens, heads, head_dim] view that the kernels will touch.
qkr_status check_view(const char* name, const qkr_view* v, int esize, int32_t batch, int64_t tokens,
                      int32_t heads)
{
    if (batch == 0 || tokens == 0 || heads == 0)
        return QKR_OK;
    if (v == nullptr || v->ptr_dev == nullptr)
        return fail(QKR_ERR_INVALID_ARGUMENT, "%s: null view or pointer", name);
    if (!aligned(v->ptr_dev, 16))
        return fail(QKR_ERR_MISALIGNED, "%s: pointer is not 16-byte aligned", name);
    const int64_t st[3] = {v->stride_batch, v->stride_tok, v->stride_head};
    const int64_t n[3] = {batch, tokens, heads};
    static const char* what[3] = {"stride_batch", "stride_tok", "stride_head"};
    const int64_t lim = kAddrBytes / esize;
    int64_t span = 0;
    for (int i = 0; i < 3; ++i) {
        // Unused strides are still turned into bytes, so they are bounded too.
        if (st[i] > lim || st[i] < -lim)
            return fail(QKR_ERR_UNSUPPORTED, "%s: %s %lld reaches past a 2^48-byte address space", name, what[i],
                        (long long)st[i]);
        if (n[i] <= 1)
            continue;
        if (st[i] < 0)
            return fail(QKR_ERR_INVALID_ARGUMENT, "%s: negative %s", name, what[i]);
        if ((st[i] * esize) % 16 != 0)
            return fail(QKR_ERR_MISALIGNED, "%s: %s %lld is not a multiple of 16 bytes", name, what[i],
                        (long long)st[i]);
        const int64_t reach = mul_capped(n[i] - 1, st[i] * esize, kAddrBytes);
        if (reach < 0 || (span += reach) > kAddrBytes)
            return fail(QKR_ERR_UNSUPPORTED, "%s: the view spans more than 2^48 bytes", name);
    }
    return QKR_OK;
}

// `rows` rows spaced `stride` elements of `es` bytes (0 <= stride, checked
// before): the row set spans at most the address space.
qkr_status check_row_span(const char* name, int64_t rows, int64_t stride, int64_t es)
{
    if (rows > 1 && (stride > kAddrBytes / es || mul_capped(rows - 1, stride * es, kAddrBytes) < 0))
        return fail(QKR_ERR_UNSUPPORTED, "%s: %lld rows %lld elements apart span more than 2^48 bytes", name,
                    (long long)rows, (long long)stride);
    return QKR_OK;
}

qkr_status check_weight(const char* name, const void* w)
{
    if (w == nullptr)
        return fail(QKR_ERR_INVALID_ARGUMENT, "%s: null weight", name);
    if (!aligned(w, 16))
        return fail(QKR_ERR_MISALIGNED, "%s: weight is not 16-byte aligned", name);
    return QKR_OK;
}

// The one predicate for the rotation: what it refuses is exactly what no
// kernel variant takes, and what it accepts fixes the variant ([IMROPE]: the
// claim and the matcher share one predicate).  `tokens` is the number of
// tokens the call indexes positions with.
qkr_status check_rope(const qkr_rope* r, int32_t head_dim, int esize, int64_t tokens, RopeArgs& out,
                      int32_t& pairing, int32_t& rotary_dim)
{
    std::memset(&out, 0, sizeof(out));
    out.mode = kPosNone;
    pairing = kNeox;
    rotary_dim = 0;
    if (r == nullptr || r->rotary_dim == 0)
        return QKR_OK;
    const int32_t R = r->rotary_dim;
    if (R < 0 || R % 2 != 0 || R > head_dim)
        return fail(QKR_ERR_INVALID_ARGUMENT, "rotary_dim %d must be even and in [0, head_dim=%d]", R, head_dim);
    if (r->pairing != QKR_PAIR_NEOX && r->pairing != QKR_PAIR_ADJACENT)
        return fail(QKR_ERR_INVALID_ARGUMENT, "unknown pairing %d", r->pairing);
    if (r->mode < QKR_POS_1D || r->mode > QKR_POS_PLANES)
        return fail(QKR_ERR_INVALID_ARGUMENT, "unknown position mode %d", r->mode);
    const int ve = 16 / esize;
    if (r->pairing == QKR_PAIR_NEOX && (R / 2) % ve != 0)
        return fail(QKR_ERR_UNSUPPORTED,
                    "NeoX pairing needs rotary_dim/2 (%d) to be a multiple of %d elements (whole 16-byte "
                    "vectors per half)", R / 2, ve);
    if (r->token_base < 0)
        return fail(QKR_ERR_INVALID_ARGUMENT, "token_base %lld < 0", (long long)r->token_base);
    const int32_t* s = r->sections;
    const int32_t half = R / 2;
    if (r->mode == QKR_POS_AXES || r->mode == QKR_POS_PLANES) {
        if (s[0] < 0 || s[1] < 0 || s[2] < 0 || s[3] != 0 || (int64_t)s[0] + s[1] + s[2] != half)
            return fail(QKR_ERR_INVALID_ARGUMENT,
                        "axis sections (%d, %d, %d, %d) must be >= 0, end with 0 and sum to rotary_dim/2 = %d",
                        s[0], s[1], s[2], s[3], half);
    }
    if (r->mode == QKR_POS_IMROPE) {
        // [IMROPE] follow-up commit: claim only n_dims/2 <= sum <= n_dims, and
        // refuse a sectioned rotation without sections rather than default.
        const int64_t sum = (int64_t)s[0] + s[1] + s[2] + s[3];
        if (s[0] < 0 || s[1] < 0 || s[2] < 0 || s[3] < 0 || sum < half || sum > R)
            return fail(QKR_ERR_INVALID_ARGUMENT,
                        "IMROPE sections (%d, %d, %d, %d) must be >= 0 with rotary_dim/2 <= sum <= rotary_dim",
                        s[0], s[1], s[2], s[3]);
    }
    if (r->mode == QKR_POS_PLANES) {
        if (r->cos_planes_dev == nullptr || r->sin_planes_dev == nullptr)
            return fail(QKR_ERR_INVALID_ARGUMENT, "PLANES mode needs cos and sin planes");
        if (!aligned(r->cos_planes_dev, 4) || !aligned(r->sin_planes_dev, 4))
            return fail(QKR_ERR_MISALIGNED, "cos/sin planes are not 4-byte aligned");
        if (tokens > 0 && (r->planes_tokens < tokens || r->planes_tokens - tokens < r->token_base))
            return fail(QKR_ERR_INVALID_ARGUMENT, "planes hold %lld tokens, the call reads %lld from token %lld",
                        (long long)r->planes_tokens, (long long)tokens, (long long)r->token_base);
        // Three planes of planes_tokens x rotary_dim/2 floats.
        if (!product_below({r->planes_tokens, 3, half, 4}, kAddrBytes + 1))
            return fail(QKR_ERR_UNSUPPORTED, "cos/sin planes of %lld tokens span more than 2^48 bytes",
                        (long long)r->planes_tokens);
    } else {
        if (r->inv_freq_dev == nullptr || r->positions_dev == nullptr)
            return fail(QKR_ERR_INVALID_ARGUMENT, "position mode %d needs inv_freq and positions", r->mode);
        if (!aligned(r->inv_freq_dev, 4) || !aligned(r->positions_dev, 4))
            return fail(QKR_ERR_MISALIGNED, "inv_freq/positions are not 4-byte aligned");
        if (tokens > 0 && (r->pos_stride < tokens || r->pos_stride - tokens < r->token_base))
            return fail(QKR_ERR_INVALID_ARGUMENT,
                        "position planes hold %lld tokens (pos_stride), the call reads %lld from token %lld",
                        (long long)r->pos_stride, (long long)tokens, (long long)r->token_base);
        // Up to four planes of pos_stride int32 positions.
        if (!product_below({r->pos_stride, 4, 4}, kAddrBytes + 1))
            return fail(QKR_ERR_UNSUPPORTED, "position planes of stride %lld span more than 2^48 bytes",
                        (long long)r->pos_stride);
    }
    out.mode = r->mode;
    out.half = half;
    for (int i = 0; i < 4; ++i)
        out.sec[i] = s[i];
    out.inv_freq = r->inv_freq_dev;
    out.positions = r->positions_dev;
    out.pos_stride = r->pos_stride;
    // Position planes the mode reads (t; t, h, w; t, h, w, e); the others
    // alias plane t and are never used.
    const int planes = r->mode == QKR_POS_IMROPE ? 4 : (r->mode == QKR_POS_AXES ? 3 : 1);
    for (int i = 0; i < 4; ++i)
        out.plane_off[i] = r->mode == QKR_POS_PLANES || i >= planes ? 0 : (int64_t)i * r->pos_stride;
    build_axis_bits(r->mode, s, half, out.axis_bits);
    out.token_base = r->token_base;
    out.cos_planes = r->cos_planes_dev;
    out.sin_planes = r->sin_planes_dev;
    out.planes_tokens = r->planes_tokens;
    pairing = r->pairing;
    rotary_dim = R;
    return QKR_OK;
}

void fill_in(TensorArgs& t, int s, const qkr_view* v, int esize)
{
    t.s[s].in = v ? static_cast<const char*>(v->ptr_dev) : nullptr;
    t.s[s].sb = v ? v->stride_batch * esize : 0;
    t.s[s].st = v ? v->stride_tok * esize : 0;
    t.s[s].sh = v ? v->stride_head * esize : 0;
}

void fill_out(TensorArgs& t, const qkr_view* v, int esize)
{
    t.out = v ? static_cast<char*>(v->ptr_dev) : nullptr;
    t.out_sb = v ? v->stride_batch * esize : 0;
    t.out_st = v ? v->stride_tok * esize : 0;
    t.out_sh = v ? v->stride_head * esize : 0;
}

// The kernel variant of a QK call (pure host code): a forced variant that
// cannot run the call is refused, never replaced.
qkr_status plan_rope(const NormRopeArgs& a, int32_t dtype, RopePlan& plan)
{
    const int32_t heads[3] = {a.t[0].heads, a.t[1].heads, a.t[2].heads};
    // Token tiles take Q and K of one stream with no slot map, and address a
    // tensor's rows of one token with 32-bit offsets.
    bool token_ok = a.t[2].heads == 0 && a.t[0].slots == nullptr && a.t[1].slots == nullptr && a.tokens0 >= a.tokens;
    const int64_t row_bytes = (int64_t)a.head_dim * (dtype == kBF16 ? 2 : 4);
    for (int i = 0; i < 2; ++i) {
        const TensorArgs& t = a.t[i];
        if (t.heads == 0)
            continue;
        for (const int64_t sh : {t.s[0].sh, t.out_sh})
            token_ok = token_ok && sh >= 0 && (int64_t)(t.heads - 1) * sh + row_bytes <= INT32_MAX;
    }
    const char* why = plan_norm_rope(dtype, a.head_dim, heads, a.rope.mode == kPosNone ? 0 : a.rope.half,
                                     a.rope.mode == kPosPlanes, token_ok, g_rope_np.load(), g_rope_lpr.load(), g_rope_stage.load(),
                                     g_rope_token.load(), g_nt.load(), &plan);
    if (why != nullptr)
        return fail(QKR_ERR_UNSUPPORTED, "forced variant: %s", why);
    return QKR_OK;
}

qkr_status launch_planned(NormRopeArgs& a, int32_t dtype, bool eager, int32_t pairing, const RopePlan& plan,
                          hipStream_t stream)
{
    (void)hipGetLastError();   // clear a stale error so the launch reports its own
    const char* variant = "";
    hipError_t e = launch_norm_rope(a, dtype, pairing, eager, plan, stream, &variant);
    if (e != hipSuccess)
        return fail(QKR_ERR_HIP, "norm_rope launch: %s", hipGetErrorString(e));
    std::snprintf(g_variant, sizeof(g_variant), "%s", variant);
    return ok();
}

qkr_status launch(NormRopeArgs& a, int32_t dtype, bool eager, int32_t pairing, hipStream_t stream)
{
    RopePlan plan;
    qkr_status st;
    if ((st = plan_rope(a, dtype, plan)))
        return st;
    return launch_planned(a, dtype, eager, pairing, plan, stream);
}

// The row kernel variant (pure host code), as plan_rope.
qkr_status plan_rows(int64_t nvec, int64_t rows, int mode, RmsPlan& plan)
{
    const char* why = plan_rms_norm((int32_t)nvec, rows, g_rms_kind.load(), g_nt.load(), mode, &plan);
    if (why != nullptr)
        return fail(QKR_ERR_UNSUPPORTED, "forced variant: %s", why);
    return QKR_OK;
}

// Mode and sections of the axis-map entries, which take sections on their
// own (no rotary_dim bounds them): each in [0, 2^20], so the sector rule's
// sums and 3 x section products stay in 32 bits, and a positive sum for
// IMROPE.
qkr_status check_map_rope(const qkr_rope* rope)
{
    if (rope->mode < QKR_POS_1D || rope->mode > QKR_POS_PLANES)
        return fail(QKR_ERR_INVALID_ARGUMENT, "unknown position mode %d", rope->mode);
    const int32_t* s = rope->sections;
    for (int i = 0; i < 4; ++i)
        if (s[i] < 0 || s[i] > (1 << 20))
            return fail(QKR_ERR_INVALID_ARGUMENT, "section %d = %d outside [0, 2^20]", i, s[i]);
    if (rope->mode == QKR_POS_IMROPE && s[0] + s[1] + s[2] + s[3] <= 0)
        return fail(QKR_ERR_INVALID_ARGUMENT, "IMROPE needs a positive section sum");
    return QKR_OK;
}

// Shared set-up of the ViT grid table; validates and returns the total.
qkr_status check_grids(const int32_t* grid_thw, int32_t num_grids, int32_t merge, int64_t& total)
{
    if (grid_thw == nullptr || num_grids <= 0)
        return fail(QKR_ERR_INVALID_ARGUMENT, "grid_thw must hold at least one grid");
    if (merge <= 0)
        return fail(QKR_ERR_INVALID_ARGUMENT, "spatial_merge %d must be >= 1", merge);
    total = 0;
    for (int32_t g = 0; g < num_grids; ++g) {
        const int32_t t = grid_thw[3 * g], h = grid_thw[3 * g + 1], w = grid_thw[3 * g + 2];
        if (t <= 0 || h <= 0 || w <= 0)
            return fail(QKR_ERR_INVALID_ARGUMENT, "grid %d (%d, %d, %d) must have t, h, w >= 1", g, t, h, w);
        if (h % merge != 0 || w % merge != 0)
            return fail(QKR_ERR_INVALID_ARGUMENT, "grid %d: h %d and w %d must be multiples of spatial_merge %d",
                        g, h, w, merge);
        // t * h * w < 2^31 each (t * h <= 2^62 cannot overflow), and so is the sum.
        const int64_t th = (int64_t)t * h;
        if (th >= kMaxRows || !product_below({th, w}, kMaxRows - total))
            return fail(QKR_ERR_UNSUPPORTED, "grids hold 2^31 tokens or more (grid %d)", g);
        total += th * w;
    }
    return QKR_OK;
}

// Grid groups of at most kMaxGrids per launch; token offsets stay absolute
// (every total stays below 2^31: check_grids).
template <class F>
hipError_t for_grid_groups(const int32_t* grid_thw, int32_t num_grids, int32_t merge, VitArgs base, F&& fn)
{
    int64_t start = 0;
    for (int32_t g0 = 0; g0 < num_grids; g0 += kMaxGrids) {
        const int32_t n = num_grids - g0 < kMaxGrids ? num_grids - g0 : kMaxGrids;
        VitArgs a = base;
        a.merge = merge;
        a.num_grids = n;
        a.tok_begin = start;
        a.div_m = make_fastdiv((uint32_t)merge);
        a.div_mm = make_fastdiv((uint32_t)(merge * merge));
        int64_t cu = start;
        for (int32_t k = 0; k < n; ++k) {
            const int32_t* g = grid_thw + 3 * (g0 + k);
            a.cu[k] = (uint32_t)cu;
            a.div_area[k] = make_fastdiv((uint32_t)((int64_t)g[1] * g[2]));
            a.div_bcols[k] = make_fastdiv((uint32_t)(g[2] / merge));
            cu += (int64_t)g[0] * g[1] * g[2];
        }
        a.cu[n] = (uint32_t)cu;
        a.tok_count = cu - start;
        const hipError_t e = fn(a);
        if (e != hipSuccess)
            return e;
        start = cu;
    }
    return hipSuccess;
}

}  // namespace

extern "C" {

const char* qkr_status_string(qkr_status status)
{
    switch (status) {
    case QKR_OK: return "QKR_OK";
    case QKR_ERR_INVALID_ARGUMENT: return "QKR_ERR_INVALID_ARGUMENT";
    case QKR_ERR_UNSUPPORTED: return "QKR_ERR_UNSUPPORTED";
    case QKR_ERR_MISALIGNED: return "QKR_ERR_MISALIGNED";
    case QKR_ERR_HIP: return "QKR_ERR_HIP";
    }
    return "unknown qkr_status";
}

const char* qkr_last_error(void) { return g_error; }

const char* qkr_debug_last_variant(void) { return g_variant; }

const char* qkr_last_variant(void) { return g_variant; }

qkr_status qkr_set_variant_override(const char* name)
{
    if (name == nullptr) {
        g_rms_kind = -1;
        g_rope_np = 0;
        g_rope_lpr = 0;
        g_rope_stage = -1;
        g_rope_token = -1;
        g_nt = 1;
        return ok();
    }
    if (std::strcmp(name, "rope:tile") == 0 || std::strcmp(name, "rope:token") == 0) {
        g_rope_token = name[6] == 'o' ? 1 : 0;
        return ok();
    }
    if (std::strcmp(name, "nt:0") == 0 || std::strcmp(name, "nt:1") == 0) {
        g_nt = name[3] - '0';
        return ok();
    }
    static const char* rms[3] = {"rms:rows", "rms:split", "rms:wide"};
    for (int i = 0; i < 3; ++i)
        if (std::strcmp(name, rms[i]) == 0) {
            g_rms_kind = i;
            return ok();
        }
    static const char* np[4] = {"rope:np1", "rope:np2", "rope:np3", "rope:np4"};
    for (int i = 0; i < 4; ++i)
        if (std::strcmp(name, np[i]) == 0) {
            g_rope_np = i + 1;
            return ok();
        }
    if (std::strcmp(name, "rope:stage0") == 0 || std::strcmp(name, "rope:stage1") == 0) {
        g_rope_stage = name[10] - '0';
        return ok();
    }
    static const char* lpr[4] = {"rope:lpr4", "rope:lpr8", "rope:lpr16", "rope:lpr32"};
    static const int lpr_val[4] = {4, 8, 16, 32};
    for (int i = 0; i < 4; ++i)
        if (std::strcmp(name, lpr[i]) == 0) {
            g_rope_lpr = lpr_val[i];
            return ok();
        }
    return fail(QKR_ERR_INVALID_ARGUMENT, "unknown variant '%s'", name);
}

qkr_status qkr_rms_norm(const void* x_dev, int64_t x_row_stride, void* y_dev, int64_t y_row_stride,
                        const void* weight_dev, int64_t rows, int32_t width, float eps, int32_t dtype,
                        qkr_stream_t stream)
{
    int esize = 0;
    bool eager = false;
    qkr_status st;
    if ((st = check_dtype(dtype, esize, eager)) || (st = check_eps(eps)))
        return st;
    if (rows < 0)
        return fail(QKR_ERR_INVALID_ARGUMENT, "rows %lld < 0", (long long)rows);
    if (width <= 0)
        return fail(QKR_ERR_INVALID_ARGUMENT, "width %d must be > 0", width);
    if (((int64_t)width * esize) % 16 != 0)
        return fail(QKR_ERR_MISALIGNED, "width %d is not a whole number of 16-byte vectors", width);
    const int64_t nvec = (int64_t)width * esize / 16;
    if (nvec > 16 * kThreads)
        return fail(QKR_ERR_UNSUPPORTED, "width %d exceeds %d elements", width, 16 * kThreads * 16 / esize);
    if (rows == 0)
        return ok();
    if (!product_below({rows, (nvec + 63) / 64}, kMaxRows))
        return fail(QKR_ERR_UNSUPPORTED, "rows %lld exceed the launch grid", (long long)rows);
    if (x_dev == nullptr || y_dev == nullptr)
        return fail(QKR_ERR_INVALID_ARGUMENT, "null x or y");
    if ((st = check_weight("weight", weight_dev)))
        return st;
    if (!aligned(x_dev, 16) || !aligned(y_dev, 16))
        return fail(QKR_ERR_MISALIGNED, "x or y is not 16-byte aligned");
    if (rows > 1) {
        if (x_row_stride < width || y_row_stride < width)
            return fail(QKR_ERR_INVALID_ARGUMENT, "row strides must be >= width");
        if ((st = check_row_span("x", rows, x_row_stride, esize)) ||
            (st = check_row_span("y", rows, y_row_stride, esize)))
            return st;
        if ((x_row_stride * esize) % 16 != 0 || (y_row_stride * esize) % 16 != 0)
            return fail(QKR_ERR_MISALIGNED, "row strides are not multiples of 16 bytes");
    }

    RmsArgs a{};
    a.x = static_cast<const char*>(x_dev);
    a.y = static_cast<char*>(y_dev);
    a.w = static_cast<const char*>(weight_dev);
    a.x_stride = x_row_stride * esize;
    a.y_stride = y_row_stride * esize;
    a.rows = rows;
    a.nvec = (int32_t)nvec;
    a.eps = eps;
    a.inv_width = 1.0f / (float)width;
    RmsPlan plan;
    if ((st = plan_rows(nvec, rows, 0, plan)))
        return st;
    (void)hipGetLastError();
    const char* variant = "";
    hipError_t e = launch_rms_norm(a, dtype, eager, plan, reinterpret_cast<hipStream_t>(stream), &variant);
    if (e != hipSuccess)
        return fail(QKR_ERR_HIP, "rms_norm launch: %s", hipGetErrorString(e));
    std::snprintf(g_variant, sizeof(g_variant), "%s", variant);
    return ok();
}

qkr_status qkr_add_rms_norm(const void* x_dev, int64_t x_row_stride, const void* r_dev, int64_t r_row_stride,
                            void* s_dev, int64_t s_row_stride, void* y_dev, int64_t y_row_stride, int32_t y_kind,
                            const float* scale_dev, const void* weight_dev, int64_t rows, int32_t width, float eps,
                            int32_t dtype, qkr_stream_t stream)
{
    int esize = 0;
    bool eager = false;
    qkr_status st;
    if ((st = check_dtype(dtype, esize, eager)) || (st = check_eps(eps)))
        return st;
    if (y_kind != QKR_OUT_ACT && y_kind != QKR_OUT_FP8_E4M3)
        return fail(QKR_ERR_INVALID_ARGUMENT, "unknown output kind %d", y_kind);
    const bool fp8 = y_kind == QKR_OUT_FP8_E4M3;
    const bool add = r_dev != nullptr;
    if (fp8 && eager)
        return fail(QKR_ERR_UNSUPPORTED, "the eager numerics are defined for activation-type outputs, not FP8");
    if (rows < 0)
        return fail(QKR_ERR_INVALID_ARGUMENT, "rows %lld < 0", (long long)rows);
    if (width <= 0)
        return fail(QKR_ERR_INVALID_ARGUMENT, "width %d must be > 0", width);
    if (((int64_t)width * esize) % 16 != 0)
        return fail(QKR_ERR_MISALIGNED, "width %d is not a whole number of 16-byte vectors", width);
    const int64_t nvec = (int64_t)width * esize / 16;
    if (nvec > 16 * kThreads)
        return fail(QKR_ERR_UNSUPPORTED, "width %d exceeds %d elements", width, 16 * kThreads * 16 / esize);
    if (add != (s_dev != nullptr))
        return fail(QKR_ERR_INVALID_ARGUMENT, "the residual and the residual output come together (both or neither)");
    if (fp8 && scale_dev == nullptr)
        return fail(QKR_ERR_INVALID_ARGUMENT, "FP8 output needs a device scale");
    if (rows == 0)
        return ok();
    if (!product_below({rows, (nvec + 63) / 64}, kMaxRows))
        return fail(QKR_ERR_UNSUPPORTED, "rows %lld exceed the launch grid", (long long)rows);
    if (x_dev == nullptr || y_dev == nullptr)
        return fail(QKR_ERR_INVALID_ARGUMENT, "null x or y");
    if ((st = check_weight("weight", weight_dev)))
        return st;
    const int ve = 16 / esize;                     // elements per 16-byte vector = FP8 bytes per store
    const int64_t y_esize = fp8 ? 1 : esize;
    if (!aligned(x_dev, 16) || (add && (!aligned(r_dev, 16) || !aligned(s_dev, 16))))
        return fail(QKR_ERR_MISALIGNED, "x, residual or residual output is not 16-byte aligned");
    if (!aligned(y_dev, fp8 ? ve : 16) || (fp8 && !aligned(scale_dev, 4)))
        return fail(QKR_ERR_MISALIGNED, "y or scale is not aligned");
    if (rows > 1) {
        const int64_t strides[3] = {x_row_stride, add ? r_row_stride : width, add ? s_row_stride : width};
        static const char* names[3] = {"x", "residual", "residual output"};
        for (int i = 0; i < 3; ++i) {
            if (strides[i] < width)
                return fail(QKR_ERR_MISALIGNED, "row strides must be >= width and multiples of 16 bytes");
            if ((st = check_row_span(names[i], rows, strides[i], esize)))
                return st;
            if ((strides[i] * esize) % 16 != 0)
                return fail(QKR_ERR_MISALIGNED, "row strides must be >= width and multiples of 16 bytes");
        }
        if (y_row_stride < width)
            return fail(QKR_ERR_MISALIGNED, "y row stride must be >= width and keep rows aligned");
        if ((st = check_row_span("y", rows, y_row_stride, y_esize)))
            return st;
        if ((y_row_stride * y_esize) % (fp8 ? ve : 16) != 0)
            return fail(QKR_ERR_MISALIGNED, "y row stride must be >= width and keep rows aligned");
    }
    // The residual output may overwrite the residual or x in place (same
    // rows); any other overlap of the outputs with the inputs is refused.
    // Row sets with the same byte stride overlap exactly when their start
    // offsets, taken modulo the stride, are less than a row apart (rows of an
    // interleaved [x | r] buffer do not); otherwise the address spans decide.
    struct Rows {
        const char* base;
        int64_t stride, bytes;   // bytes between rows, bytes per row
    };
    auto rows_of = [&](const void* p, int64_t stride, int64_t es) {
        return Rows{static_cast<const char*>(p), rows > 1 ? stride * es : 0, (int64_t)width * es};
    };
    auto overlap = [&](const Rows& u, const Rows& v) {
        const char* ue = u.base + (rows - 1) * u.stride + u.bytes;
        const char* ve = v.base + (rows - 1) * v.stride + v.bytes;
        if (!(u.base < ve && v.base < ue))
            return false;
        if (rows > 1 && u.stride == v.stride && u.stride >= u.bytes && u.stride >= v.bytes) {
            const int64_t s = u.stride;
            const int64_t d = ((v.base - u.base) % s + s) % s;   // v's rows start d bytes into u's
            return d < u.bytes || s - d < v.bytes;
        }
        return true;
    };
    const Rows rx = rows_of(x_dev, x_row_stride, esize), ry = rows_of(y_dev, y_row_stride, y_esize);
    if (overlap(ry, rx))
        return fail(QKR_ERR_INVALID_ARGUMENT, "y overlaps x");
    if (add) {
        const Rows rr = rows_of(r_dev, r_row_stride, esize), ro = rows_of(s_dev, s_row_stride, esize);
        if (overlap(ry, rr) || overlap(ry, ro))
            return fail(QKR_ERR_INVALID_ARGUMENT, "y overlaps the residual");
        const bool same_r = s_dev == r_dev && s_row_stride == r_row_stride;
        const bool same_x = s_dev == x_dev && s_row_stride == x_row_stride;
        if ((overlap(ro, rr) && !same_r) || (overlap(ro, rx) && !same_x))
            return fail(QKR_ERR_INVALID_ARGUMENT, "the residual output overlaps an input other than in place");
    }

    RmsArgs a{};
    a.x = static_cast<const char*>(x_dev);
    a.y = static_cast<char*>(y_dev);
    a.w = static_cast<const char*>(weight_dev);
    a.r = static_cast<const char*>(r_dev);
    a.s = static_cast<char*>(s_dev);
    a.scale = scale_dev;
    a.x_stride = x_row_stride * esize;
    a.y_stride = y_row_stride * y_esize;
    a.r_stride = add ? r_row_stride * esize : 0;
    a.s_stride = add ? s_row_stride * esize : 0;
    a.rows = rows;
    a.nvec = (int32_t)nvec;
    a.eps = eps;
    a.inv_width = 1.0f / (float)width;
    const int mode = (add ? 1 : 0) | (fp8 ? 2 : 0);
    RmsPlan plan;
    if ((st = plan_rows(nvec, rows, mode, plan)))
        return st;
    (void)hipGetLastError();
    const char* variant = "";
    hipError_t e = launch_rms_norm(a, dtype, eager, plan, reinterpret_cast<hipStream_t>(stream), &variant);
    if (e != hipSuccess)
        return fail(QKR_ERR_HIP, "add_rms_norm launch: %s", hipGetErrorString(e));
    std::snprintf(g_variant, sizeof(g_variant), "%s", variant);
    return ok();
}

qkr_status qkr_debug_fp8_e4m3(const float* x_dev, int64_t n, const float* scale_dev, uint8_t* out_dev,
                              qkr_stream_t stream)
{
    if (n < 0 || (n > 0 && (x_dev == nullptr || out_dev == nullptr)))
        return fail(QKR_ERR_INVALID_ARGUMENT, "debug_fp8_e4m3: null pointers or negative n");
    if (n >= kMaxRows)
        return fail(QKR_ERR_UNSUPPORTED, "debug_fp8_e4m3: n too large");
    (void)hipGetLastError();
    return hip_status(launch_debug_fp8(x_dev, n, scale_dev, out_dev, reinterpret_cast<hipStream_t>(stream)),
                      "debug_fp8_e4m3 launch");
}

qkr_status qkr_qk_norm_rope(int32_t batch, int64_t tokens, int32_t head_dim, int32_t dtype, float eps,
                            const qkr_view* q, const qkr_view* q_out, int32_t q_heads, const void* q_weight_dev,
                            const qkr_view* k, const qkr_view* k_out, int32_t k_heads, const void* k_weight_dev,
                            const qkr_rope* rope, qkr_stream_t stream)
{
    int esize = 0;
    bool eager = false;
    qkr_status st;
    if ((st = check_dtype(dtype, esize, eager)) || (st = check_eps(eps)) || (st = check_head_dim(head_dim, esize)))
        return st;
    if (batch < 0 || tokens < 0 || q_heads < 0 || k_heads < 0)
        return fail(QKR_ERR_INVALID_ARGUMENT, "negative batch, tokens or heads");
    const int64_t heads_total = (int64_t)q_heads + k_heads;
    if (heads_total > (1 << 20))
        return fail(QKR_ERR_UNSUPPORTED, "too many heads");
    if (tokens >= kMaxRows || !product_below({batch, tokens, heads_total}, kMaxRows))
        return fail(QKR_ERR_UNSUPPORTED, "batch * tokens * heads must stay below 2^31 rows per call");
    if ((st = check_view("q", q, esize, batch, tokens, q_heads)) ||
        (st = check_view("q_out", q_out, esize, batch, tokens, q_heads)) ||
        (st = check_view("k", k, esize, batch, tokens, k_heads)) ||
        (st = check_view("k_out", k_out, esize, batch, tokens, k_heads)))
        return st;
    if (q_heads > 0 && (st = check_weight("q_weight", q_weight_dev)))
        return st;
    if (k_heads > 0 && (st = check_weight("k_weight", k_weight_dev)))
        return st;
    NormRopeArgs a{};
    int32_t pairing = 0, rotary_dim = 0;
    if ((st = check_rope(rope, head_dim, esize, tokens, a.rope, pairing, rotary_dim)))
        return st;
    if (batch == 0 || tokens == 0 || q_heads + k_heads == 0)
        return ok();

    fill_in(a.t[0], 0, q_heads ? q : nullptr, esize);
    fill_out(a.t[0], q_heads ? q_out : nullptr, esize);
    a.t[0].s[0].weight = q_heads ? static_cast<const char*>(q_weight_dev) : nullptr;
    a.t[0].heads = q_heads;
    fill_in(a.t[1], 0, k_heads ? k : nullptr, esize);
    fill_out(a.t[1], k_heads ? k_out : nullptr, esize);
    a.t[1].s[0].weight = k_heads ? static_cast<const char*>(k_weight_dev) : nullptr;
    a.t[1].heads = k_heads;
    a.t[2].heads = 0;
    a.batch = batch;
    a.tokens = (int32_t)tokens;
    a.tokens0 = (int32_t)tokens;
    a.head_dim = head_dim;
    a.rotary_dim = rotary_dim;
    a.eps = eps;
    a.inv_d = 1.0f / (float)head_dim;
    return launch(a, dtype, eager, pairing, reinterpret_cast<hipStream_t>(stream));
}

qkr_status qkr_qk_norm_rope_cache(int64_t tokens, int32_t head_dim, int32_t dtype, float eps, const qkr_view* q,
                                  const qkr_view* q_out, int32_t q_heads, const void* q_weight_dev,
                                  const qkr_view* k, const qkr_view* v, int32_t kv_heads, const void* k_weight_dev,
                                  const qkr_view* k_cache, const qkr_view* v_cache,
                                  const int64_t* slot_mapping_dev, int64_t num_slots, const qkr_rope* rope,
                                  qkr_stream_t stream)
{
    int esize = 0;
    bool eager = false;
    qkr_status st;
    if ((st = check_dtype(dtype, esize, eager)) || (st = check_eps(eps)) || (st = check_head_dim(head_dim, esize)))
        return st;
    if (tokens < 0 || q_heads < 0 || kv_heads < 0 || num_slots < 0)
        return fail(QKR_ERR_INVALID_ARGUMENT, "negative tokens, heads or num_slots");
    if ((int64_t)q_heads + kv_heads > (1 << 20))
        return fail(QKR_ERR_UNSUPPORTED, "too many heads");
    if (tokens >= kMaxRows || !product_below({tokens, (int64_t)q_heads + 2 * (int64_t)kv_heads}, kMaxRows))
        return fail(QKR_ERR_UNSUPPORTED, "tokens * heads must stay below 2^31 rows per call");
    if ((v == nullptr) != (v_cache == nullptr))
        return fail(QKR_ERR_INVALID_ARGUMENT, "v and v_cache come together (both or neither)");
    if ((st = check_view("q", q, esize, 1, tokens, q_heads)) ||
        (st = check_view("q_out", q_out, esize, 1, tokens, q_heads)) ||
        (st = check_view("k", k, esize, 1, tokens, kv_heads)) ||
        (st = check_view("k_cache", k_cache, esize, 1, num_slots, kv_heads)))
        return st;
    if (v != nullptr && ((st = check_view("v", v, esize, 1, tokens, kv_heads)) ||
                         (st = check_view("v_cache", v_cache, esize, 1, num_slots, kv_heads))))
        return st;
    if (q_heads > 0 && (st = check_weight("q_weight", q_weight_dev)))
        return st;
    if (kv_heads > 0 && (st = check_weight("k_weight", k_weight_dev)))
        return st;
    if (tokens > 0 && kv_heads > 0) {
        if (slot_mapping_dev == nullptr)
            return fail(QKR_ERR_INVALID_ARGUMENT, "null slot mapping");
        if (!aligned(slot_mapping_dev, 8))
            return fail(QKR_ERR_MISALIGNED, "slot mapping is not 8-byte aligned");
        if (num_slots > 0 && (k_cache == nullptr || k_cache->ptr_dev == nullptr))
            return fail(QKR_ERR_INVALID_ARGUMENT, "null k_cache");
    }
    NormRopeArgs a{};
    int32_t pairing = 0, rotary_dim = 0;
    if ((st = check_rope(rope, head_dim, esize, tokens, a.rope, pairing, rotary_dim)))
        return st;
    if (tokens == 0 || q_heads + kv_heads == 0)
        return ok();

    fill_in(a.t[0], 0, q_heads ? q : nullptr, esize);
    fill_out(a.t[0], q_heads ? q_out : nullptr, esize);
    a.t[0].s[0].weight = q_heads ? static_cast<const char*>(q_weight_dev) : nullptr;
    a.t[0].heads = q_heads;
    // K and V leave through the caches (num_slots == 0: every slot is
    // outside, nothing is written).
    const int32_t cache_heads = num_slots > 0 ? kv_heads : 0;
    fill_in(a.t[1], 0, cache_heads ? k : nullptr, esize);
    fill_out(a.t[1], cache_heads ? k_cache : nullptr, esize);
    a.t[1].s[0].weight = cache_heads ? static_cast<const char*>(k_weight_dev) : nullptr;
    a.t[1].heads = cache_heads;
    a.t[1].slots = slot_mapping_dev;
    a.t[1].nslots = num_slots;
    if (v != nullptr) {
        fill_in(a.t[2], 0, cache_heads ? v : nullptr, esize);
        fill_out(a.t[2], cache_heads ? v_cache : nullptr, esize);
        a.t[2].heads = cache_heads;
        a.t[2].slots = slot_mapping_dev;
        a.t[2].nslots = num_slots;
    }
    a.batch = 1;
    a.tokens = (int32_t)tokens;
    a.tokens0 = (int32_t)tokens;
    a.head_dim = head_dim;
    a.rotary_dim = rotary_dim;
    a.eps = eps;
    a.inv_d = 1.0f / (float)head_dim;
    return launch(a, dtype, eager, pairing, reinterpret_cast<hipStream_t>(stream));
}

qkr_status qkr_joint_qk_norm_rope(int32_t batch, int32_t heads, int32_t head_dim, int32_t dtype, float eps,
                                  const qkr_stream* text, const qkr_stream* image, const qkr_view* q_out,
                                  const qkr_view* k_out, const qkr_view* v_out, const qkr_rope* rope,
                                  qkr_stream_t stream)
{
    int esize = 0;
    bool eager = false;
    qkr_status st;
    if ((st = check_dtype(dtype, esize, eager)) || (st = check_eps(eps)) || (st = check_head_dim(head_dim, esize)))
        return st;
    if (text == nullptr || image == nullptr)
        return fail(QKR_ERR_INVALID_ARGUMENT, "null text or image stream");
    if (batch < 0 || heads < 0 || text->tokens < 0 || image->tokens < 0)
        return fail(QKR_ERR_INVALID_ARGUMENT, "negative batch, heads or tokens");
    if (heads > (1 << 18))
        return fail(QKR_ERR_UNSUPPORTED, "too many heads");
    if (text->tokens >= kMaxRows || image->tokens >= kMaxRows)
        return fail(QKR_ERR_UNSUPPORTED, "a stream holds 2^31 tokens or more");
    const int64_t joint = text->tokens + image->tokens;
    if (joint >= kMaxRows || !product_below({batch, joint, 3, heads}, kMaxRows))
        return fail(QKR_ERR_UNSUPPORTED, "batch * tokens * 3 heads must stay below 2^31 rows per call");
    const qkr_stream* streams[2] = {text, image};
    static const char* names[2][3] = {{"text.q", "text.k", "text.v"}, {"image.q", "image.k", "image.v"}};
    for (int s = 0; s < 2; ++s) {
        const qkr_stream* x = streams[s];
        if ((st = check_view(names[s][0], &x->q, esize, batch, x->tokens, heads)) ||
            (st = check_view(names[s][1], &x->k, esize, batch, x->tokens, heads)) ||
            (st = check_view(names[s][2], &x->v, esize, batch, x->tokens, heads)))
            return st;
        if (x->tokens > 0 && heads > 0 &&
            ((st = check_weight(s ? "image.q_weight" : "text.q_weight", x->q_weight_dev)) ||
             (st = check_weight(s ? "image.k_weight" : "text.k_weight", x->k_weight_dev))))
            return st;
    }
    if ((st = check_view("q_out", q_out, esize, batch, joint, heads)) ||
        (st = check_view("k_out", k_out, esize, batch, joint, heads)) ||
        (st = check_view("v_out", v_out, esize, batch, joint, heads)))
        return st;
    NormRopeArgs a{};
    int32_t pairing = 0, rotary_dim = 0;
    if ((st = check_rope(rope, head_dim, esize, joint, a.rope, pairing, rotary_dim)))
        return st;
    if (batch == 0 || joint == 0 || heads == 0)
        return ok();

    const qkr_view* outs[3] = {q_out, k_out, v_out};
    for (int ti = 0; ti < 3; ++ti) {
        for (int s = 0; s < 2; ++s) {
            const qkr_stream* x = streams[s];
            const qkr_view* v = ti == 0 ? &x->q : (ti == 1 ? &x->k : &x->v);
            fill_in(a.t[ti], s, x->tokens > 0 ? v : nullptr, esize);
            a.t[ti].s[s].weight = ti == 2 || x->tokens == 0
                                    ? nullptr
                                    : static_cast<const char*>(ti == 0 ? x->q_weight_dev : x->k_weight_dev);
        }
        fill_out(a.t[ti], outs[ti], esize);
        a.t[ti].heads = heads;
    }
    a.batch = batch;
    a.tokens = (int32_t)joint;
    a.tokens0 = (int32_t)text->tokens;
    a.head_dim = head_dim;
    a.rotary_dim = rotary_dim;
    a.eps = eps;
    a.inv_d = 1.0f / (float)head_dim;
    return launch(a, dtype, eager, pairing, reinterpret_cast<hipStream_t>(stream));
}

qkr_status qkr_mrope_cos_sin_setup(const float* inv_freq_t_dev, int32_t half_t, const float* inv_freq_h_dev,
                                   int32_t half_h, const float* inv_freq_w_dev, int32_t half_w,
                                   const int32_t* grid_thw, int32_t num_grids, int32_t spatial_merge,
                                   float* cos_out_dev, float* sin_out_dev, int64_t n_tokens, qkr_stream_t stream)
{
    if (half_t < 0 || half_h < 0 || half_w < 0 || (int64_t)half_t + half_h + half_w <= 0)
        return fail(QKR_ERR_INVALID_ARGUMENT, "axis halves (%d, %d, %d) must be >= 0 with a positive sum",
                    half_t, half_h, half_w);
    const float* inv[3] = {inv_freq_t_dev, inv_freq_h_dev, inv_freq_w_dev};
    const int32_t half[3] = {half_t, half_h, half_w};
    for (int i = 0; i < 3; ++i) {
        if (half[i] > 0 && inv[i] == nullptr)
            return fail(QKR_ERR_INVALID_ARGUMENT, "axis %d has %d frequencies but a null inv_freq", i, half[i]);
        if (!aligned(inv[i], 4))
            return fail(QKR_ERR_MISALIGNED, "inv_freq of axis %d is not 4-byte aligned", i);
    }
    int64_t total = 0;
    qkr_status st;
    if ((st = check_grids(grid_thw, num_grids, spatial_merge, total)))
        return st;
    if (n_tokens != total)
        return fail(QKR_ERR_INVALID_ARGUMENT, "n_tokens %lld != sum of t*h*w = %lld", (long long)n_tokens,
                    (long long)total);
    // One thread per (token, column) on a 1-D grid.
    if (!product_below({n_tokens, (int64_t)half_t + half_h + half_w}, kMaxRows))
        return fail(QKR_ERR_UNSUPPORTED, "n_tokens * (half_t + half_h + half_w) must stay below 2^31");
    if (cos_out_dev == nullptr || sin_out_dev == nullptr)
        return fail(QKR_ERR_INVALID_ARGUMENT, "null cos or sin output");
    if (!aligned(cos_out_dev, 4) || !aligned(sin_out_dev, 4))
        return fail(QKR_ERR_MISALIGNED, "cos/sin outputs are not 4-byte aligned");

    VitArgs base{};
    for (int i = 0; i < 3; ++i) {
        base.inv[i] = inv[i];
        base.half[i] = half[i];
    }
    base.off[0] = 0;
    base.off[1] = half_t;
    base.off[2] = half_t + half_h;
    base.half_rot = half_t + half_h + half_w;
    base.cos_out = cos_out_dev;
    base.sin_out = sin_out_dev;
    base.n_tokens = n_tokens;
    base.div_groups = make_fastdiv((uint32_t)((base.half_rot + 3) / 4));
    // 16-byte stores need aligned planes and sections of whole 4-column groups.
    base.vec_ok = aligned(cos_out_dev, 16) && aligned(sin_out_dev, 16) && half_t % 4 == 0 && half_h % 4 == 0 &&
                  half_w % 4 == 0;
    (void)hipGetLastError();
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const hipError_t e = for_grid_groups(grid_thw, num_grids, spatial_merge, base,
                                         [&](const VitArgs& a) { return launch_vit_setup(a, s); });
    if (e == hipSuccess)
        std::snprintf(g_variant, sizeof(g_variant), "vit_setup");
    return hip_status(e, "mrope_cos_sin_setup launch");
}

qkr_status qkr_vit_qk_norm_rope(int64_t tokens, int32_t head_dim, int32_t dtype, float eps, const qkr_view* q,
                                const qkr_view* q_out, int32_t q_heads, const void* q_weight_dev,
                                const qkr_view* k, const qkr_view* k_out, int32_t k_heads,
                                const void* k_weight_dev, int32_t pairing, const float* inv_freq_t_dev,
                                int32_t half_t, const float* inv_freq_h_dev, int32_t half_h,
                                const float* inv_freq_w_dev, int32_t half_w, const int32_t* grid_thw,
                                int32_t num_grids, int32_t spatial_merge, qkr_stream_t stream)
{
    int esize = 0;
    bool eager = false;
    qkr_status st;
    if ((st = check_dtype(dtype, esize, eager)) || (st = check_eps(eps)) || (st = check_head_dim(head_dim, esize)))
        return st;
    if (tokens < 0 || q_heads < 0 || k_heads < 0)
        return fail(QKR_ERR_INVALID_ARGUMENT, "negative tokens or heads");
    if ((int64_t)q_heads + k_heads > (1 << 20))
        return fail(QKR_ERR_UNSUPPORTED, "too many heads");
    if (tokens >= kMaxRows || !product_below({tokens, (int64_t)q_heads + k_heads}, kMaxRows))
        return fail(QKR_ERR_UNSUPPORTED, "tokens * heads must stay below 2^31 rows per call");
    if ((st = check_view("q", q, esize, 1, tokens, q_heads)) ||
        (st = check_view("q_out", q_out, esize, 1, tokens, q_heads)) ||
        (st = check_view("k", k, esize, 1, tokens, k_heads)) ||
        (st = check_view("k_out", k_out, esize, 1, tokens, k_heads)))
        return st;
    if (q_heads > 0 && (st = check_weight("q_weight", q_weight_dev)))
        return st;
    if (k_heads > 0 && (st = check_weight("k_weight", k_weight_dev)))
        return st;
    if (pairing != QKR_PAIR_NEOX && pairing != QKR_PAIR_ADJACENT)
        return fail(QKR_ERR_INVALID_ARGUMENT, "unknown pairing %d", pairing);
    if (half_t < 0 || half_h < 0 || half_w < 0 || (int64_t)half_t + half_h + half_w <= 0)
        return fail(QKR_ERR_INVALID_ARGUMENT, "axis halves (%d, %d, %d) must be >= 0 with a positive sum",
                    half_t, half_h, half_w);
    if ((int64_t)half_t + half_h + half_w > head_dim / 2)
        return fail(QKR_ERR_INVALID_ARGUMENT, "rotary dims 2 * (%d + %d + %d) exceed head_dim %d", half_t,
                    half_h, half_w, head_dim);
    const int32_t half = half_t + half_h + half_w;
    if (pairing == QKR_PAIR_NEOX && half % (16 / esize) != 0)
        return fail(QKR_ERR_UNSUPPORTED, "NeoX pairing needs rotary_dim/2 (%d) to be a multiple of %d elements",
                    half, 16 / esize);
    const float* inv[3] = {inv_freq_t_dev, inv_freq_h_dev, inv_freq_w_dev};
    const int32_t halves[3] = {half_t, half_h, half_w};
    for (int i = 0; i < 3; ++i) {
        if (halves[i] > 0 && inv[i] == nullptr)
            return fail(QKR_ERR_INVALID_ARGUMENT, "axis %d has %d frequencies but a null inv_freq", i, halves[i]);
        if (!aligned(inv[i], 4))
            return fail(QKR_ERR_MISALIGNED, "inv_freq of axis %d is not 4-byte aligned", i);
    }
    int64_t total = 0;
    if ((st = check_grids(grid_thw, num_grids, spatial_merge, total)))
        return st;
    if (tokens != total)
        return fail(QKR_ERR_INVALID_ARGUMENT, "tokens %lld != sum of t*h*w = %lld", (long long)tokens,
                    (long long)total);
    if (tokens == 0 || q_heads + k_heads == 0)
        return ok();

    NormRopeArgs base{};
    base.t[0].heads = q_heads;
    base.t[0].s[0].weight = q_heads ? static_cast<const char*>(q_weight_dev) : nullptr;
    base.t[1].heads = k_heads;
    base.t[1].s[0].weight = k_heads ? static_cast<const char*>(k_weight_dev) : nullptr;
    base.t[2].heads = 0;
    base.batch = 1;
    base.head_dim = head_dim;
    base.rotary_dim = 2 * half;
    base.eps = eps;
    base.inv_d = 1.0f / (float)head_dim;
    base.rope.mode = kPosVit;
    base.rope.half = half;
    base.rope.sec[0] = half_t;
    base.rope.sec[1] = half_h;
    base.rope.sec[2] = half_w;
    base.rope.sec[3] = 0;
    build_axis_bits(kPosAxes, base.rope.sec, half, base.rope.axis_bits);
    for (int i = 0; i < 3; ++i)
        base.vit.inv[i] = inv[i];
    base.vit.merge = spatial_merge;
    base.vit.div_m = make_fastdiv((uint32_t)spatial_merge);
    base.vit.div_mm = make_fastdiv((uint32_t)(spatial_merge * spatial_merge));

    RopePlan plan;
    if ((st = plan_rope(base, dtype, plan)))
        return st;
    // One launch per group of grids; views start at the group's first token,
    // positions use absolute token indices (token_base).
    int64_t start = 0;
    for (int32_t g0 = 0; g0 < num_grids; g0 += kMaxFusedGrids) {
        const int32_t n = num_grids - g0 < kMaxFusedGrids ? num_grids - g0 : kMaxFusedGrids;
        NormRopeArgs a = base;
        a.vit.num_grids = n;
        int64_t cu = start;
        for (int32_t k2 = 0; k2 < n; ++k2) {
            const int32_t* g = grid_thw + 3 * (g0 + k2);
            a.vit.cu[k2] = cu;
            // h * w is at most t * h * w < 2^31; w / merge >= 1 (w is a multiple of merge).
            a.vit.div_area[k2] = make_fastdiv((uint32_t)((int64_t)g[1] * g[2]));
            a.vit.div_bcols[k2] = make_fastdiv((uint32_t)(g[2] / spatial_merge));
            cu += (int64_t)g[0] * g[1] * g[2];
        }
        a.vit.cu[n] = cu;
        const int64_t count = cu - start;
        const qkr_view* ins[2] = {q, k};
        const qkr_view* outs[2] = {q_out, k_out};
        const int32_t heads[2] = {q_heads, k_heads};
        for (int ti = 0; ti < 2; ++ti) {
            if (heads[ti] == 0)
                continue;
            qkr_view vi = *ins[ti], vo = *outs[ti];
            vi.ptr_dev = static_cast<char*>(vi.ptr_dev) + start * vi.stride_tok * esize;
            vo.ptr_dev = static_cast<char*>(vo.ptr_dev) + start * vo.stride_tok * esize;
            fill_in(a.t[ti], 0, &vi, esize);
            fill_out(a.t[ti], &vo, esize);
        }
        a.tokens = (int32_t)count;
        a.tokens0 = (int32_t)count;
        a.rope.token_base = start;
        if ((st = launch_planned(a, dtype, eager, pairing, plan, reinterpret_cast<hipStream_t>(stream))))
            return st;
        start = cu;
    }
    return ok();
}

qkr_status qkr_debug_axis_map(const qkr_rope* rope, int32_t n_pairs, int32_t* out_dev, qkr_stream_t stream)
{
    qkr_status st;
    if (rope == nullptr || n_pairs < 0 || (n_pairs > 0 && out_dev == nullptr))
        return fail(QKR_ERR_INVALID_ARGUMENT, "debug_axis_map: null rope/output or negative n_pairs");
    if ((st = check_map_rope(rope)))
        return st;
    if (n_pairs > kMaxPairs)
        return fail(QKR_ERR_UNSUPPORTED, "debug_axis_map: at most %d pairs", kMaxPairs);
    RopeArgs r{};
    build_axis_bits(rope->mode, rope->sections, n_pairs, r.axis_bits);
    (void)hipGetLastError();
    return hip_status(launch_debug_axis_map(r, n_pairs, out_dev, reinterpret_cast<hipStream_t>(stream)),
                      "debug_axis_map launch");
}

qkr_status qkr_axis_map_host(const qkr_rope* rope, int32_t n_pairs, int32_t* out_host)
{
    qkr_status st;
    if (rope == nullptr || n_pairs < 0 || (n_pairs > 0 && out_host == nullptr))
        return fail(QKR_ERR_INVALID_ARGUMENT, "axis_map_host: null rope/output or negative n_pairs");
    if ((st = check_map_rope(rope)))
        return st;
    for (int32_t p = 0; p < n_pairs; ++p)
        out_host[p] = pair_axis(rope->mode, rope->sections, p);
    return ok();
}

qkr_status qkr_debug_vit_positions(const int32_t* grid_thw, int32_t num_grids, int32_t spatial_merge,
                                   int32_t* out_dev, int64_t n_tokens, qkr_stream_t stream)
{
    int64_t total = 0;
    qkr_status st;
    if ((st = check_grids(grid_thw, num_grids, spatial_merge, total)))
        return st;
    if (n_tokens != total || out_dev == nullptr)
        return fail(QKR_ERR_INVALID_ARGUMENT, "n_tokens must equal sum t*h*w and out must be non-null");
    VitArgs base{};
    base.n_tokens = n_tokens;
    (void)hipGetLastError();
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    return hip_status(for_grid_groups(grid_thw, num_grids, spatial_merge, base,
                                      [&](const VitArgs& a) { return launch_debug_vit_positions(a, out_dev, s); }),
                      "debug_vit_positions launch");
}

qkr_status qkr_vit_positions_host(const int32_t* grid_thw, int32_t num_grids, int32_t spatial_merge,
                                  int32_t* out_host, int64_t n_tokens)
{
    int64_t total = 0;
    qkr_status st;
    if ((st = check_grids(grid_thw, num_grids, spatial_merge, total)))
        return st;
    if (n_tokens != total || out_host == nullptr)
        return fail(QKR_ERR_INVALID_ARGUMENT, "n_tokens must equal sum t*h*w and out must be non-null");
    VitArgs base{};
    base.n_tokens = n_tokens;
    for_grid_groups(grid_thw, num_grids, spatial_merge, base, [&](const VitArgs& a) {
        for (int64_t i = 0; i < a.tok_count; ++i) {
            const int64_t n = a.tok_begin + i;
            vit_position(a, (uint32_t)n, &out_host[n], &out_host[n_tokens + n], &out_host[2 * n_tokens + n]);
        }
        return hipSuccess;
    });
    return ok();
}

}  // extern "C"
