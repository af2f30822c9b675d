/*
 * CPU oracle for per-row RMSNorm fused with rotary position embedding.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load or call this library.  It shares no
 * code with the HIP library.  Build: gcc -O2 -ffp-contract=off (no fast-math),
 * so every operation below is one IEEE double operation in source order.
 *
 * Sources (web pages; cited by the short name in brackets):
 *   [Ovis]   vllm-omni pull request "[Kernel][Ovis-Image] Fuse text/image QK
 *            RMSNorm + cat + RoPE into one Triton launch"
 *   [Vulkan] vllm.cpp pull request "perf(vulkan): decode RmsNorm ran on ONE
 *            workgroup -- 7.85 -> 1.59 ms/token"
 *   [IMROPE] llama.cpp fork pull request "hrx: the multi-section rotation of
 *            Qwen3-VL runs on the device, not on the CPU"
 *   [ViT]    vLLM API page "vllm.model_executor.layers.rotary_embedding.
 *            mrope_vit_setup"
 *   [VecRMS] vLLM pull request "Vectorize RMS norm variance using
 *            vectorize_read_with_alignment"
 *
 * Readings taken where the pages leave a step open are listed with the
 * function that takes them.  What pins each function against something other
 * than itself is in tests/test_oracle_pins.py.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Rounding                                                                  */
/* ------------------------------------------------------------------------ */

/* bf16 keeps 8 significant bits and fp32's exponent range.  A normal value in
 * [2^(e-1), 2^e) therefore sits on a grid of spacing 2^(e-8); below 2^-126 the
 * spacing stays at 2^-133 (subnormals).  nearbyint() rounds half to even in
 * the default rounding mode.  Results past the largest finite bf16
 * (0x1.FEp127) become infinity. */
double oracle_round_bf16(double v)
{
    if (v == 0.0 || !isfinite(v))
        return v;
    int e;
    (void)frexp(v, &e);
    int q = e - 8;
    if (q < -133)
        q = -133;
    double r = ldexp(nearbyint(ldexp(v, -q)), q);
    if (fabs(r) > 0x1.FEp127)
        r = copysign(INFINITY, v);
    return r;
}

static float round_out(double v, int32_t out_kind)
{
    if (out_kind == ORACLE_OUT_BF16)
        return (float)oracle_round_bf16(v);   /* exact: a bf16 value fits a float */
    return (float)v;                          /* round to nearest even fp32 */
}

/* Products and differences of two floats taken in double and then rounded
 * to float are the correctly rounded float results (double carries more
 * than twice float's 24 bits plus two), so the helpers below are IEEE fp32
 * operations, each rounded once. */
static float mul32(float a, float b) { return (float)((double)a * (double)b); }
static float sub32(float a, float b) { return (float)((double)a - (double)b); }
static float add32(float a, float b) { return (float)((double)a + (double)b); }

/* ------------------------------------------------------------------------ */
/* RMSNorm of one row                                                        */
/* ------------------------------------------------------------------------ */

/* u_i = x_i * rrms * w_i with rrms = 1 / sqrt(sum(x^2) / d + eps).
 * The normalisation statistic is the mean of the squares and eps is added
 * inside the square root ([Ovis] and [VecRMS]: RMSNorm with eps 1e-6; the
 * weight multiplies the normalised value, [VecRMS] review thread quoting the
 * output expression of rms_norm_kernel).
 *
 * Eager numerics (ORACLE_NUMERICS_EAGER): the rounding points of an eager
 * RMSNorm kernel, whose output expression the [VecRMS] review thread quotes
 * as ((scalar_t)(x * s_variance)) * weight[idx].  Reading: s_variance is the
 * fp32 value of rrms; x * s_variance is one fp32 product; it is rounded to the
 * activation type (scalar_t); that value times the weight is rounded to the
 * activation type once more.  u_i then already lies on the activation grid. */
static void norm_row(const float* x, const float* w, int32_t d, float eps, int32_t numerics,
                     int32_t act_kind, double* u)
{
    double ss = 0.0;
    for (int32_t i = 0; i < d; ++i)
        ss += (double)x[i] * (double)x[i];
    double rrms = 1.0 / sqrt(ss / (double)d + (double)eps);
    if (numerics == ORACLE_NUMERICS_EAGER) {
        const float r32 = (float)rrms;
        for (int32_t i = 0; i < d; ++i) {
            const double xs = (double)round_out((double)mul32(x[i], r32), act_kind);
            u[i] = (double)round_out(xs * (double)w[i], act_kind);
        }
        return;
    }
    for (int32_t i = 0; i < d; ++i)
        u[i] = (double)x[i] * rrms * (double)w[i];
}

/* Plain row RMSNorm ([Vulkan] decode RmsNorm of width 5120; [VecRMS]).
 * Reading: one rounding of x * rrms * w to the output type (eager numerics:
 * the two roundings of norm_row). */
void oracle_rms_norm(const float* x, int64_t rows, int32_t width, const float* weight,
                     float eps, int32_t out_kind, int32_t numerics, float* y)
{
    double* u = (double*)malloc(sizeof(double) * (size_t)width);
    for (int64_t r = 0; r < rows; ++r) {
        norm_row(x + r * width, weight, width, eps, numerics, out_kind, u);
        for (int32_t i = 0; i < width; ++i)
            y[r * width + i] = round_out(u[i], out_kind);
    }
    free(u);
}

/* ------------------------------------------------------------------------ */
/* Residual add + RMSNorm, optionally with a static FP8 E4M3 output          */
/* ------------------------------------------------------------------------ */

/* OCP FP8 E4M3 (the variant without infinities): sign, a 4-bit exponent with
 * bias 7 and a 3-bit mantissa.  Exponent field e > 0: 2^(e-7) * (1 + m/8);
 * e == 0: 2^-6 * m/8; e == 15 with m == 7 is NaN, so the largest finite
 * magnitude is 2^8 * 1.75 = 448.  ([VecRMS] names the static FP8 RMSNorm
 * kernel; the format is the one gfx950 converts to natively.) */
double oracle_fp8_e4m3_decode(uint8_t code)
{
    const int e = (code >> 3) & 15, m = code & 7;
    double v;
    if (e == 15 && m == 7)
        v = NAN;
    else if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(8.0 + (double)m, e - 10);
    return (code & 0x80) ? -v : v;
}

/* Reading: a static quantiser saturates at the largest finite magnitude and
 * rounds half to even on the E4M3 grid: spacing 2^-9 below 2^-6 (subnormals,
 * whose top step lands on 2^-6 itself), spacing 2^(k-3) in [2^k, 2^(k+1)).
 * Finite inputs only; the sign of zero is kept. */
uint8_t oracle_fp8_e4m3_encode(double v)
{
    const uint8_t sign = signbit(v) ? 0x80 : 0x00;
    const double a = fabs(v);
    if (a >= 448.0)
        return sign | 0x7E;
    if (a < 0x1p-6)
        return sign | (uint8_t)nearbyint(ldexp(a, 9));   /* 0..8; 8 is the code of 2^-6 */
    int k;
    (void)frexp(a, &k);
    k -= 1;                                   /* a in [2^k, 2^(k+1)), -6 <= k <= 8 */
    double q = nearbyint(ldexp(a, 3 - k));    /* 8..16 */
    if (q == 16.0) {
        q = 8.0;
        k += 1;
    }
    return sign | (uint8_t)(((k + 7) << 3) | ((int)q - 8));
}

/* [Vulkan] decode RmsNorm: the calls carry the residual add and the weight
 * multiply, and the residual stream is held bit-exactly by rounding the sum
 * in registers.  Reading: s = x + r rounded once to the activation type is
 * both the stored residual stream and the norm's input; the norm then follows
 * norm_row.  For the FP8 output the quantised code is decided in fp32, as a
 * kernel holding y in a register decides it: fl32(y), then the correctly
 * rounded fp32 quotient by the scale (a double quotient of two floats rounded
 * to float is the correctly rounded float quotient), then the encoding. */
void oracle_add_rms_norm(const float* x, const float* r, int64_t rows, int32_t width, const float* weight,
                         float eps, int32_t act_kind, int32_t out_kind, int32_t numerics, float scale,
                         float* s_out, float* y_out, uint8_t* code_out)
{
    float* s = (float*)malloc(sizeof(float) * (size_t)width);
    double* u = (double*)malloc(sizeof(double) * (size_t)width);
    for (int64_t row = 0; row < rows; ++row) {
        const float* xr = x + row * width;
        for (int32_t i = 0; i < width; ++i) {
            const double sum = r ? (double)xr[i] + (double)r[row * width + i] : (double)xr[i];
            s[i] = round_out(sum, act_kind);
        }
        if (s_out)
            memcpy(s_out + row * width, s, sizeof(float) * (size_t)width);
        norm_row(s, weight, width, eps, numerics, act_kind, u);
        for (int32_t i = 0; i < width; ++i) {
            if (out_kind == ORACLE_OUT_FP8_E4M3) {
                const float y32 = (float)u[i];
                const float q = (float)((double)y32 / (double)scale);
                if (code_out)
                    code_out[row * width + i] = oracle_fp8_e4m3_encode((double)q);
            } else if (y_out) {
                y_out[row * width + i] = round_out(u[i], out_kind);
            }
        }
    }
    free(u);
    free(s);
}

/* ------------------------------------------------------------------------ */
/* Which position axis a rotary pair reads                                   */
/* ------------------------------------------------------------------------ */

/* AXES / PLANES: the pairs are split into contiguous runs, sections[0] pairs
 * on t, then sections[1] on h, then sections[2] on w ([ViT] setup kernel: the
 * t, h and w column ranges of the planes follow one another).
 * IMROPE ([IMROPE] "The change", and the review comment that sets the rule
 * beside ggml_mrope_cache_init): the pairs repeat in periods of
 * S = s0+s1+s2+s3; inside a period the t, h and w pairs interleave, the k-th
 * pair of axis a (t = 0, h = 1, w = 2) sitting at offset 3k + a for k < s_a,
 * and every offset no axis claims reads the fourth component e.  Written here
 * by laying one period out, axis by axis, and reading pair p at offset
 * p mod S. */
int32_t oracle_axis(const oracle_rope* rope, int32_t p)
{
    const int32_t* s = rope->sections;
    switch (rope->mode) {
    case ORACLE_POS_1D:
        return ORACLE_AXIS_T;
    case ORACLE_POS_AXES:
    case ORACLE_POS_PLANES: {
        int32_t end = 0;
        for (int32_t a = 0; a < 3; ++a) {
            end += s[a];
            if (p < end)
                return a;
        }
        return -1;   /* pair outside every section: invalid input */
    }
    case ORACLE_POS_IMROPE: {
        const int32_t period = s[0] + s[1] + s[2] + s[3];
        int32_t* layout = (int32_t*)malloc(sizeof(int32_t) * (size_t)period);
        for (int32_t o = 0; o < period; ++o)
            layout[o] = ORACLE_AXIS_E;
        for (int32_t a = 0; a < 3; ++a)
            for (int32_t k = 0; k < s[a] && 3 * k + a < period; ++k)
                layout[3 * k + a] = a;
        const int32_t axis = layout[p % period];
        free(layout);
        return axis;
    }
    default:
        return -1;
    }
}

/* ------------------------------------------------------------------------ */
/* cos and sin of one (token, pair)                                          */
/* ------------------------------------------------------------------------ */

/* The angle is the fp32 product of the fp32 position and the fp32 inverse
 * frequency, rounded once ([ViT] setup kernel multiplies the float32 position
 * by inv_freq).  Its cos and sin are then taken in double.  The position is
 * read at plane * pos_stride + token_base + token: a launch over a token chunk
 * keeps the whole-length planes and is told where its tokens start ([IMROPE]
 * "The change" and "Proof", the chunk-offset bug).  PLANES mode reads the cos
 * and sin that the setup wrote for the pair's axis ([ViT] the consumer reads
 * only each axis's section columns). */
static void pair_cos_sin(const oracle_rope* rope, int64_t tok, int32_t p, double* c, double* s)
{
    int32_t a = oracle_axis(rope, p);
    int64_t t = rope->token_base + tok;
    if (rope->mode == ORACLE_POS_PLANES) {
        int64_t half = rope->rotary_dim / 2;
        int64_t idx = ((int64_t)a * rope->planes_tokens + t) * half + p;
        *c = (double)rope->cos_planes[idx];
        *s = (double)rope->sin_planes[idx];
        return;
    }
    int32_t pos = rope->positions[(int64_t)a * rope->pos_stride + t];
    float theta = (float)((float)pos * rope->inv_freq[p]);
    *c = cos((double)theta);
    *s = sin((double)theta);
}

/* ------------------------------------------------------------------------ */
/* One (token, head) row: norm, contract rounding, rotation, final rounding  */
/* ------------------------------------------------------------------------ */

/* Rounding contract ([Ovis] kernel review): the normalised value (weight
 * included) is rounded to bf16 once, the rotation runs on that value and the
 * result is rounded once more.  For fp32 outputs there is no intermediate
 * rounding.
 *
 * Pairing: NeoX pairs element p with p + R/2 ([IMROPE]: the sectioned mode
 * keeps mode 2's pairing); the adjacent pairing pairs 2p with 2p+1 ([Ovis]
 * interleaved=True path).  Rotation by +theta, the standard rotate-half
 * convention a' = a cos - b sin, b' = b cos + a sin (the pages print no sign).
 * Elements at or beyond R pass through. */
static void norm_rope_row(const float* x, const float* w, int32_t d, float eps, int32_t out_kind,
                          int32_t numerics, const oracle_rope* rope, int64_t tok, double* n, float* out)
{
    const int eager = numerics == ORACLE_NUMERICS_EAGER;
    norm_row(x, w, d, eps, numerics, out_kind, n);
    if (out_kind == ORACLE_OUT_BF16 && !eager)
        for (int32_t i = 0; i < d; ++i)
            n[i] = oracle_round_bf16(n[i]);

    int32_t r = (rope != NULL) ? rope->rotary_dim : 0;
    for (int32_t i = r; i < d; ++i)
        out[i] = round_out(n[i], out_kind);
    for (int32_t p = 0; p < r / 2; ++p) {
        int32_t i, j;
        if (rope->pairing == ORACLE_PAIR_NEOX) {
            i = p;
            j = p + r / 2;
        } else {
            i = 2 * p;
            j = 2 * p + 1;
        }
        double c, s;
        pair_cos_sin(rope, tok, p, &c, &s);
        if (eager) {
            /* Eager numerics ([Ovis] "Supplemental eager bitwise measurements":
             * the preset that reproduced the eager chain turns floating-point
             * fusion off, and that chain reads its RoPE table in the
             * activation type, bf16 in the measured case).  Reading: the table
             * holds cos and sin computed in fp32 (each rounded once to fp32)
             * and stored in the activation type; each product is rounded to
             * fp32; their difference or sum is rounded to fp32; then the final
             * rounding to the output type. */
            const float ct = round_out((double)(float)c, out_kind), st = round_out((double)(float)s, out_kind);
            const float ni = (float)n[i], nj = (float)n[j];
            out[i] = round_out((double)sub32(mul32(ni, ct), mul32(nj, st)), out_kind);
            out[j] = round_out((double)add32(mul32(nj, ct), mul32(ni, st)), out_kind);
            continue;
        }
        out[i] = round_out(n[i] * c - n[j] * s, out_kind);
        out[j] = round_out(n[j] * c + n[i] * s, out_kind);
    }
}

void oracle_qk_norm_rope(const float* x, int64_t tokens, int32_t heads, int32_t head_dim,
                         const float* weight, float eps, int32_t out_kind, int32_t numerics,
                         const oracle_rope* rope, float* out)
{
    double* n = (double*)malloc(sizeof(double) * (size_t)head_dim);
    for (int64_t t = 0; t < tokens; ++t)
        for (int32_t h = 0; h < heads; ++h) {
            int64_t row = (t * heads + h) * (int64_t)head_dim;
            norm_rope_row(x + row, weight, head_dim, eps, out_kind, numerics, rope, t, n, out + row);
        }
    free(n);
}

/* [IMROPE] "The change": the rotation kernel has a set_rows twin, which
 * writes each rotated row into a destination row picked by an index (the
 * step that stores K into the KV cache).  Reading: row slots[t] of the cache
 * receives token t's K (normalised and rotated) and V (unchanged) for every
 * KV head; a slot outside the cache writes nothing (the usual mark of a
 * padding token); a mapping that sends two tokens to one slot leaves that
 * slot's content unspecified, so the tests use injective mappings. */
void oracle_qk_norm_rope_cache(const float* q, int32_t q_heads, const float* k, const float* v,
                               int32_t kv_heads, int64_t tokens, int32_t head_dim, const float* q_weight,
                               const float* k_weight, float eps, int32_t out_kind, int32_t numerics,
                               const oracle_rope* rope, const int64_t* slots, int64_t num_slots, float* q_out,
                               float* k_cache, float* v_cache)
{
    const int64_t row = (int64_t)kv_heads * head_dim;
    float* k_rot = (float*)malloc(sizeof(float) * (size_t)(tokens * row > 0 ? tokens * row : 1));
    oracle_qk_norm_rope(q, tokens, q_heads, head_dim, q_weight, eps, out_kind, numerics, rope, q_out);
    oracle_qk_norm_rope(k, tokens, kv_heads, head_dim, k_weight, eps, out_kind, numerics, rope, k_rot);
    for (int64_t t = 0; t < tokens; ++t) {
        const int64_t slot = slots[t];
        if (slot < 0 || slot >= num_slots)
            continue;
        memcpy(k_cache + slot * row, k_rot + t * row, sizeof(float) * (size_t)row);
        if (v != NULL && v_cache != NULL)
            memcpy(v_cache + slot * row, v + t * row, sizeof(float) * (size_t)row);
    }
    free(k_rot);
}

/* ------------------------------------------------------------------------ */
/* Joint text/image op                                                       */
/* ------------------------------------------------------------------------ */

/* [Ovis] "Purpose": four RMSNorms, three concatenations and the RoPE pass of
 * a double block become one op whose outputs are the joint
 * [B, S_txt + S_img, H, D] Q/K/V, text first.  Each stream keeps its own q and
 * k norm weights; positions are indexed by the joint token; V is routed
 * unchanged (the bitwise-candidate comment: routed V matches exactly). */
void oracle_joint_qk_norm_rope(int32_t batch, int32_t heads, int32_t head_dim,
                               const float* q_txt, const float* k_txt, const float* v_txt,
                               int64_t tokens_txt, const float* qw_txt, const float* kw_txt,
                               const float* q_img, const float* k_img, const float* v_img,
                               int64_t tokens_img, const float* qw_img, const float* kw_img,
                               float eps, int32_t out_kind, int32_t numerics, const oracle_rope* rope,
                               float* q_out, float* k_out, float* v_out)
{
    int64_t joint = tokens_txt + tokens_img;
    int64_t row_elems = (int64_t)heads * head_dim;
    double* n = (double*)malloc(sizeof(double) * (size_t)head_dim);
    for (int32_t b = 0; b < batch; ++b)
        for (int64_t tau = 0; tau < joint; ++tau) {
            const float *q, *k, *v, *qw, *kw;
            if (tau < tokens_txt) {
                int64_t src = ((int64_t)b * tokens_txt + tau) * row_elems;
                q = q_txt + src; k = k_txt + src; v = v_txt + src;
                qw = qw_txt; kw = kw_txt;
            } else {
                int64_t src = ((int64_t)b * tokens_img + (tau - tokens_txt)) * row_elems;
                q = q_img + src; k = k_img + src; v = v_img + src;
                qw = qw_img; kw = kw_img;
            }
            int64_t dst = ((int64_t)b * joint + tau) * row_elems;
            for (int32_t h = 0; h < heads; ++h) {
                int64_t o = (int64_t)h * head_dim;
                norm_rope_row(q + o, qw, head_dim, eps, out_kind, numerics, rope, tau, n, q_out + dst + o);
                norm_rope_row(k + o, kw, head_dim, eps, out_kind, numerics, rope, tau, n, k_out + dst + o);
            }
            memcpy(v_out + dst, v, sizeof(float) * (size_t)row_elems);
        }
    free(n);
}

/* ------------------------------------------------------------------------ */
/* ViT positions and cos/sin planes                                          */
/* ------------------------------------------------------------------------ */

/* [ViT] setup kernel's token order: the grids follow one another; a grid's
 * tokens run frame by frame; inside a frame they run over the spatial-merge
 * blocks (m x m patches) in raster order of the block grid (block row, then
 * block column), and inside a block over its m x m cells row by row.  The
 * (t, h, w) of every token is written out by walking that order, one token
 * after the other. */
void oracle_vit_positions(const int32_t* grid_thw, int32_t num_grids, int32_t merge,
                          int32_t* pos, int64_t n_tokens)
{
    int64_t n = 0;
    for (int32_t g = 0; g < num_grids; ++g) {
        const int32_t frames = grid_thw[3 * g], h = grid_thw[3 * g + 1], w = grid_thw[3 * g + 2];
        for (int32_t t = 0; t < frames; ++t)
            for (int32_t brow = 0; brow < h / merge; ++brow)
                for (int32_t bcol = 0; bcol < w / merge; ++bcol)
                    for (int32_t i = 0; i < merge; ++i)
                        for (int32_t j = 0; j < merge; ++j) {
                            if (n < n_tokens) {
                                pos[n] = t;
                                pos[n_tokens + n] = brow * merge + i;
                                pos[2 * n_tokens + n] = bcol * merge + j;
                            }
                            ++n;
                        }
    }
}

/* (3, n_tokens) positions, freshly allocated (the caller frees them). */
static int32_t* vit_position_table(const int32_t* grid_thw, int32_t num_grids, int32_t merge, int64_t n_tokens)
{
    int32_t* pos = (int32_t*)malloc(sizeof(int32_t) * (size_t)(3 * (n_tokens > 0 ? n_tokens : 1)));
    oracle_vit_positions(grid_thw, num_grids, merge, pos, n_tokens);
    return pos;
}

/* Plane a, columns [off_a, off_a + half_a): cos and sin of
 * fl32(fl32(pos_a) * inv_a[j]), each rounded once to fp32.  Other columns of
 * plane a are not written ([ViT]: left uninitialized). */
void oracle_vit_cos_sin(const float* inv_t, int32_t half_t, const float* inv_h, int32_t half_h,
                        const float* inv_w, int32_t half_w, const int32_t* grid_thw,
                        int32_t num_grids, int32_t merge, float* cos_out, float* sin_out,
                        int64_t n_tokens)
{
    int64_t half_rot = (int64_t)half_t + half_h + half_w;
    const float* inv[3] = {inv_t, inv_h, inv_w};
    int32_t len[3] = {half_t, half_h, half_w};
    int32_t off[3] = {0, half_t, half_t + half_h};
    int32_t* table = vit_position_table(grid_thw, num_grids, merge, n_tokens);
    for (int64_t n = 0; n < n_tokens; ++n) {
        for (int32_t a = 0; a < 3; ++a)
            for (int32_t j = 0; j < len[a]; ++j) {
                float theta = (float)((float)table[(int64_t)a * n_tokens + n] * inv[a][j]);
                int64_t idx = ((int64_t)a * n_tokens + n) * half_rot + off[a] + j;
                cos_out[idx] = (float)cos((double)theta);
                sin_out[idx] = (float)sin((double)theta);
            }
    }
    free(table);
}

/* Setup and rotation in one step ([ViT] positions computed arithmetically
 * from the grids, applied as the contiguous t/h/w sections of the rotary
 * pairs): each token's (t, h, w) become a one-token, three-plane position
 * buffer and the per-axis inv_freq a single [R/2] ladder, then the row goes
 * through the same norm and rotation as every other mode. */
void oracle_vit_qk_norm_rope(const float* x, int64_t n_tokens, int32_t heads, int32_t head_dim,
                             const float* weight, float eps, int32_t out_kind, int32_t numerics, int32_t pairing,
                             const float* inv_t, int32_t half_t, const float* inv_h, int32_t half_h,
                             const float* inv_w, int32_t half_w, const int32_t* grid_thw,
                             int32_t num_grids, int32_t merge, float* out)
{
    int32_t half = half_t + half_h + half_w;
    float* inv = (float*)malloc(sizeof(float) * (size_t)(half > 0 ? half : 1));
    for (int32_t j = 0; j < half_t; ++j)
        inv[j] = inv_t[j];
    for (int32_t j = 0; j < half_h; ++j)
        inv[half_t + j] = inv_h[j];
    for (int32_t j = 0; j < half_w; ++j)
        inv[half_t + half_h + j] = inv_w[j];
    double* n = (double*)malloc(sizeof(double) * (size_t)head_dim);
    int32_t* table = vit_position_table(grid_thw, num_grids, merge, n_tokens);
    for (int64_t tok = 0; tok < n_tokens; ++tok) {
        int32_t pos[3] = {table[tok], table[n_tokens + tok], table[2 * n_tokens + tok]};
        oracle_rope rope;
        memset(&rope, 0, sizeof(rope));
        rope.mode = ORACLE_POS_AXES;
        rope.pairing = pairing;
        rope.rotary_dim = 2 * half;
        rope.inv_freq = inv;
        rope.sections[0] = half_t;
        rope.sections[1] = half_h;
        rope.sections[2] = half_w;
        rope.positions = pos;
        rope.pos_stride = 1;
        rope.token_base = 0;
        for (int32_t h = 0; h < heads; ++h) {
            int64_t row = (tok * heads + h) * (int64_t)head_dim;
            norm_rope_row(x + row, weight, head_dim, eps, out_kind, numerics, &rope, 0, n, out + row);
        }
    }
    free(table);
    free(n);
    free(inv);
}
