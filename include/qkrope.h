/*
 * qkrope: per-(token, head) RMSNorm fused with rotary position embedding on
 * attention Q/K, for AMD Instinct MI355X (gfx950).  C ABI.
 *
 * The operations come from these pages (cited by the short name in brackets):
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
 * Conventions shared by every entry point
 *   - Pointers named *_dev are device (HBM) pointers; grid_thw is a host
 *     pointer.  The caller owns every buffer, outputs included; the library
 *     allocates nothing and keeps no state between calls.
 *   - Strides are in elements.  The last (head_dim / width) dimension is
 *     contiguous.  Every base pointer must be 16-byte aligned and every stride
 *     a multiple of 16 bytes (rows are moved as 128-bit vectors); otherwise
 *     QKR_ERR_MISALIGNED.  Offsets are computed in 64 bits, so views deep
 *     inside buffers larger than 4 GiB are fine ([Ovis] 64-bit row
 *     addressing).
 *   - Size limits: one call covers fewer than 2^31 rows (batch x tokens x
 *     heads, or `rows`) and at most 2^20 heads, and every view, row set,
 *     position or cos/sin plane it touches spans at most 2^48 bytes (the
 *     GPU's virtual address space); every stride, used or not, lies within
 *     +-2^48 bytes.  The checks cannot overflow; a call beyond them returns
 *     QKR_ERR_UNSUPPORTED.
 *   - Activations, weights and outputs share `dtype`.  Positions are int32,
 *     inverse frequencies and cos/sin planes are fp32.
 *   - `stream` is the caller's HIP stream (NULL: the null stream).  Work is
 *     enqueued asynchronously; nothing synchronises the host.
 *   - Arguments are validated on the host before any HIP call.  A refusal
 *     returns a non-zero qkr_status, launches nothing and leaves a message for
 *     qkr_last_error() (per calling thread).  There is no fallback path.
 *   - Input and output rows may alias exactly (same pointer and strides: each
 *     row is read whole before it is written); partial overlap is undefined.
 *   - Results are deterministic: fixed launch shape, no atomics.
 */
#ifndef QKROPE_H
#define QKROPE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t;
typedef struct ihipStream_t* qkr_stream_t; /* a hipStream_t */

typedef enum {
    QKR_OK = 0,
    QKR_ERR_INVALID_ARGUMENT = 1, /* a size, pointer, mode or section is out of range */
    QKR_ERR_UNSUPPORTED = 2,      /* valid, but a geometry this library does not run   */
    QKR_ERR_MISALIGNED = 3,       /* a pointer or stride is not 16-byte aligned        */
    QKR_ERR_HIP = 4               /* the HIP runtime refused the launch                */
} qkr_status;

typedef enum { QKR_F32 = 0, QKR_BF16 = 1 } qkr_dtype;

/* Rounding points, OR-ed into the dtype argument of every entry point that
 * takes one (dtype = QKR_BF16 | QKR_NUMERICS_EAGER):
 *   QKR_NUMERICS_CONTRACT (the default): the normalised value, weight
 *     included, rounded once to the activation type; the rotation in fp32;
 *     one final rounding ([Ovis] kernel review: the documented rounding
 *     contract).  qkr_rms_norm: one rounding of x * rrms * w.
 *   QKR_NUMERICS_EAGER: the rounding points of an eager RMSNorm + RoPE chain
 *     ([Ovis] "Supplemental eager bitwise measurements": a preset that turns
 *     floating-point fusion off and reproduced such a chain bit for bit;
 *     [VecRMS] review thread: that chain's RMSNorm output expression
 *     ((scalar_t)(x * s_variance)) * weight): x * rrms rounded to the
 *     activation type, times the weight, rounded again; cos and sin computed
 *     in fp32 and rounded to the activation type (the chain's RoPE table);
 *     every product and sum of the rotation rounded to fp32 on its own (no
 *     fused multiply-add); one final rounding.  It fixes the rounding points
 *     only: the sum of squares and the reciprocal square root stay this
 *     library's, so bit-for-bit equality with another library's chain is not
 *     promised.  Not defined for FP8 outputs (QKR_ERR_UNSUPPORTED).
 * Any other bit above the low byte is refused (QKR_ERR_INVALID_ARGUMENT). */
typedef enum { QKR_NUMERICS_CONTRACT = 0, QKR_NUMERICS_EAGER = 0x100 } qkr_numerics;

/* Rotary pairing.  NEOX pairs element p with p + R/2 ([IMROPE]: the sectioned
 * mode keeps the NeoX pairing); ADJACENT pairs 2p with 2p + 1 ([Ovis]:
 * interleaved=True). */
typedef enum { QKR_PAIR_NEOX = 0, QKR_PAIR_ADJACENT = 1 } qkr_pairing;

/* Where pair p takes its position.
 *   1D      one position plane.
 *   AXES    sections[0..2] contiguous runs of pairs read planes t, h, w
 *           ([Ovis] multi-axis image positions; [ViT] t/h/w column ranges).
 *   IMROPE  interleaved multi-section rule of [IMROPE] ("The change"):
 *           sector = p mod (s0+s1+s2+s3); sector mod 3 == 1 -> h while
 *           sector < 3 s1, == 2 -> w while sector < 3 s2, == 0 -> t while
 *           sector < 3 s0, else the fourth plane e.
 *   PLANES  cos/sin come from (3, planes_tokens, R/2) fp32 planes written by
 *           qkr_mrope_cos_sin_setup; pair p reads the plane of its axis, the
 *           axes being contiguous runs of sections[0..2] pairs ([ViT]). */
typedef enum { QKR_POS_1D = 0, QKR_POS_AXES = 1, QKR_POS_IMROPE = 2, QKR_POS_PLANES = 3 } qkr_pos_mode;

/* Rotary embedding parameters.  The angle of pair p at token t is
 * fl32(fl32(pos) * inv_freq[p]) with pos = positions[axis * pos_stride +
 * token_base + t]; cos and sin are computed in registers, never read from a
 * cache (except in PLANES mode).  A call over a chunk of a longer sequence
 * passes the whole-length position planes and its first token in token_base
 * ([IMROPE] "The change": chunked launches keep the whole positions buffer). */
typedef struct {
    int32_t mode;               /* qkr_pos_mode                                            */
    int32_t pairing;            /* qkr_pairing                                             */
    int32_t rotary_dim;         /* R: even, 0 <= R <= head_dim; 0 = norm only              */
    int32_t sections[4];        /* AXES/PLANES: pairs on t, h, w (sum R/2, [3] = 0);
                                   IMROPE: s0..s3 with R/2 <= sum <= R ([IMROPE] claim
                                   window); unused otherwise                               */
    const float* inv_freq_dev;  /* [R/2] fp32 (1D, AXES, IMROPE)                           */
    const int32_t* positions_dev; /* [planes][pos_stride] int32: 1 plane (1D), 3 (AXES),
                                     4 (IMROPE)                                            */
    int64_t pos_stride;         /* elements between planes; >= token_base + tokens         */
    int64_t token_base;         /* first token of this call inside every plane, >= 0       */
    const float* cos_planes_dev; /* PLANES: [3][planes_tokens][R/2] fp32                   */
    const float* sin_planes_dev;
    int64_t planes_tokens;      /* PLANES: tokens per plane; >= token_base + tokens        */
} qkr_rope;

/* A [batch, tokens, heads, head_dim] tensor of rows. */
typedef struct {
    void* ptr_dev;        /* element (0, 0, 0, 0)                                          */
    int64_t stride_batch; /* elements between batches (ignored when batch == 1)            */
    int64_t stride_tok;   /* elements between tokens                                       */
    int64_t stride_head;  /* elements between heads                                        */
} qkr_view;

/* Plain row RMSNorm ([Vulkan] decode RmsNorm; [VecRMS]):
 *   y[r, i] = round(x[r, i] * rrms_r * weight[i]),
 *   rrms_r = 1 / sqrt(mean_i(x[r, i]^2) + eps), sum of squares in fp32,
 * one rounding to the output type.  x, y: [rows, width] with row strides in
 * elements; weight: [width].  rows == 0 is a no-op.  From 2048 to 4096 rows
 * (and for rows of fewer than 64 16-byte vectors) each row runs on one
 * wavefront, otherwise on a workgroup of four wavefronts. */
qkr_status qkr_rms_norm(const void* x_dev, int64_t x_row_stride, void* y_dev, int64_t y_row_stride,
                        const void* weight_dev, int64_t rows, int32_t width, float eps,
                        int32_t dtype, qkr_stream_t stream);

/* Output kinds of qkr_add_rms_norm. */
typedef enum { QKR_OUT_ACT = 0, QKR_OUT_FP8_E4M3 = 1 } qkr_out_kind;

/* Residual add + RMSNorm, with the output in the activation type or as static
 * FP8 codes ([Vulkan] decode RmsNorm: its calls carry the residual add and the
 * weight multiply, and the residual stream is held bit-exactly by rounding the
 * sum in registers; [VecRMS]: the static FP8 RMSNorm kernel):
 *   s[r, i] = round(x[r, i] + res[r, i])          the new residual stream -> s_dev
 *   y[r, i] = s[r, i] * rrms_r * weight[i],  rrms_r = 1 / sqrt(mean_i(s[r, i]^2) + eps)
 *   y_kind QKR_OUT_ACT:      y rounded once to the activation type
 *   y_kind QKR_OUT_FP8_E4M3: one byte per element, the OCP E4M3 code of the
 *                            correctly rounded fp32 quotient y / *scale_dev
 *                            (round half to even, saturating at +-448)
 * x, res, s: [rows, width] of dtype with row strides in elements; y: row
 * stride in elements of its own type (bytes for FP8).  res_dev == NULL means
 * no add (s_dev must then be NULL too: plain RMSNorm with the chosen output).
 * s may be res or x itself (same pointer and stride: in-place update of the
 * residual stream); no other overlap of s or y with the inputs is accepted.
 * scale_dev: device fp32 scalar, read by the kernel (FP8 only); the caller
 * keeps it finite and positive.  Inputs are finite.  FP8 rows need y aligned
 * to 16 / sizeof(dtype) bytes.  Refusals as for qkr_rms_norm. */
qkr_status qkr_add_rms_norm(const void* x_dev, int64_t x_row_stride, const void* res_dev, int64_t res_row_stride,
                            void* s_dev, int64_t s_row_stride, void* y_dev, int64_t y_row_stride, int32_t y_kind,
                            const float* scale_dev, const void* weight_dev, int64_t rows, int32_t width, float eps,
                            int32_t dtype, qkr_stream_t stream);

/* Per-(token, head) RMSNorm of Q and K followed by RoPE ([Ovis] single-stream
 * fused_qk_norm_rope; [IMROPE] sectioned rotation after the per-head norm):
 *   n = x * rrms * w over each head_dim row (fp32 sum of squares);
 *   bf16: n is rounded to bf16, rotated in fp32, rounded once more ([Ovis]
 *   kernel review: the documented rounding contract); fp32: no intermediate
 *   rounding.  Elements at or past rotary_dim pass through normalised.
 * q/q_out: q_heads rows per token with weight q_weight [head_dim]; likewise
 * k.  Either tensor may be absent (heads == 0).  rope == NULL: norm only.
 * Positions are indexed by token (shared across the batch). */
qkr_status qkr_qk_norm_rope(int32_t batch, int64_t tokens, int32_t head_dim, int32_t dtype, float eps,
                            const qkr_view* q, const qkr_view* q_out, int32_t q_heads,
                            const void* q_weight_dev,
                            const qkr_view* k, const qkr_view* k_out, int32_t k_heads,
                            const void* k_weight_dev,
                            const qkr_rope* rope, qkr_stream_t stream);

/* QK RMSNorm + RoPE with K written into a cache ([IMROPE] "The change": the
 * rotation kernel's set_rows twin, which stores each rotated row into the row
 * an index picks):
 *   q_out  = the qk_norm_rope result for q (batch 1: views' stride_batch unused);
 *   token t's rotated K rows (all kv_heads) -> row slot_mapping_dev[t] of k_cache,
 *   token t's V rows, copied unchanged      -> the same row of v_cache.
 * k_cache / v_cache are qkr_views over [num_slots][kv_heads][head_dim] (stride_tok
 * = elements between slots, e.g. a paged [blocks][block_size][H][D] cache seen
 * as blocks * block_size slots).  slot_mapping_dev: device int64 [tokens]; a
 * slot outside [0, num_slots) writes nothing (e.g. -1 for padding tokens);
 * two tokens mapped to one slot leave that slot's content unspecified; cache
 * rows no token maps to are untouched.  v and v_cache are both NULL or both
 * given.  The caches must not overlap the inputs or q_out.  Refusals as for
 * qkr_qk_norm_rope, plus a null or misaligned slot mapping. */
qkr_status qkr_qk_norm_rope_cache(int64_t tokens, int32_t head_dim, int32_t dtype, float eps, const qkr_view* q,
                                  const qkr_view* q_out, int32_t q_heads, const void* q_weight_dev,
                                  const qkr_view* k, const qkr_view* v, int32_t kv_heads, const void* k_weight_dev,
                                  const qkr_view* k_cache, const qkr_view* v_cache,
                                  const int64_t* slot_mapping_dev, int64_t num_slots, const qkr_rope* rope,
                                  qkr_stream_t stream);

/* One stream (text or image) of the joint op: Q, K, V views of `tokens`
 * tokens (e.g. chunked views of one packed QKV projection) and the stream's
 * own q/k norm weights [head_dim]. */
typedef struct {
    qkr_view q, k, v;
    int64_t tokens;
    const void* q_weight_dev;
    const void* k_weight_dev;
} qkr_stream;

/* Joint text/image QK RMSNorm + concatenation + RoPE ([Ovis] "Purpose":
 * fused_joint_qkv_norm_rope).  Each stream is normalised with its own
 * weights; outputs are the joint [batch, text.tokens + image.tokens, heads,
 * head_dim] Q, K and V, text first; the rotation reads positions by joint
 * token; V rows are copied bit for bit. */
qkr_status qkr_joint_qk_norm_rope(int32_t batch, int32_t heads, int32_t head_dim, int32_t dtype,
                                  float eps, const qkr_stream* text, const qkr_stream* image,
                                  const qkr_view* q_out, const qkr_view* k_out,
                                  const qkr_view* v_out, const qkr_rope* rope,
                                  qkr_stream_t stream);

/* ViT multi-axis cos/sin setup ([ViT] VitMropeSetup / _vit_mrope_setup_kernel).
 * For token n of the grids grid_thw[g] = (t, h, w) (host array, num_grids
 * entries, tokens of grid g following those of grid g-1), the (t, h, w)
 * position comes from the spatial-merge token order; plane a receives
 * cos/sin of fl32(fl32(pos_a) * inv_freq_a[j]) in its own columns
 * [off_a, off_a + half_a) of the (3, n_tokens, half_t + half_h + half_w) fp32
 * outputs.  Other columns are not written.  n_tokens must equal sum t*h*w;
 * h and w must be multiples of spatial_merge.  The grid table travels in
 * kernel arguments (no host-to-device copy). */
qkr_status qkr_mrope_cos_sin_setup(const float* inv_freq_t_dev, int32_t half_t,
                                   const float* inv_freq_h_dev, int32_t half_h,
                                   const float* inv_freq_w_dev, int32_t half_w,
                                   const int32_t* grid_thw, int32_t num_grids,
                                   int32_t spatial_merge, float* cos_out_dev, float* sin_out_dev,
                                   int64_t n_tokens, qkr_stream_t stream);

/* ViT per-head QK RMSNorm + RoPE with the cos/sin setup folded in: the
 * (t, h, w) position of every token comes from the patch grids (host array
 * grid_thw[num_grids][3], spatial merge order, as in qkr_mrope_cos_sin_setup)
 * and pair p rotates by fl32(fl32(pos_a) * inv_freq_a[p - off_a]) for the
 * contiguous t/h/w sections (half_t, half_h, half_w pairs), cos and sin
 * computed in registers: no planes are written or read and there is no setup
 * launch ([ViT]: positions computed arithmetically from the grids, no cos/sin
 * cache).  rotary_dim = 2 (half_t + half_h + half_w) <= head_dim.  Q and K are
 * [tokens, heads, head_dim] views with tokens = sum t*h*w; the rounding
 * contract is that of qkr_qk_norm_rope.  More than 32 grids take several
 * launches. */
qkr_status qkr_vit_qk_norm_rope(int64_t tokens, int32_t head_dim, int32_t dtype, float eps,
                                const qkr_view* q, const qkr_view* q_out, int32_t q_heads,
                                const void* q_weight_dev,
                                const qkr_view* k, const qkr_view* k_out, int32_t k_heads,
                                const void* k_weight_dev, int32_t pairing,
                                const float* inv_freq_t_dev, int32_t half_t,
                                const float* inv_freq_h_dev, int32_t half_h,
                                const float* inv_freq_w_dev, int32_t half_w,
                                const int32_t* grid_thw, int32_t num_grids, int32_t spatial_merge,
                                qkr_stream_t stream);

/* Text of a status code (static storage). */
const char* qkr_status_string(qkr_status status);

/* Detail of the last refusal on the calling thread ("" if none). */
const char* qkr_last_error(void);

/* ---- Introspection and test hooks (not for the hot path) ---------------- */

/* Force a kernel variant by name for subsequent calls on any thread, or NULL
 * for the automatic choice ([Vulkan] PR description: an override forces a
 * module so that every arm runs on every machine).  Names: "rms:rows",
 * "rms:split", "rms:wide", "rope:np1", "rope:np2", "rope:np3", "rope:np4"
 * (passes of rows per wavefront), "rope:lpr4", "rope:lpr8", "rope:lpr16",
 * "rope:lpr32" (lanes per row), "rope:stage0" / "rope:stage1" (QK stores
 * straight from registers / through LDS in contiguous runs), "rope:tile" /
 * "rope:token" (the QK tile kernel / token tiles: one wavefront per token,
 * Q and K rows together, for rows of 5, 6 or 9 to 14 16-byte vectors),
 * "nt:0" / "nt:1" (plain / nontemporal row accesses).  Overrides accumulate
 * until NULL resets all of them.  Unknown names are refused.  A forced
 * variant is never swapped for another: a call it cannot run (a row longer
 * than one wavefront holds under "rms:rows" or "rms:split", the residual add
 * under "rms:split", too few lanes per row for the head_dim, staged stores
 * outside 2 to 8 lanes per row, token tiles with another row width, with V,
 * a slot map, two streams, more than 320 Q and K row vectors per token, or
 * with a tile-kernel choice (passes, lanes per row, staging) forced too)
 * returns QKR_ERR_UNSUPPORTED before any HIP call. */
qkr_status qkr_set_variant_override(const char* name);

/* Name of the kernel variant the last successful launch on the calling
 * thread used ("" if none) ([Vulkan] PR description: the test pins the
 * module by name through the dispatch record). */
const char* qkr_debug_last_variant(void);

/* The same text as qkr_debug_last_variant (earlier name, kept). */
const char* qkr_last_variant(void);

/* The position axis (0 t, 1 h, 2 w, 3 e) of each of n_pairs (<= 128) pairs
 * under `rope`, as the kernels see it: the host-built axis table they receive,
 * decoded by the same device function, written to out_dev [n_pairs] int32.
 * Only rope->mode and rope->sections are read; each section must lie in
 * [0, 2^20] (QKR_ERR_INVALID_ARGUMENT otherwise), with a positive sum for
 * IMROPE. */
qkr_status qkr_debug_axis_map(const qkr_rope* rope, int32_t n_pairs, int32_t* out_dev,
                              qkr_stream_t stream);

/* The (t, h, w) position of every ViT token, computed by the same device
 * function the setup kernel uses, written to out_dev [3][n_tokens] int32.
 * n_tokens must equal the sum of t*h*w, which stays below 2^31. */
qkr_status qkr_debug_vit_positions(const int32_t* grid_thw, int32_t num_grids, int32_t spatial_merge,
                                   int32_t* out_dev, int64_t n_tokens, qkr_stream_t stream);

/* The FP8 E4M3 quantiser of qkr_add_rms_norm applied to x_dev [n] fp32:
 * out_dev [n] uint8 = code(x / *scale_dev) with the kernel's quotient, or
 * code(x) when scale_dev is NULL.  n < 2^31. */
qkr_status qkr_debug_fp8_e4m3(const float* x_dev, int64_t n, const float* scale_dev, uint8_t* out_dev,
                              qkr_stream_t stream);

/* Host builds of the same two index functions (no GPU needed): out_host
 * [n_pairs] and [3][n_tokens] int32. */
qkr_status qkr_axis_map_host(const qkr_rope* rope, int32_t n_pairs, int32_t* out_host);
qkr_status qkr_vit_positions_host(const int32_t* grid_thw, int32_t num_grids, int32_t spatial_merge,
                                  int32_t* out_host, int64_t n_tokens);

#ifdef __cplusplus
}
#endif
#endif /* QKROPE_H */
