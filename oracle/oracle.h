/*
 * CPU oracle for per-row RMSNorm fused with rotary position embedding.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load or call this library.  It shares no
 * code, header, table or helper with the HIP library it checks.
 *
 * Conventions
 *   - Activations, weights and outputs travel as float arrays.  A bf16 tensor
 *     is handed over decoded to float (exact), and a bf16 result comes back as
 *     a float that holds a bf16 value.
 *   - Row-major contiguous layouts: x[token][head][dim].
 *   - All arithmetic is in double between the rounding points the method fixes.
 */
#ifndef QK_ROPE_ORACLE_H
#define QK_ROPE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_OUT_F32 = 0, ORACLE_OUT_BF16 = 1, ORACLE_OUT_FP8_E4M3 = 2 };
enum { ORACLE_POS_1D = 0, ORACLE_POS_AXES = 1, ORACLE_POS_IMROPE = 2, ORACLE_POS_PLANES = 3 };
enum { ORACLE_PAIR_NEOX = 0, ORACLE_PAIR_ADJACENT = 1 };
enum { ORACLE_AXIS_T = 0, ORACLE_AXIS_H = 1, ORACLE_AXIS_W = 2, ORACLE_AXIS_E = 3 };
/* Rounding points.  CONTRACT: the normalised value (weight included) rounded
 * once to the output type, the rotation exact, one final rounding.  EAGER: an
 * eager RMSNorm + RoPE chain's points -- fl32(x * fl32(rrms)) rounded to the
 * activation type, times the weight, rounded again; cos and sin rounded to
 * the activation type; every product and sum of the rotation rounded to fp32
 * (no fused multiply-add); the final rounding. */
enum { ORACLE_NUMERICS_CONTRACT = 0, ORACLE_NUMERICS_EAGER = 1 };

typedef struct {
    int32_t mode;            /* ORACLE_POS_*                                         */
    int32_t pairing;         /* ORACLE_PAIR_*                                        */
    int32_t rotary_dim;      /* R: even; elements >= R pass through                  */
    const float* inv_freq;   /* [R/2], one inverse frequency per pair (not PLANES)   */
    int32_t sections[4];     /* AXES/PLANES: pairs per axis, contiguous, t,h,w order;
                                IMROPE: s0..s3 of the sector rule                    */
    const int32_t* positions;/* [n_planes][pos_stride] int32 (not PLANES)            */
    int64_t pos_stride;      /* elements between position planes                     */
    int64_t token_base;      /* first token of this call inside every plane          */
    const float* cos_planes; /* PLANES: [3][planes_tokens][R/2]                      */
    const float* sin_planes;
    int64_t planes_tokens;
} oracle_rope;

/* Round a real to the nearest bf16 value, ties to even. */
double oracle_round_bf16(double v);

/* Plain row RMSNorm: y = round(x * rrms * w), rrms = 1/sqrt(mean(x^2) + eps)
 * (EAGER numerics: y = round(round(fl32(x * fl32(rrms))) * w)). */
void oracle_rms_norm(const float* x, int64_t rows, int32_t width, const float* weight,
                     float eps, int32_t out_kind, int32_t numerics, float* y);

/* OCP FP8 E4M3 ("fn": no infinities, NaN = S.1111.111): value of a code, and
 * the code of a finite real (round half to even, saturating at +-448). */
double oracle_fp8_e4m3_decode(uint8_t code);
uint8_t oracle_fp8_e4m3_encode(double v);

/* Residual add + RMSNorm.  s = x + r rounded once to act_kind (F32 or BF16)
 * is the new residual stream (s_out) and the norm's input; y = s * rrms(s) * w.
 * out_kind F32 / BF16: y rounded once into y_out.  FP8_E4M3: code_out =
 * encode(fl32(fl32(y) / scale)) (a static per-tensor scale).  r == NULL means
 * no residual (s = x).  Unused outputs may be NULL. */
void oracle_add_rms_norm(const float* x, const float* r, int64_t rows, int32_t width, const float* weight,
                         float eps, int32_t act_kind, int32_t out_kind, int32_t numerics, float scale,
                         float* s_out, float* y_out, uint8_t* code_out);

/* Position axis that pair p reads (ORACLE_AXIS_*). */
int32_t oracle_axis(const oracle_rope* rope, int32_t p);

/* Per-(token, head) RMSNorm followed by the rotation of every pair.
 * x, out: [tokens][heads][head_dim].  rope == NULL or rotary_dim == 0 means
 * norm only. */
void oracle_qk_norm_rope(const float* x, int64_t tokens, int32_t heads, int32_t head_dim,
                         const float* weight, float eps, int32_t out_kind, int32_t numerics,
                         const oracle_rope* rope, float* out);

/* QK RMSNorm + RoPE with the K rows written into a cache: Q as
 * oracle_qk_norm_rope into q_out [tokens][q_heads][d]; the rotated K rows of
 * token t and its V rows (copied unchanged) go to row slots[t] of k_cache and
 * v_cache [num_slots][kv_heads][d]; a slot outside [0, num_slots) writes
 * nothing, and cache rows no token maps to are left as they are.  v and
 * v_cache may be NULL together. */
void oracle_qk_norm_rope_cache(const float* q, int32_t q_heads, const float* k, const float* v,
                               int32_t kv_heads, int64_t tokens, int32_t head_dim, const float* q_weight,
                               const float* k_weight, float eps, int32_t out_kind, int32_t numerics,
                               const oracle_rope* rope, const int64_t* slots, int64_t num_slots, float* q_out,
                               float* k_cache, float* v_cache);

/* Joint text/image op: each stream is normalised with its own weights, the
 * streams are concatenated text first and the joint sequence is rotated with
 * positions indexed by joint token.  V rows are copied unchanged.
 * Stream inputs: [batch][tokens_s][heads][head_dim]; outputs:
 * [batch][tokens_txt + tokens_img][heads][head_dim]. */
void oracle_joint_qk_norm_rope(int32_t batch, int32_t heads, int32_t head_dim,
                               const float* q_txt, const float* k_txt, const float* v_txt,
                               int64_t tokens_txt, const float* qw_txt, const float* kw_txt,
                               const float* q_img, const float* k_img, const float* v_img,
                               int64_t tokens_img, const float* qw_img, const float* kw_img,
                               float eps, int32_t out_kind, int32_t numerics, const oracle_rope* rope,
                               float* q_out, float* k_out, float* v_out);

/* ViT patch positions: pos[3][n_tokens] = (t, h, w) of every token of the
 * grids [num_grids][3] (t, h, w patch counts) under spatial merge m. */
void oracle_vit_positions(const int32_t* grid_thw, int32_t num_grids, int32_t merge,
                          int32_t* pos, int64_t n_tokens);

/* ViT cos/sin planes [3][n_tokens][half_t + half_h + half_w]; plane a holds
 * only axis a's columns, the rest is left untouched. */
void oracle_vit_cos_sin(const float* inv_t, int32_t half_t, const float* inv_h, int32_t half_h,
                        const float* inv_w, int32_t half_w, const int32_t* grid_thw,
                        int32_t num_grids, int32_t merge, float* cos_out, float* sin_out,
                        int64_t n_tokens);

/* ViT QK RMSNorm + RoPE with positions taken from the patch grids (the setup
 * and the rotation in one step, no cos/sin planes): pair p of token n reads
 * axis a by contiguous sections (half_t, half_h, half_w) and rotates by
 * fl32(fl32(pos_a(n)) * inv_a[p - off_a]).  x, out: [n_tokens][heads][head_dim];
 * rotary_dim = 2 * (half_t + half_h + half_w). */
void oracle_vit_qk_norm_rope(const float* x, int64_t n_tokens, int32_t heads, int32_t head_dim,
                             const float* weight, float eps, int32_t out_kind, int32_t numerics,
                             int32_t pairing,
                             const float* inv_t, int32_t half_t, const float* inv_h, int32_t half_h,
                             const float* inv_w, int32_t half_w, const int32_t* grid_thw,
                             int32_t num_grids, int32_t merge, float* out);

#ifdef __cplusplus
}
#endif
#endif
