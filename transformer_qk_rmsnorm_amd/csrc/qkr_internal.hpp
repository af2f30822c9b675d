// Internal interface between the C-ABI host layer (qkr_api.cpp) and the
// gfx950 kernels (qkr_kernels.hip).  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qkr_fastdiv.hpp"

namespace qkr {

constexpr int kMaxGrids = 64;     // ViT grids per setup launch (metadata rides in kernel arguments)
constexpr int kMaxFusedGrids = 32; // ViT grids per fused norm + rotation launch
constexpr int kThreads = 256;     // threads per workgroup of the row kernels (4 waves)
// Workgroups per launch.  A dispatch counts its work-items in 32 bits; calls
// that need more workgroups take several launches, each told its first tile
// or row.
constexpr int64_t kMaxBlocksPerLaunch = (int64_t)1 << 23;

enum PosMode : int32_t { kPos1D = 0, kPosAxes = 1, kPosImrope = 2, kPosPlanes = 3, kPosNone = 4, kPosVit = 5 };
enum Pairing : int32_t { kNeox = 0, kAdjacent = 1 };
enum Dtype : int32_t { kF32 = 0, kBF16 = 1 };

constexpr int kMaxPairs = 128;    // rotary_dim / 2 <= head_dim / 2 <= 128

// Rotation parameters as the kernels read them.
struct RopeArgs {
    int32_t mode;        // PosMode
    int32_t half;        // R / 2
    int32_t sec[4];      // raw sections (AXES/PLANES: pairs per axis; IMROPE: s0..s3)
    alignas(16) uint32_t axis_bits[kMaxPairs / 16];   // axis of pair p: bits 2(p%16).. of word p/16 (host-built)
    const float* inv_freq;
    const int32_t* positions;
    int64_t pos_stride;
    int64_t plane_off[4];                 // element offset of the t, h, w, e position planes
    int64_t token_base;
    const float* cos_planes;
    const float* sin_planes;
    int64_t planes_tokens;
};

// ViT patch grids for the fused mode: positions are computed per token from
// the grid table (absolute token offsets) with host-computed divisors.
struct VitGridArgs {
    int32_t num_grids;
    int32_t merge;
    FastDiv div_m;                       // merge
    FastDiv div_mm;                      // merge * merge
    int64_t cu[kMaxFusedGrids + 1];      // first token of each grid, then the end
    FastDiv div_area[kMaxFusedGrids];    // h * w of each grid
    FastDiv div_bcols[kMaxFusedGrids];   // w / merge (merge blocks per block row) of each grid
    const float* inv[3];                 // per-axis inverse frequencies
};

// One of Q, K, V.  Input views exist per stream (stream 1 only for the joint
// op); strides are in bytes.  weight == nullptr marks a copied tensor (V); a
// tensor with heads == 0 takes no work.
struct StreamView {
    const char* in;
    int64_t sb, st, sh;         // batch, token and head strides
    const char* weight;
};
struct TensorArgs {
    StreamView s[2];            // one indexed load fetches a stream's fields
    char* out;
    int64_t out_sb, out_st, out_sh;
    const int64_t* slots;       // non-null: token t's rows go to output row slots[t] (stride out_st)
    int64_t nslots;             // slots outside [0, nslots) write nothing
    int32_t heads;
};

// A tile is one wavefront's work: up to rows_per_tile heads of one tensor of
// one token.  Tiles of a token are numbered tensor by tensor.
struct NormRopeArgs {
    TensorArgs t[3];
    int32_t batch;
    int32_t tokens;             // tokens per batch (joint count for the joint op)
    int32_t tokens0;            // tokens of stream 0; tokens at or past it belong to stream 1
    int32_t head_dim;
    int32_t rotary_dim;
    uint32_t ntiles;            // batch * tokens * tiles per token (< 2^31), set by the launcher
    uint32_t tile_base;         // first tile of this launch (set by the launcher)
    int32_t tile_first[3];      // first tile of tensors 0, 1, 2 within a token (set by the launcher)
    FastDiv div_tpt;            // tiles per token
    FastDiv div_tokens;         // tokens per batch
    float eps;
    float inv_d;                // 1 / head_dim
    uint32_t nv_recip;          // ceil(2^16 / vectors per row): row of a staged vector
    RopeArgs rope;
    VitGridArgs vit;            // kPosVit only
};

struct RmsArgs {
    const char* x;
    char* y;
    const char* w;
    const char* r;              // residual (add modes)
    char* s;                    // new residual stream (add modes)
    const float* scale;         // static FP8 scale (FP8 mode)
    int64_t x_stride;           // bytes
    int64_t y_stride;           // bytes
    int64_t r_stride;           // bytes
    int64_t s_stride;           // bytes
    int64_t rows;
    int64_t item_base;          // first row (split: first row slice) of this launch, set by the launcher
    int32_t nvec;               // 16-byte vectors per row
    int32_t splits;             // workgroups per row (split variant)
    int32_t split_len;          // vectors stored by one split
    FastDiv div_splits;
    float eps;
    float inv_width;
};

// ViT setup (and position map) launch over at most kMaxGrids grids.  Token
// counts stay below 2^31, so positions are found with 32-bit arithmetic and
// host-built divisors.
struct VitArgs {
    const float* inv[3];
    float* cos_out;
    float* sin_out;
    int64_t n_tokens;           // tokens in the whole output planes
    int64_t tok_begin;          // first token this launch covers
    int64_t tok_count;          // tokens this launch covers
    int32_t half[3];
    int32_t off[3];
    int32_t half_rot;
    int32_t merge;
    int32_t num_grids;          // grids in this launch
    int32_t vec_ok;             // whole 4-column groups may leave as 16-byte stores (host-checked)
    uint32_t cu[kMaxGrids + 1]; // token offsets of this launch's grids (absolute)
    FastDiv div_area[kMaxGrids];   // h * w of each grid
    FastDiv div_bcols[kMaxGrids];  // w / merge of each grid
    FastDiv div_m, div_mm;         // merge, merge^2
    FastDiv div_groups;            // 4-column groups per token: ceil(half_rot / 4)
};

// Axis of pair p (0 t, 1 h, 2 w, 3 e).  Host and device share this one
// definition so the host can be checked without a GPU.
//   IMROPE: pairs repeat with period S = s0 + s1 + s2 + s3.  At offset
//     o = p mod S, the residue o mod 3 names an axis (t, h, w) and o div 3
//     counts that axis's pairs so far in the period: the pair belongs to the
//     axis while the count is below the axis's section, otherwise to e.
//   AXES / PLANES: contiguous runs of s0 (t), s1 (h) and the rest (w).
__host__ __device__ inline int32_t pair_axis(int32_t mode, const int32_t* sec, int32_t p)
{
    if (mode == kPosImrope) {
        const int32_t o = p % (sec[0] + sec[1] + sec[2] + sec[3]);
        const int32_t axis = o % 3, count = o / 3;
        const int32_t limit = axis == 0 ? sec[0] : (axis == 1 ? sec[1] : sec[2]);
        return count < limit ? axis : 3;
    }
    if (mode == kPosAxes || mode == kPosPlanes) {
        if (p < sec[0]) return 0;
        if (p < sec[0] + sec[1]) return 1;
        return 2;
    }
    return 0;
}

// The axis table of the rotation kernels: 2 bits per pair, pair p in bits
// 2 (p % 16) and up of word p / 16.  Pairs past n_pairs read axis 0.
inline void build_axis_bits(int32_t mode, const int32_t* sec, int32_t n_pairs, uint32_t* bits)
{
    for (int i = 0; i < kMaxPairs / 16; ++i)
        bits[i] = 0;
    for (int32_t p = 0; p < n_pairs && p < kMaxPairs; ++p)
        bits[p >> 4] |= (uint32_t)pair_axis(mode, sec, p) << ((p & 15) * 2);
}

// (t, h, w) of ViT token `tok`.  Its grid is the last one whose first token
// it has reached (grids are non-empty).  Inside the grid, a frame holds h * w
// tokens; inside a frame, tokens come in merge blocks of m * m cells, the
// blocks numbered in raster order over the (h / m) x (w / m) block grid and
// the cells row by row: frame-local index = block * m^2 + cell.  The grid is
// picked by a select loop over the launch's grids; the divisions use the
// host's divisors.  Host and device share this one definition.
__host__ __device__ inline void vit_position(const VitArgs& a, uint32_t tok, int32_t* tpos, int32_t* hpos,
                                             int32_t* wpos)
{
    uint32_t start = a.cu[0];
    FastDiv d_frame = a.div_area[0], d_bcols = a.div_bcols[0];
    for (int32_t k = 1; k < a.num_grids; ++k) {
        // Every field of grid k is read before the choice: a choice between a
        // field and the value so far is otherwise compiled into a branch
        // around that field's load (tokens differ per lane), with a wait of
        // its own for each field.
        uint32_t ck = a.cu[k], ad = a.div_area[k].d, am = a.div_area[k].m, as = a.div_area[k].sh;
        uint32_t bd = a.div_bcols[k].d, bm = a.div_bcols[k].m, bs = a.div_bcols[k].sh;
#if defined(__HIP_DEVICE_COMPILE__)
        asm("" : "+s"(ck), "+s"(ad), "+s"(am), "+s"(as), "+s"(bd), "+s"(bm), "+s"(bs));
#endif
        const bool in_k = tok >= ck;
        start = in_k ? ck : start;
        d_frame.d = in_k ? ad : d_frame.d;
        d_frame.m = in_k ? am : d_frame.m;
        d_frame.sh = in_k ? as : d_frame.sh;
        d_bcols.d = in_k ? bd : d_bcols.d;
        d_bcols.m = in_k ? bm : d_bcols.m;
        d_bcols.sh = in_k ? bs : d_bcols.sh;
    }
    const uint32_t local = tok - start;
    const uint32_t frame = fast_div(local, d_frame);
    const uint32_t in_frame = local - frame * d_frame.d;
    const uint32_t block = fast_div(in_frame, a.div_mm);
    const uint32_t cell = in_frame - block * a.div_mm.d;
    const uint32_t brow = fast_div(block, d_bcols);
    const uint32_t crow = fast_div(cell, a.div_m);
    *tpos = (int32_t)frame;
    *hpos = (int32_t)(brow * a.div_m.d + crow);
    *wpos = (int32_t)((block - brow * d_bcols.d) * a.div_m.d + (cell - crow * a.div_m.d));
}

// QK RMSNorm + RoPE kernel for one lanes-per-row value (LPR in 1, 2, 4, 8, 16,
// 32), chosen by element type, rotation source (0 none, 1 positions, 2
// planes, 3 ViT grids), pairing, nontemporal accesses, staged stores, the
// eager numerics and passes per wave.  Each (LPR, EAGER) pair is defined in its own build of
// qkr_rope_part.hip.
using NormRopeFn = void (*)(NormRopeArgs);
template <int LPR, bool EAGER>
NormRopeFn pick_norm_rope(int32_t dtype, int rope, int32_t pairing, bool nt, bool stage, int np);
// Token-tile kernel (one wavefront per token, Q and K rows together) for L
// lanes per row, L in 3, 5, 6, 7; each (L, EAGER) pair is defined in its own
// build of qkr_token_part.hip.
template <int L, bool EAGER>
NormRopeFn pick_norm_rope_token(int32_t dtype, int rope, int32_t pairing, bool nt);
// Most row vectors of one token the token-tile kernel holds (Q and K rows).
constexpr int kTokenTileVecs = 320;

// Kernel variant of a QK norm + rotation call.
struct RopePlan {
    int lpr;     // lanes per row
    int np;      // passes (row groups) per wave
    bool stage;  // stores through LDS in contiguous runs
    bool nt;     // nontemporal row accesses
    int token;   // lanes per row of the token-tile kernel; 0: the tile kernel
    int waves_cap;   // tile kernel: most waves per SIMD (0: none), held by reserving LDS
};

// Kernel variant of a row norm call.
struct RmsPlan {
    int kind;    // 0 rows, 1 split, 2 wide
    int vpl;     // 16-byte vectors per lane
    bool nt;
    int mode;    // bit 0 residual add, bit 1 FP8 E4M3 output
};

// Variant choice, pure host code.  Requests: np / lpr 0 = automatic, stage
// -1 = automatic, kind -1 = automatic; nt 1 nontemporal, 0 plain.  Returns
// nullptr, or (static text) why a forced choice cannot run the call: a
// forced variant is never replaced by another.
// planes: cos/sin come from planes (the PLANES mode); token_ok: the call has
// no V tensor, no slot map and one stream, and each tensor's rows of one
// token span less than 2^31 bytes (what the token-tile kernel takes);
// token_req -1 automatic, 0 the tile kernel, 1 the token-tile kernel.
const char* plan_norm_rope(int32_t dtype, int32_t head_dim, const int32_t heads[3], int32_t half, bool planes,
                           bool token_ok, int np_req, int lpr_req, int stage_req, int token_req, int nt_req,
                           RopePlan* plan);
const char* plan_rms_norm(int32_t nvec, int64_t rows, int kind_req, int nt_req, int mode, RmsPlan* plan);

// Kernel launchers (qkr_kernels.hip).  Each returns the variant name it
// launched through *variant; launch errors surface through hipGetLastError.
// eager: the eager-chain rounding points instead of the contract.
hipError_t launch_norm_rope(const NormRopeArgs& a, int32_t dtype, int32_t pairing, bool eager, const RopePlan& plan,
                            hipStream_t stream, const char** variant);
hipError_t launch_rms_norm(RmsArgs a, int32_t dtype, bool eager, const RmsPlan& plan, hipStream_t stream,
                           const char** variant);
hipError_t launch_debug_fp8(const float* x, int64_t n, const float* scale, uint8_t* out, hipStream_t stream);
hipError_t launch_vit_setup(const VitArgs& a, hipStream_t stream);
hipError_t launch_debug_axis_map(const RopeArgs& r, int32_t n_pairs, int32_t* out, hipStream_t stream);
hipError_t launch_debug_vit_positions(const VitArgs& a, int32_t* out, hipStream_t stream);

}  // namespace qkr
