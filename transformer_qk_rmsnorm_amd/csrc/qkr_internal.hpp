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
    FastDiv div_mw[kMaxFusedGrids];      // merge * w of each grid
    const float* inv[3];                 // per-axis inverse frequencies
};

// One of Q, K, V.  Input views exist per stream (stream 1 only for the joint
// op); strides are in bytes.  weight == nullptr marks a copied tensor (V); a
// tensor with heads == 0 takes no work.
struct TensorArgs {
    const char* in[2];
    int64_t in_sb[2], in_st[2], in_sh[2];
    const char* weight[2];
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
    int32_t nvec;               // 16-byte vectors per row
    int32_t splits;             // workgroups per row (split variant)
    int32_t split_len;          // vectors stored by one split
    FastDiv div_splits;
    float eps;
    float inv_width;
};

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
    int64_t cu[kMaxGrids + 1];  // token offsets of this launch's grids (absolute)
    int32_t hw[kMaxGrids][2];   // h, w of each grid
};

// Axis of pair p (0 t, 1 h, 2 w, 3 e).  Host and device share this one
// definition so the host can be checked without a GPU.
__host__ __device__ inline int32_t pair_axis(int32_t mode, const int32_t* sec, int32_t p)
{
    if (mode == kPosImrope) {
        // interleaved multi-section sector rule
        const int32_t sect_dims = sec[0] + sec[1] + sec[2] + sec[3];
        const int32_t sector = p % sect_dims;
        const int32_t m3 = sector % 3;
        if (m3 == 1 && sector < 3 * sec[1]) return 1;
        if (m3 == 2 && sector < 3 * sec[2]) return 2;
        if (m3 == 0 && sector < 3 * sec[0]) return 0;
        return 3;
    }
    if (mode == kPosAxes || mode == kPosPlanes) {
        // contiguous runs: [0, s0) t, [s0, s0+s1) h, the rest w
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

// (t, h, w) of ViT token `tok`: its grid is the last one whose first token
// it has reached (grids are non-empty, so this is the number of grid ends
// reached), then frame, spatial-merge block and cell inside the block.  The
// grid is picked by a select loop, not an index, so the device build never
// indexes kernel arguments with a per-lane value.
__host__ __device__ inline void vit_position(const int64_t* cu, const int32_t (*hw)[2], int32_t num_grids,
                                             int32_t merge, int64_t tok, int32_t* tpos, int32_t* hpos,
                                             int32_t* wpos)
{
    int64_t start = cu[0], h = hw[0][0], w = hw[0][1];
    for (int32_t k = 1; k < num_grids; ++k) {
        const bool in_k = tok >= cu[k];
        start = in_k ? cu[k] : start;
        h = in_k ? hw[k][0] : h;
        w = in_k ? hw[k][1] : w;
    }
    const int64_t local = tok - start;
    const int64_t area = h * w;
    const int64_t rem = local % area;
    const int64_t mw = (int64_t)merge * w;
    const int64_t bh = rem / mw;
    const int64_t r = rem - bh * mw;
    const int64_t mm = (int64_t)merge * merge;
    const int64_t bw = r / mm;
    const int64_t r2 = r - bw * mm;
    *tpos = (int32_t)(local / area);
    *hpos = (int32_t)(bh * merge + r2 / merge);
    *wpos = (int32_t)(bw * merge + r2 % merge);
}

// QK RMSNorm + RoPE kernel for one lanes-per-row value (LPR in 1, 2, 4, 8, 16,
// 32), chosen by element type, rotation source (0 none, 1 positions, 2
// planes, 3 ViT grids), pairing, nontemporal accesses, staged stores and
// passes per wave.  Each LPR is defined in its own build of qkr_rope_part.hip.
using NormRopeFn = void (*)(NormRopeArgs);
template <int LPR>
NormRopeFn pick_norm_rope(int32_t dtype, int rope, int32_t pairing, bool nt, bool stage, int np);

// Kernel launchers (qkr_kernels.hip).  Each returns the variant name it
// launched through *variant; launch errors surface through hipGetLastError.
// norm_rope: np = passes (row groups) per wave and lpr = lanes per row, 0 =
// automatic (an lpr too small for the row is ignored); stage = 1 stores
// through LDS in contiguous runs, 0 directly, -1 automatic; nt = 1
// nontemporal row accesses, 0 plain.
hipError_t launch_norm_rope(const NormRopeArgs& a, int32_t dtype, int32_t pairing, int np, int lpr, int stage,
                            int nt, hipStream_t stream, const char** variant);
// rms: kind 0 rows, 1 split, 2 wide; -1 = automatic.  mode: bit 0 residual
// add, bit 1 FP8 E4M3 output (add modes never take the split variant: its
// workgroups read the whole row while others write the residual).
hipError_t launch_rms_norm(RmsArgs a, int32_t dtype, int kind, int nt, int mode, hipStream_t stream,
                           const char** variant);
hipError_t launch_debug_fp8(const float* x, int64_t n, const float* scale, uint8_t* out, hipStream_t stream);
hipError_t launch_vit_setup(const VitArgs& a, hipStream_t stream);
hipError_t launch_debug_axis_map(const RopeArgs& r, int32_t n_pairs, int32_t* out, hipStream_t stream);
hipError_t launch_debug_vit_positions(const VitArgs& a, int32_t* out, hipStream_t stream);

}  // namespace qkr
