// Variant choice of the two kernel families (pure host code, run before any
// HIP call): the kernel variant a call runs, from its shape.  A forced request
// that cannot run the call comes back as the reason, never as another
// variant.  The choices follow measurements on MI355X, quoted beside them.
#include "qkr_internal.hpp"

namespace qkr {
namespace {

// Vectors per lane of the row kernel, rounded up to an instantiated size.
int round_vpl(int need)
{
    static const int sizes[] = {1, 2, 3, 4, 5, 6, 8, 10, 12, 16};
    for (int s : sizes)
        if (need <= s)
            return s;
    return -1;
}

}  // namespace

const char* plan_norm_rope(int32_t dtype, int32_t head_dim, const int32_t heads[3], int32_t half, bool planes,
                           bool token_ok, int np_req, int lpr_req, int stage_req, int token_req, int nt_req,
                           RopePlan* plan)
{
    const int ve = dtype == kBF16 ? 8 : 4;
    const int nv = head_dim / ve;
    // Token tiles (one wavefront per token, Q and K rows together, L lanes
    // per row) wherever they can run, cos/sin planes aside: a row's vector
    // pairs need 3, 5, 6 or 7 lanes, so the tile kernel's row groups of 4 or
    // 8 would leave lanes idle, and the token's Q and K rows fit the wave's
    // LDS slice.  Measured
    // on MI355X, 8192 tokens, token / tile time (runs of the same build):
    // bf16 head_dim 80, 16 + 16 heads: 1-D positions 0.95 / 0.98 (adjacent
    // pairing 0.94), t/h/w axes 0.93, cos/sin planes 0.95, norm only 0.86 /
    // 0.89; 8 + 8 heads 0.98 with positions, 1.03 with planes (the one loss
    // measured); 2 + 2 heads 0.78 (positions), 0.80 (planes); head_dim 96
    // (12 + 12) positions 0.91, planes 0.93, norm only 0.93; 112 (11 + 11)
    // positions 0.92, planes 0.92 / 0.95; 48 (26 + 26) positions 0.98 to
    // 1.01, planes 0.91 / 0.95, norm only 0.87; fp32 head_dim 40 positions
    // 0.97, planes 0.97; fp32 24 positions 0.98.  Planes from the ViT setup
    // (7952 tokens, sections 8 / 16 / 16, written just before the apply) run
    // 1.008 at the kernel and 1.02 over the setup + apply step, so planes stay
    // on the tile kernel.  The tile kernel's knobs (np, lpr, stage) force the
    // tile kernel.
    const int token_lanes = (nv + 1) / 2;
    const bool token_shape = token_lanes == 3 || token_lanes == 5 || token_lanes == 6 || token_lanes == 7;
    const bool token_fits = (int64_t)(heads[0] + heads[1]) * nv <= kTokenTileVecs && half <= 64;
    const bool tile_knobs = np_req > 0 || lpr_req > 0 || stage_req >= 0;
    if (token_req == 1) {
        if (tile_knobs)
            return "rope:token: the passes, lanes-per-row and staging choices belong to the tile kernel";
        if (!token_ok)
            return "rope:token: token tiles take Q and K only (no V, no slot map, one stream)";
        if (!token_shape)
            return "rope:token: token tiles serve rows of 5, 6, 9 to 14 16-byte vectors (3, 5, 6 or 7 lanes)";
        if (!token_fits)
            return "rope:token: the token's Q and K rows exceed the 320 vectors of the wave's slice";
    }
    if (token_req == 1 || (token_req < 0 && !tile_knobs && !planes && token_ok && token_shape && token_fits)) {
        plan->lpr = token_lanes;
        plan->np = 0;
        plan->stage = false;
        plan->nt = nt_req != 0;
        plan->token = token_lanes;
        plan->waves_cap = 0;
        return nullptr;
    }
    plan->token = 0;
    // Lanes per row: the smallest power of two that gives every lane at most
    // two vectors of the row.
    int lpr = 1;
    while (2 * lpr < nv)
        lpr *= 2;
    if (lpr_req > 0) {
        if (2 * lpr_req < nv)
            return "rope:lpr: too few lanes per row for this head_dim (each lane holds at most two vectors)";
        lpr = lpr_req;
    }
    const int rpp = 64 / lpr;
    int np = np_req;
    if (np <= 0) {
        // Two passes per tile where a tensor has two or more passes of heads,
        // unless a third or more of the tiles' passes would then be idle (a
        // tensor's last tile holding one pass of heads).  Measured on MI355X
        // with two / one / three passes: the joint op (24 heads of 128 per
        // tensor, a quarter of the passes idle) 29.7 / 30.0 / 30.3 us, fused
        // ViT (16 + 16 heads of 80) 19.8 / 24.1 / 21.2 us, a 2048-token
        // IMROPE chunk (16 + 8 heads of 128, a quarter idle) 5.96 / 6.67 /
        // 6.18 us, the cache write (16 Q + 8 K + 8 V heads of 128, a third
        // idle) 24.69 / 24.31 / 25.10 us.
        int max_passes = 0, slots = 0, idle = 0;
        for (int i = 0; i < 3; ++i) {
            const int passes = (heads[i] + rpp - 1) / rpp;
            max_passes = passes > max_passes ? passes : max_passes;
            slots += (passes + 1) / 2 * 2;
            idle += (passes + 1) / 2 * 2 - passes;
        }
        np = max_passes >= 2 && 3 * idle < slots ? 2 : 1;
    }
    if (np < 1 || np > 4)
        return "rope:np: passes per wave must be 1 to 4";
    // Staged stores where a half row is not a whole number of 128-byte lines;
    // they exist for 2 to 8 lanes per row (rows of up to 16 vectors).
    const bool can_stage = lpr >= 2 && lpr <= 8;
    bool stage = nv % 16 != 0 && can_stage;
    if (stage_req >= 0) {
        if (stage_req != 0 && !can_stage)
            return "rope:stage1: staged stores exist for 2 to 8 lanes per row only";
        stage = stage_req != 0;
    }
    plan->lpr = lpr;
    plan->np = np;
    plan->stage = stage;
    plan->nt = nt_req != 0;
    // At most seven waves per SIMD where a wave moves 4 KB or more each way
    // (its rows in flight at once): an eighth wave adds requests to memory
    // that is already saturated.  Measured on MI355X (same machine,
    // alternating runs): the joint op (np 2, eight rows of 256 bytes per
    // pass, 64 registers) 28.95 us at eight waves, 28.80 us at seven; the
    // IMROPE chunk, one round of waves, 5.74 us either way; the cache write
    // (np 1, 2 KB per wave) prefers eight: 24.2 against 25.1 us at seven.
    const int64_t wave_bytes = (int64_t)rpp * np * head_dim * (dtype == kBF16 ? 2 : 4);
    plan->waves_cap = wave_bytes >= 4096 ? 7 : 0;
    return nullptr;
}

const char* plan_rms_norm(int32_t nvec, int64_t rows, int kind_req, int nt_req, int mode, RmsPlan* plan)
{
    const bool add = (mode & 1) != 0;
    const int vpl_wave = round_vpl((nvec + 63) / 64);              // rows, split
    const int vpl_wide = round_vpl((nvec + kThreads - 1) / kThreads);
    int kind = kind_req;
    if (kind < 0) {
        // A wavefront per row from 2048 to 4096 rows, a workgroup per row
        // below and above.  Up to 4096 rows (256 compute units x 4 SIMDs x 4
        // waves) the wave-per-row launch is a single round of waves; past it
        // the workgroups, four waves each over one row, overlap better.
        // Measured on MI355X, rows of 5120 bf16, wide / one wave per row, us:
        // 512 rows 3.44 / 5.28, 1024 5.25 / 5.87, 1536 7.28 / 7.00, 2048
        // 8.99 / 7.68, 3072 12.4 / 11.0, 4096 15.8 / 14.1, 6144 22.4 / 21.3,
        // 8192 29.1 / 30.1; with the residual add 1024 8.91 / 7.80, 2048
        // 15.6 / 14.0, 4096 28.6 / 27.9, 6144 41.5 / 47.1, 8192 54.9 / 60.4.
        // The split variant (1 row 2.23 us against 2.16 wide, 32 rows 3.31
        // against 2.82) never wins; it stays reachable through the variant
        // override.  Rows of fewer than 64 vectors keep a wave each (a
        // workgroup would leave most of its lanes idle); rows too long for
        // one wavefront go to the workgroup-wide variant.
        kind = nvec >= 64 && (rows < 2048 || rows > 4096) ? 2 : 0;
        if (kind == 0 && vpl_wave < 0)
            kind = 2;
    } else {
        if (kind == 1 && add)
            return "rms:split: the split variant cannot take the residual add (its workgroups read the whole "
                   "row while others write the residual)";
        if (kind != 2 && vpl_wave < 0)
            return "rms:rows / rms:split: the row does not fit one wavefront (more than 1024 vectors)";
    }
    const int vpl = kind == 2 ? vpl_wide : vpl_wave;
    if (vpl < 0)
        return "rms: the row is longer than 4096 vectors";
    plan->kind = kind;
    plan->vpl = vpl;
    plan->nt = nt_req != 0;
    plan->mode = mode;
    return nullptr;
}

}  // namespace qkr
