// Host-visible kernel argument blocks and launchers (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gqa_device.h"

namespace gqa {

// A call's mask after host-side resolution (resolve_mask in api.hip). Key s is
// visible to query t iff
//   s < prefix  or  t - wl <= s <= t + wr,
// and, with segment ids, q_seg[b,t] == kv_seg[b,s]. Sides that bound nothing
// for these sizes are kNoWindow; wr may be negative (an end-aligned causal
// diagonal with T > S). causal / coff record where wr came from: a causal
// diagonal s <= t + coff, top-left (coff = 0) or end-aligned (coff = S - T).
struct MaskSpec {
    int causal, coff, wl, wr, prefix;
};
// Is there more to the mask than the plain causal diagonal (or nothing)?
inline bool mask_extra(const MaskSpec &m) {
    return m.prefix > 0 || m.wl < kNoWindow || m.wr < (m.causal ? m.coff : kNoWindow);
}
// Only a causal left window beyond the plain causal diagonal?
inline bool mask_left_window_only(const MaskSpec &m) {
    return m.causal && m.prefix == 0 && m.wl < kNoWindow && m.wr == m.coff;
}

struct FwdArgs {
    const __bf16 *q, *k, *v;
    __bf16 *o;
    float *lse;                      // may be null
    const int32_t *q_seg, *kv_seg;   // both null or both set
    int B, K, G, T, S;
    // The lazy mask, as resolved by resolve_mask: key s is visible to query t
    // when s < prefix or t - wl <= s <= t + wr (and, with segment ids, when
    // the ids are equal). causal says that wr is a causal diagonal s <= t +
    // coff (possibly capped by a right window side); it selects the kernels'
    // causal structure (heaviest blocks first, diagonal tile last).
    int causal;
    int coff;
    int wl, wr;
    int prefix;
    int load_placement;  // ping-pong kernel: where a wave issues its tile loads (FwdTuning)
    int gw;         // query heads per workgroup (divides G)
    int bq;         // queries per workgroup; gw * bq is a multiple of 32
    int n_gsplit;   // G / gw
    int n_qblocks;  // ceil(T / bq)
    // Split-KV (o_part non-null): the grid is n_splits copies of the usual
    // one; copy j covers key tiles [j split_tiles, (j+1) split_tiles) and
    // writes its normalised fp32 O and its lse for every row to
    // o_part[j][row][H] and lse_part[j][row] (row = (b K + k) G T + g T + t).
    // A merge kernel then combines the copies into o and lse.
    int n_splits;
    int split_tiles;
    float *o_part;
    float *lse_part;
    // Per-head masks (null: every head takes wl, wr, prefix above): int32
    // [K][G][3] in device memory, window left, window right and prefix of
    // query head (k, g), normalised in the kernels by head_mask_of. Only the
    // general kernel reads it; such a call never splits.
    const int32_t *head_mask;
};

// Split-KV plan of a shape (pure host function): n_splits == 1 means none.
// split_target: the workgroups the plan aims for (0 never splits).
struct SplitPlan {
    int n_splits, split_tiles;
};
SplitPlan fwd_split_plan(int B, int K, int G, int T, int S, int H, int split_target);

// Schedule choices of the forward that leave its arithmetic unchanged (the
// outputs are bitwise equal across them), chosen per call from the tuning
// table compiled in from tuning/mi355x.json, or given by the caller.
//   load_placement  ping-pong kernel: a wave issues its K/V tile loads in its
//                   softmax phase (0), at the start of its MFMA phase (1) or
//                   spread over its MFMA phase (2)
//   split_target    split-KV: workgroups the split plan aims for (0: none)
struct FwdTuning {
    int load_placement, split_target;
};
FwdTuning fwd_tuning(int G, int T, int S, int H, const MaskSpec &m, bool segments);
int fwd_split_target(int T, int S, int H);
hipError_t launch_fwd_merge(const FwdArgs &a, int H, hipStream_t stream);

struct FwdConfig {
    int nw, gw, bq, bkv;
};

// Tile configuration for a shape (pure host function), and the one the
// split-KV path uses (4 waves per workgroup).
FwdConfig fwd_config(int G, int T, int H);
FwdConfig fwd_config_split(int G, int T, int H);
// H = 256 dense shapes that run the ping-pong kernel, and its configuration.
bool fwd_pp256_applies(int G, int T, int S, const MaskSpec &m, bool segments);
// split-KV on the ping-pong kernel (with fwd_config's blocks)
bool fwd_pp_split_applies(int G, int T, int S, int H, const MaskSpec &m, bool segments);
FwdConfig fwd_config_pp256();
hipError_t launch_fwd(const FwdArgs &a, int H, hipStream_t stream);

struct BwdArgs {
    const __bf16 *q, *k, *v, *o, *dout;
    const float *lse;
    float *dq, *dk, *dv;
    float *delta;                    // workspace: D = rowsum(P * dP) in fp32, [B,K,G,T]
    float *lse2;                     // workspace: lse * log2(e) per row, +inf for a row that sees no key
    const int32_t *q_seg, *kv_seg;
    int B, K, G, T, S;
    int causal, coff, wl, wr, prefix;  // the resolved mask, as in FwdArgs
    const int32_t *head_mask;          // per-head masks, as in FwdArgs (general kernels only)
};

hipError_t launch_bwd(const BwdArgs &a, int H, hipStream_t stream);

}  // namespace gqa
