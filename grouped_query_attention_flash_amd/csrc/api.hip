// C ABI of the library: argument validation, tile selection and launch.
// The declarations and their contracts are in include/gqa_attn.h.
#include "gqa_attn.h"
#include "gqa_launch.h"

#include <climits>
#include <cstdint>
#include <mutex>

namespace {

thread_local int g_last_hip_error = 0;

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_common(const void *q, const void *k, const void *v, const void *o,
                 const int32_t *q_seg, const int32_t *kv_seg,
                 int B, int K, int G, int T, int S, int H) {
    if (!q || !k || !v || !o) return GQA_ATTN_ERR_NULL;
    if (B < 1 || K < 1 || G < 1 || T < 1 || S < 1) return GQA_ATTN_ERR_SHAPE;
    // 32-bit grid and per-(b, kv head) offsets must not overflow: each slice
    // is addressed in bytes by a signed 32-bit offset (buffer descriptors)
    const long long q_slice = (long long)G * T * H, kv_slice = (long long)S * H;
    if (2 * q_slice >= INT_MAX || 2 * kv_slice >= INT_MAX) return GQA_ATTN_ERR_SHAPE;
    if ((long long)B * K * G * ((long long)T + 31) >= INT_MAX) return GQA_ATTN_ERR_SHAPE;
    if (H != 64 && H != 128 && H != 256) return GQA_ATTN_ERR_HEADDIM;
    if ((q_seg == nullptr) != (kv_seg == nullptr)) return GQA_ATTN_ERR_SEGMENTS;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16)) return GQA_ATTN_ERR_ALIGN;
    if (q_seg && (!aligned(q_seg, 4) || !aligned(kv_seg, 4))) return GQA_ATTN_ERR_ALIGN;
    return GQA_ATTN_OK;
}

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// Mask arguments: causal 0 (none), 1 (top-left) or 2 (end-aligned); window
// sides -1 (unbounded) or >= 0; prefix >= 0.
int check_mask(int causal, int wl, int wr, int prefix) {
    if (causal < 0 || causal > 2) return GQA_ATTN_ERR_MASK;
    if (wl < -1 || wr < -1 || prefix < 0) return GQA_ATTN_ERR_MASK;
    return GQA_ATTN_OK;
}

// The lazy mask of a call in the kernels' terms (gqa::MaskSpec): a key is
// visible when s < prefix or t - wl <= s <= t + wr. A causal diagonal s <= t +
// coff (coff = 0 top-left, S - T end-aligned) caps the right side. Sides that
// bound nothing for these sizes (t - wl <= 0 and t + wr >= S - 1 for every
// query) become kNoWindow, so that huge caller values cannot overflow and a
// mask that hides nothing takes the unmasked kernels.
gqa::MaskSpec resolve_mask(int causal, int wl, int wr, int prefix, int T, int S) {
    gqa::MaskSpec m;
    m.wl = (wl < 0 || wl >= T - 1) ? gqa::kNoWindow : wl;
    m.wr = (wr < 0 || wr >= S - 1) ? gqa::kNoWindow : wr;
    m.causal = causal != 0;
    m.coff = causal == 2 ? S - T : 0;
    if (m.causal) {
        if (m.coff >= S - 1 && m.wr == gqa::kNoWindow) {
            m.causal = 0;  // every query sees every key (e.g. end-aligned, T = 1)
            m.coff = 0;
        } else {
            m.wr = m.wr < m.coff ? m.wr : m.coff;
        }
    }
    m.prefix = prefix < S ? prefix : S;
    if (m.prefix == S) {  // every key is a prefix key: nothing is hidden
        m.causal = 0;
        m.coff = 0;
        m.wl = m.wr = gqa::kNoWindow;
        m.prefix = 0;
    }
    return m;
}

int hip_fail(hipError_t e) {
    g_last_hip_error = (int)e;
    return GQA_ATTN_ERR_HIP;
}

}  // namespace

extern "C" {

int attn_check_fwd(const void *q, const void *k, const void *v, const void *o, const float *lse,
                   const int32_t *q_seg, const int32_t *kv_seg,
                   int B, int K, int G, int T, int S, int H, int causal) {
    int rc = check_common(q, k, v, o, q_seg, kv_seg, B, K, G, T, S, H);
    if (rc) return rc;
    rc = check_mask(causal, -1, -1, 0);
    if (rc) return rc;
    if (lse && !aligned(lse, 4)) return GQA_ATTN_ERR_ALIGN;
    return GQA_ATTN_OK;
}

// Forward with a schedule (tuning) and an optional split-KV plan
// (plan.n_splits > 1 needs the workspace: partial outputs first, then
// partial lse).
static int run_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
                   const int32_t *q_seg, const int32_t *kv_seg,
                   int B, int K, int G, int T, int S, int H, const gqa::MaskSpec &m,
                   gqa::FwdTuning tune, gqa::SplitPlan plan, void *workspace, void *stream,
                   const int32_t *head_mask = nullptr) {
    const bool segments = q_seg != nullptr;
    const gqa::FwdConfig cfg =
        head_mask ? gqa::fwd_config(G, T, H)  // per-head masks: the general kernel, one pass
        : plan.n_splits > 1
            ? (gqa::fwd_pp_split_applies(G, T, S, H, m, segments) ? gqa::fwd_config(G, T, H)
                                                                  : gqa::fwd_config_split(G, T, H))
        : (H == 256 && gqa::fwd_pp256_applies(G, T, S, m, segments)) ? gqa::fwd_config_pp256()
                                                                     : gqa::fwd_config(G, T, H);
    gqa::FwdArgs a;
    a.q = (const __bf16 *)q;
    a.k = (const __bf16 *)k;
    a.v = (const __bf16 *)v;
    a.o = (__bf16 *)o;
    a.lse = lse;
    a.q_seg = q_seg;
    a.kv_seg = kv_seg;
    a.B = B, a.K = K, a.G = G, a.T = T, a.S = S;
    a.causal = m.causal;
    a.coff = m.coff;
    a.wl = m.wl;
    a.wr = m.wr;
    a.prefix = m.prefix;
    a.load_placement = tune.load_placement;
    a.gw = cfg.gw;
    a.bq = cfg.bq;
    a.n_gsplit = G / cfg.gw;
    a.n_qblocks = (T + cfg.bq - 1) / cfg.bq;
    a.n_splits = plan.n_splits;
    a.split_tiles = plan.split_tiles;
    a.o_part = nullptr;
    a.lse_part = nullptr;
    a.head_mask = head_mask;
    if (plan.n_splits > 1) {
        const size_t rows = (size_t)B * K * G * T;
        a.o_part = (float *)workspace;
        a.lse_part = a.o_part + (size_t)plan.n_splits * rows * H;
    }
    hipError_t e = gqa::launch_fwd(a, H, (hipStream_t)stream);
    if (e == hipSuccess && plan.n_splits > 1) e = gqa::launch_fwd_merge(a, H, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e);
    return GQA_ATTN_OK;
}

int attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
             const int32_t *q_seg, const int32_t *kv_seg,
             int B, int K, int G, int T, int S, int H, int causal, void *stream) {
    int rc = attn_check_fwd(q, k, v, o, lse, q_seg, kv_seg, B, K, G, T, S, H, causal);
    if (rc) return rc;
    const gqa::MaskSpec m = resolve_mask(causal, -1, -1, 0, T, S);
    return run_fwd(q, k, v, o, lse, q_seg, kv_seg, B, K, G, T, S, H, m,
                   gqa::fwd_tuning(G, T, S, H, m, q_seg != nullptr), gqa::SplitPlan{1, 0}, nullptr, stream);
}

size_t attn_fwd_workspace_bytes(int B, int K, int G, int T, int S, int H) {
    if (B < 1 || K < 1 || G < 1 || T < 1 || S < 1) return 0;
    if (H != 64 && H != 128 && H != 256) return 0;
    const gqa::SplitPlan plan = gqa::fwd_split_plan(B, K, G, T, S, H, gqa::fwd_split_target(T, S, H));
    if (plan.n_splits <= 1) return 0;
    const size_t rows = (size_t)B * K * G * T;
    return round256(sizeof(float) * (size_t)plan.n_splits * rows * (H + 1));
}

int attn_check_fwd_ws(const void *q, const void *k, const void *v, const void *o, const float *lse,
                      const int32_t *q_seg, const int32_t *kv_seg,
                      int B, int K, int G, int T, int S, int H, int causal,
                      const void *workspace, size_t workspace_bytes) {
    int rc = attn_check_fwd(q, k, v, o, lse, q_seg, kv_seg, B, K, G, T, S, H, causal);
    if (rc) return rc;
    const size_t need = attn_fwd_workspace_bytes(B, K, G, T, S, H);
    if (need == 0) return GQA_ATTN_OK;
    if (!workspace || workspace_bytes < need) return GQA_ATTN_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return GQA_ATTN_ERR_ALIGN;
    return GQA_ATTN_OK;
}

int attn_fwd_ws(const void *q, const void *k, const void *v, void *o, float *lse,
                const int32_t *q_seg, const int32_t *kv_seg,
                int B, int K, int G, int T, int S, int H, int causal,
                void *workspace, size_t workspace_bytes, void *stream) {
    int rc = attn_check_fwd_ws(q, k, v, o, lse, q_seg, kv_seg, B, K, G, T, S, H, causal, workspace, workspace_bytes);
    if (rc) return rc;
    const gqa::MaskSpec m = resolve_mask(causal, -1, -1, 0, T, S);
    const gqa::FwdTuning tune = gqa::fwd_tuning(G, T, S, H, m, q_seg != nullptr);
    return run_fwd(q, k, v, o, lse, q_seg, kv_seg, B, K, G, T, S, H, m, tune,
                   gqa::fwd_split_plan(B, K, G, T, S, H, tune.split_target), workspace, stream);
}

int attn_check_fwd_mask(const void *q, const void *k, const void *v, const void *o, const float *lse,
                        const int32_t *q_seg, const int32_t *kv_seg,
                        int B, int K, int G, int T, int S, int H, int causal, int window_left, int window_right,
                        int prefix, const void *workspace, size_t workspace_bytes) {
    int rc = attn_check_fwd_ws(q, k, v, o, lse, q_seg, kv_seg, B, K, G, T, S, H, causal, workspace, workspace_bytes);
    if (rc) return rc;
    return check_mask(causal, window_left, window_right, prefix);
}

int attn_fwd_mask(const void *q, const void *k, const void *v, void *o, float *lse,
                  const int32_t *q_seg, const int32_t *kv_seg,
                  int B, int K, int G, int T, int S, int H, int causal, int window_left, int window_right, int prefix,
                  void *workspace, size_t workspace_bytes, void *stream) {
    int rc = attn_check_fwd_mask(q, k, v, o, lse, q_seg, kv_seg, B, K, G, T, S, H, causal, window_left,
                                 window_right, prefix, workspace, workspace_bytes);
    if (rc) return rc;
    const gqa::MaskSpec m = resolve_mask(causal, window_left, window_right, prefix, T, S);
    const gqa::FwdTuning tune = gqa::fwd_tuning(G, T, S, H, m, q_seg != nullptr);
    return run_fwd(q, k, v, o, lse, q_seg, kv_seg, B, K, G, T, S, H, m, tune,
                   gqa::fwd_split_plan(B, K, G, T, S, H, tune.split_target), workspace, stream);
}

size_t attn_fwd_tuned_workspace_bytes(int B, int K, int G, int T, int S, int H, int split_target) {
    if (B < 1 || K < 1 || G < 1 || T < 1 || S < 1) return 0;
    if (H != 64 && H != 128 && H != 256) return 0;
    if (split_target < -1 || split_target > (1 << 20)) return 0;
    const int target = split_target < 0 ? gqa::fwd_split_target(T, S, H) : split_target;
    const gqa::SplitPlan plan = gqa::fwd_split_plan(B, K, G, T, S, H, target);
    if (plan.n_splits <= 1) return 0;
    const size_t rows = (size_t)B * K * G * T;
    return round256(sizeof(float) * (size_t)plan.n_splits * rows * (H + 1));
}

int attn_fwd_tuning(int B, int K, int G, int T, int S, int H, int causal, int window_left, int window_right,
                    int prefix, int segments, int *load_placement, int *split_target) {
    if (!load_placement || !split_target) return GQA_ATTN_ERR_NULL;
    if (B < 1 || K < 1 || G < 1 || T < 1 || S < 1) return GQA_ATTN_ERR_SHAPE;
    if (H != 64 && H != 128 && H != 256) return GQA_ATTN_ERR_HEADDIM;
    int rc = check_mask(causal, window_left, window_right, prefix);
    if (rc) return rc;
    const gqa::FwdTuning t =
        gqa::fwd_tuning(G, T, S, H, resolve_mask(causal, window_left, window_right, prefix, T, S), segments != 0);
    *load_placement = t.load_placement;
    *split_target = t.split_target;
    return GQA_ATTN_OK;
}

int attn_fwd_tuned(const void *q, const void *k, const void *v, void *o, float *lse,
                   const int32_t *q_seg, const int32_t *kv_seg,
                   int B, int K, int G, int T, int S, int H, int causal, int window_left, int window_right, int prefix,
                   int load_placement, int split_target, void *workspace, size_t workspace_bytes, void *stream) {
    int rc = attn_check_fwd(q, k, v, o, lse, q_seg, kv_seg, B, K, G, T, S, H, 0);
    if (rc) return rc;
    rc = check_mask(causal, window_left, window_right, prefix);
    if (rc) return rc;
    if (load_placement < -1 || load_placement > 2 || split_target < -1 || split_target > (1 << 20))
        return GQA_ATTN_ERR_TUNING;
    const size_t need = attn_fwd_tuned_workspace_bytes(B, K, G, T, S, H, split_target);
    if (need > 0 && (!workspace || workspace_bytes < need)) return GQA_ATTN_ERR_WORKSPACE;
    if (need > 0 && !aligned(workspace, 16)) return GQA_ATTN_ERR_ALIGN;
    const gqa::MaskSpec m = resolve_mask(causal, window_left, window_right, prefix, T, S);
    gqa::FwdTuning tune = gqa::fwd_tuning(G, T, S, H, m, q_seg != nullptr);
    if (load_placement >= 0) tune.load_placement = load_placement;
    if (split_target >= 0) tune.split_target = split_target;
    return run_fwd(q, k, v, o, lse, q_seg, kv_seg, B, K, G, T, S, H, m, tune,
                   gqa::fwd_split_plan(B, K, G, T, S, H, tune.split_target), workspace, stream);
}

int attn_check_fwd_local(const void *q, const void *k, const void *v, const void *o, const float *lse,
                         const int32_t *q_seg, const int32_t *kv_seg,
                         int B, int K, int G, int T, int S, int H, int causal, int window_left, int window_right,
                         const void *workspace, size_t workspace_bytes) {
    return attn_check_fwd_mask(q, k, v, o, lse, q_seg, kv_seg, B, K, G, T, S, H, causal, window_left, window_right,
                               0, workspace, workspace_bytes);
}

int attn_fwd_local(const void *q, const void *k, const void *v, void *o, float *lse,
                   const int32_t *q_seg, const int32_t *kv_seg,
                   int B, int K, int G, int T, int S, int H, int causal, int window_left, int window_right,
                   void *workspace, size_t workspace_bytes, void *stream) {
    return attn_fwd_mask(q, k, v, o, lse, q_seg, kv_seg, B, K, G, T, S, H, causal, window_left, window_right, 0,
                         workspace, workspace_bytes, stream);
}

int attn_fwd_split_count(int B, int K, int G, int T, int S, int H) {
    if (B < 1 || K < 1 || G < 1 || T < 1 || S < 1) return 0;
    if (H != 64 && H != 128 && H != 256) return 0;
    return gqa::fwd_split_plan(B, K, G, T, S, H, gqa::fwd_split_target(T, S, H)).n_splits;
}

size_t attn_bwd_workspace_bytes(int B, int K, int G, int T, int S, int H) {
    (void)H;
    if (B < 1 || K < 1 || G < 1 || T < 1 || S < 1) return 0;
    // D, then lse * log2(e), one fp32 per query row each
    return 2 * round256(sizeof(float) * (size_t)B * K * G * T);
}

int attn_check_bwd(const void *q, const void *k, const void *v, const void *o, const float *lse,
                   const void *dO, const float *dq, const float *dk, const float *dv,
                   const int32_t *q_seg, const int32_t *kv_seg,
                   int B, int K, int G, int T, int S, int H, int causal,
                   const void *workspace, size_t workspace_bytes) {
    int rc = check_common(q, k, v, dq, q_seg, kv_seg, B, K, G, T, S, H);
    if (rc) return rc;
    rc = check_mask(causal, -1, -1, 0);
    if (rc) return rc;
    if (!lse || !dO || !dq || !dk || !dv) return GQA_ATTN_ERR_NULL;
    if (o && !aligned(o, 16)) return GQA_ATTN_ERR_ALIGN;
    if (!aligned(lse, 16) || !aligned(dO, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16))
        return GQA_ATTN_ERR_ALIGN;
    if (!workspace || workspace_bytes < attn_bwd_workspace_bytes(B, K, G, T, S, H)) return GQA_ATTN_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return GQA_ATTN_ERR_ALIGN;
    return GQA_ATTN_OK;
}

static int run_bwd(const void *q, const void *k, const void *v, const void *o, const float *lse,
                   const void *dO, float *dq, float *dk, float *dv,
                   const int32_t *q_seg, const int32_t *kv_seg,
                   int B, int K, int G, int T, int S, int H, const gqa::MaskSpec &m,
                   void *workspace, void *stream, const int32_t *head_mask = nullptr) {
    gqa::BwdArgs a;
    a.q = (const __bf16 *)q;
    a.k = (const __bf16 *)k;
    a.v = (const __bf16 *)v;
    a.o = (const __bf16 *)o;
    a.dout = (const __bf16 *)dO;
    a.lse = lse;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.delta = (float *)workspace;
    a.lse2 = a.delta + round256(sizeof(float) * (size_t)B * K * G * T) / sizeof(float);
    a.q_seg = q_seg;
    a.kv_seg = kv_seg;
    a.B = B, a.K = K, a.G = G, a.T = T, a.S = S;
    a.causal = m.causal;
    a.coff = m.coff;
    a.wl = m.wl;
    a.wr = m.wr;
    a.prefix = m.prefix;
    a.head_mask = head_mask;
    hipError_t e = gqa::launch_bwd(a, H, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e);
    return GQA_ATTN_OK;
}

int attn_bwd(const void *q, const void *k, const void *v, const void *o, const float *lse,
             const void *dO, float *dq, float *dk, float *dv,
             const int32_t *q_seg, const int32_t *kv_seg,
             int B, int K, int G, int T, int S, int H, int causal,
             void *workspace, size_t workspace_bytes, void *stream) {
    int rc = attn_check_bwd(q, k, v, o, lse, dO, dq, dk, dv, q_seg, kv_seg, B, K, G, T, S, H, causal,
                            workspace, workspace_bytes);
    if (rc) return rc;
    return run_bwd(q, k, v, o, lse, dO, dq, dk, dv, q_seg, kv_seg, B, K, G, T, S, H,
                   resolve_mask(causal, -1, -1, 0, T, S), workspace, stream);
}

int attn_check_bwd_mask(const void *q, const void *k, const void *v, const void *o, const float *lse,
                        const void *dO, const float *dq, const float *dk, const float *dv,
                        const int32_t *q_seg, const int32_t *kv_seg,
                        int B, int K, int G, int T, int S, int H, int causal, int window_left, int window_right,
                        int prefix, const void *workspace, size_t workspace_bytes) {
    int rc = attn_check_bwd(q, k, v, o, lse, dO, dq, dk, dv, q_seg, kv_seg, B, K, G, T, S, H, causal, workspace,
                            workspace_bytes);
    if (rc) return rc;
    return check_mask(causal, window_left, window_right, prefix);
}

int attn_bwd_mask(const void *q, const void *k, const void *v, const void *o, const float *lse,
                  const void *dO, float *dq, float *dk, float *dv,
                  const int32_t *q_seg, const int32_t *kv_seg,
                  int B, int K, int G, int T, int S, int H, int causal, int window_left, int window_right, int prefix,
                  void *workspace, size_t workspace_bytes, void *stream) {
    int rc = attn_check_bwd_mask(q, k, v, o, lse, dO, dq, dk, dv, q_seg, kv_seg, B, K, G, T, S, H, causal,
                                 window_left, window_right, prefix, workspace, workspace_bytes);
    if (rc) return rc;
    return run_bwd(q, k, v, o, lse, dO, dq, dk, dv, q_seg, kv_seg, B, K, G, T, S, H,
                   resolve_mask(causal, window_left, window_right, prefix, T, S), workspace, stream);
}

int attn_check_bwd_local(const void *q, const void *k, const void *v, const void *o, const float *lse,
                         const void *dO, const float *dq, const float *dk, const float *dv,
                         const int32_t *q_seg, const int32_t *kv_seg,
                         int B, int K, int G, int T, int S, int H, int causal, int window_left, int window_right,
                         const void *workspace, size_t workspace_bytes) {
    return attn_check_bwd_mask(q, k, v, o, lse, dO, dq, dk, dv, q_seg, kv_seg, B, K, G, T, S, H, causal,
                               window_left, window_right, 0, workspace, workspace_bytes);
}

int attn_bwd_local(const void *q, const void *k, const void *v, const void *o, const float *lse,
                   const void *dO, float *dq, float *dk, float *dv,
                   const int32_t *q_seg, const int32_t *kv_seg,
                   int B, int K, int G, int T, int S, int H, int causal, int window_left, int window_right,
                   void *workspace, size_t workspace_bytes, void *stream) {
    return attn_bwd_mask(q, k, v, o, lse, dO, dq, dk, dv, q_seg, kv_seg, B, K, G, T, S, H, causal, window_left,
                         window_right, 0, workspace, workspace_bytes, stream);
}

// ---------------------------------------------------------------------------
// Per-head masks: head_mask is a device int32 array [K][G][3] holding, for
// query head (k, g), its window left side, window right side and prefix
// length; causal masking applies to every head. The kernels normalise each
// entry as resolve_mask does a call's (head_mask_of), so every value is a
// valid mask; the host checks only the pointer.
int attn_check_fwd_head_masks(const void *q, const void *k, const void *v, const void *o, const float *lse,
                              const int32_t *q_seg, const int32_t *kv_seg,
                              int B, int K, int G, int T, int S, int H, int causal, const int32_t *head_mask) {
    int rc = attn_check_fwd(q, k, v, o, lse, q_seg, kv_seg, B, K, G, T, S, H, causal);
    if (rc) return rc;
    if (!head_mask) return GQA_ATTN_ERR_NULL;
    if (!aligned(head_mask, 4)) return GQA_ATTN_ERR_ALIGN;
    return GQA_ATTN_OK;
}

int attn_fwd_head_masks(const void *q, const void *k, const void *v, void *o, float *lse,
                        const int32_t *q_seg, const int32_t *kv_seg,
                        int B, int K, int G, int T, int S, int H, int causal, const int32_t *head_mask,
                        void *stream) {
    int rc = attn_check_fwd_head_masks(q, k, v, o, lse, q_seg, kv_seg, B, K, G, T, S, H, causal, head_mask);
    if (rc) return rc;
    const gqa::MaskSpec m = resolve_mask(causal, -1, -1, 0, T, S);
    return run_fwd(q, k, v, o, lse, q_seg, kv_seg, B, K, G, T, S, H, m, gqa::FwdTuning{0, 0}, gqa::SplitPlan{1, 0},
                   nullptr, stream, head_mask);
}

int attn_check_bwd_head_masks(const void *q, const void *k, const void *v, const void *o, const float *lse,
                              const void *dO, const float *dq, const float *dk, const float *dv,
                              const int32_t *q_seg, const int32_t *kv_seg,
                              int B, int K, int G, int T, int S, int H, int causal, const int32_t *head_mask,
                              const void *workspace, size_t workspace_bytes) {
    int rc = attn_check_bwd(q, k, v, o, lse, dO, dq, dk, dv, q_seg, kv_seg, B, K, G, T, S, H, causal, workspace,
                            workspace_bytes);
    if (rc) return rc;
    if (!head_mask) return GQA_ATTN_ERR_NULL;
    if (!aligned(head_mask, 4)) return GQA_ATTN_ERR_ALIGN;
    return GQA_ATTN_OK;
}

int attn_bwd_head_masks(const void *q, const void *k, const void *v, const void *o, const float *lse,
                        const void *dO, float *dq, float *dk, float *dv,
                        const int32_t *q_seg, const int32_t *kv_seg,
                        int B, int K, int G, int T, int S, int H, int causal, const int32_t *head_mask,
                        void *workspace, size_t workspace_bytes, void *stream) {
    int rc = attn_check_bwd_head_masks(q, k, v, o, lse, dO, dq, dk, dv, q_seg, kv_seg, B, K, G, T, S, H, causal,
                                       head_mask, workspace, workspace_bytes);
    if (rc) return rc;
    return run_bwd(q, k, v, o, lse, dO, dq, dk, dv, q_seg, kv_seg, B, K, G, T, S, H,
                   resolve_mask(causal, -1, -1, 0, T, S), workspace, stream, head_mask);
}

// ---------------------------------------------------------------------------
// The allocation-free forward (attn_fwd_noalloc). Its split-KV partial results
// go to this file-scope device array instead of a caller workspace; each GPU
// the library runs on holds one copy until the process ends. In host code
// the name `scratch` is a host-side stand-in, not a device address: host code
// only ever uses the per-device address hipGetSymbolAddress returns.
}  // extern "C"

static constexpr size_t kScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];  // per device, resolved on its first call

// The device address of this GPU's copy of `scratch` (the current device,
// which must be the one the caller's stream belongs to).
int scratch_on_current_device(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    if (dev < 0 || dev >= kMaxDevices) return hip_fail(hipErrorInvalidDevice);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e);
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return GQA_ATTN_OK;
}

}  // namespace

extern "C" {

int attn_fwd_noalloc(const void *q, const void *k, const void *v, void *o, float *lse,
                     const int32_t *q_seg, const int32_t *kv_seg,
                     int B, int K, int G, int T, int S, int H, int causal, int window_left, int window_right,
                     int prefix, void *stream) {
    int rc = attn_check_fwd(q, k, v, o, lse, q_seg, kv_seg, B, K, G, T, S, H, 0);
    if (rc) return rc;
    rc = check_mask(causal, window_left, window_right, prefix);
    if (rc) return rc;
    const size_t need = attn_fwd_workspace_bytes(B, K, G, T, S, H);
    if (need > kScratchBytes) return GQA_ATTN_ERR_WORKSPACE;
    void *ws = nullptr;
    if (need > 0) {
        rc = scratch_on_current_device(&ws);
        if (rc) return rc;
    }
    const gqa::MaskSpec m = resolve_mask(causal, window_left, window_right, prefix, T, S);
    const gqa::FwdTuning tune = gqa::fwd_tuning(G, T, S, H, m, q_seg != nullptr);
    return run_fwd(q, k, v, o, lse, q_seg, kv_seg, B, K, G, T, S, H, m, tune,
                   gqa::fwd_split_plan(B, K, G, T, S, H, tune.split_target), ws, stream);
}

const char *attn_strerror(int code) {
    switch (code) {
        case GQA_ATTN_OK: return "success";
        case GQA_ATTN_ERR_NULL: return "a required pointer is NULL";
        case GQA_ATTN_ERR_SHAPE:
            return "invalid sizes: B, K, G, T, S must be >= 1, each (b, kv head) slice of q or k < 2^30 elements and "
                   "B*K*G*(T+31) < 2^31";
        case GQA_ATTN_ERR_HEADDIM: return "unsupported head dimension H (supported: 64, 128, 256)";
        case GQA_ATTN_ERR_ALIGN: return "misaligned pointer (tensors need 16-byte alignment, segment ids 4-byte)";
        case GQA_ATTN_ERR_SEGMENTS: return "q_seg and kv_seg must both be given or both be NULL";
        case GQA_ATTN_ERR_WORKSPACE:
            return "workspace is NULL or smaller than the call's attn_fwd_workspace_bytes() / "
                   "attn_bwd_workspace_bytes()";
        case GQA_ATTN_ERR_HIP: return "a HIP launch failed (see attn_last_hip_error)";
        case GQA_ATTN_ERR_TUNING:
            return "invalid schedule: load_placement must be -1 (table), 0, 1 or 2 and split_target -1 (table) or "
                   "0 .. 2^20";
        case GQA_ATTN_ERR_MASK:
            return "invalid mask: causal must be 0, 1 (top-left) or 2 (end-aligned), window sides -1 or >= 0, "
                   "prefix >= 0";
        default: return "unknown error code";
    }
}

int attn_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
