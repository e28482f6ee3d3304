/*
 * gqa_attn.h -- C ABI of the fused grouped-query flash-attention library
 * for AMD Instinct MI355X (gfx950).
 *
 * Notation follows danielwatson6.github.io/fa, section "Notation":
 *   B batch, T queries, S keys/values, K kv heads, G query heads per kv head,
 *   H head dimension.
 * Layouts (row-major, contiguous, H innermost):
 *   q, o, dO, dq : [B, K, G, T, H]   (query head k*G + g reads kv head k)
 *   k, v, dk, dv : [B, K, S, H]
 *   lse          : [B, K, G, T] fp32
 *   q_seg        : [B, T] int32,  kv_seg : [B, S] int32
 *
 * What is computed (same page, attn_naive in "What is wrong with naive
 * attention?", and the fused kernel of "Optimizing the kernel"):
 *   O[t,:] = sum_s softmax_s(q[t,:].k[s,:] + mask[t,s]) v[s,:]
 * with no further scaling: q must arrive pre-multiplied by H^-1/2.
 * bf16 inputs, fp32 accumulation, bf16 output (the page's kernel writes its
 * output in the input dtype). The T x S weights are never stored.
 * Masks are generated lazily, never materialised:
 *   causal (apple/axlearn PR 845, lazy causal mask), argument `causal`:
 *     0  none;
 *     1  top-left aligned: key s visible to query t iff s <= t;
 *     2  end-aligned: key s visible to query t iff s <= t + (S - T), so the
 *        last query sees every key, as a block of T new queries appended to
 *        an S-token context does (the decoding regime of
 *        danielwatson6.github.io/fa, "Quick digression: what about
 *        inference?"). With T == S the two alignments agree; with T > S the
 *        first T - S queries see no key.
 *   segments (fjformer Pallas flash-attention docs, SegmentIds): key s visible
 *     to query t iff q_seg[b,t] == kv_seg[b,s]; combined with the rest by AND.
 *   window and prefix (attn_fwd_mask / attn_bwd_mask below), also per query
 *     head (attn_fwd_head_masks / attn_bwd_head_masks).
 * A query row that sees no key gets O = 0 and lse = -inf.
 *
 * Conventions for every call:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the
 *     library never allocates, frees or retains them. It holds no state.
 *   - Tensor pointers must be 16-byte aligned (128-bit loads); int32 segment
 *     arrays 4-byte aligned.
 *   - Arguments are validated on the host BEFORE anything is enqueued; on a
 *     nonzero return nothing has been launched and no output is written.
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*, NULL =
 *     the default stream) without any host synchronisation.
 *   - Returns 0 on success or a positive GQA_ATTN_ERR_* code. The codes carry
 *     the library's GQA_ATTN_ prefix (rather than a bare ATTN_) so that they
 *     cannot collide with another attention library's enums in one program.
 *   - Thread-safe: concurrent calls on different streams are independent.
 * Error checking stands in for the pages' own argument checks: the shape
 * asserts at the top of the fused kernel's wrapper
 * (danielwatson6.github.io/fa, "Optimizing the kernel") and the ValueError
 * that fjformer's BlockSizes dataclass raises on inconsistent block sizes.
 * Unlike those, every size >= 1 is accepted here (ragged tiles are masked).
 */
#ifndef GQA_ATTN_H
#define GQA_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    GQA_ATTN_OK = 0,
    GQA_ATTN_ERR_NULL = 1,      /* a required pointer is NULL                    */
    GQA_ATTN_ERR_SHAPE = 2,     /* B,K,G,T,S < 1, a (b, kv head) slice of q or k of 2^30 elements or
                                   more, or B*K*G*(T+31) of 2^31 or more (32-bit grid sizes) */
    GQA_ATTN_ERR_HEADDIM = 3,   /* H not in {64, 128, 256}                       */
    GQA_ATTN_ERR_ALIGN = 4,     /* a pointer is not 16-byte (4 for ids) aligned  */
    GQA_ATTN_ERR_SEGMENTS = 5,  /* exactly one of q_seg / kv_seg given           */
    GQA_ATTN_ERR_WORKSPACE = 6, /* workspace NULL or smaller than required       */
    GQA_ATTN_ERR_HIP = 7,       /* a HIP launch failed: see attn_last_hip_error  */
    GQA_ATTN_ERR_MASK = 8,      /* causal not 0/1/2, a window side below -1, or a
                                   negative prefix                               */
    GQA_ATTN_ERR_TUNING = 9     /* an explicit schedule choice out of range      */
};

/* Forward pass (danielwatson6.github.io/fa, "Optimizing the kernel": the fused
 * two-axis kernel with the output carry kept on chip; its running max and sum
 * follow the numerically stable scan of "Chunked attention").
 *   q        bf16 [B,K,G,T,H], pre-scaled by H^-1/2
 *   k, v     bf16 [B,K,S,H]
 *   o        bf16 [B,K,G,T,H]  (written)
 *   lse      fp32 [B,K,G,T]    (written: natural-log logsumexp of each row's
 *            visible logits, the residual the backward needs), or NULL
 *   q_seg    int32 [B,T] and kv_seg int32 [B,S]: both or neither (NULL)
 *   causal   0, 1 (top-left) or 2 (end-aligned), as above
 * Errors: NULL q/k/v/o -> ERR_NULL; bad sizes -> ERR_SHAPE; H -> ERR_HEADDIM;
 * alignment -> ERR_ALIGN; one segment array -> ERR_SEGMENTS; causal outside
 * 0..2 -> ERR_MASK; launch -> ERR_HIP. */
int attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
             const int32_t *q_seg, const int32_t *kv_seg,
             int B, int K, int G, int T, int S, int H, int causal, void *stream);

/* Host-only validation of attn_fwd's arguments (pointer values are checked for
 * NULL and alignment but never dereferenced). Same return codes. It is the
 * argument check that the shape asserts of the fused kernel's wrapper
 * (danielwatson6.github.io/fa, "Optimizing the kernel") and the BlockSizes
 * ValueError (fjformer page, "BlockSizes dataclass") perform, callable
 * without a GPU. */
int attn_check_fwd(const void *q, const void *k, const void *v, const void *o, const float *lse,
                   const int32_t *q_seg, const int32_t *kv_seg,
                   int B, int K, int G, int T, int S, int H, int causal);

/* Forward pass for shapes with few query rows per kv head, such as decoding
 * (T = 1, S the context length), where the pages note that the intensity
 * falls to about G FLOP per byte (danielwatson6.github.io/fa, "Quick
 * digression: what about inference?"). Same arguments and result as
 * attn_fwd, plus a caller-owned device workspace. When the usual grid would
 * leave the GPU idle, the key range is split across workgroups: each split
 * writes a normalised fp32 partial output and its logsumexp to the
 * workspace, and a merge kernel combines them with the online softmax's
 * rescaling (O = sum_j exp(lse_j - lse) O_j, lse = ln sum_j exp(lse_j)).
 * Otherwise it runs exactly as attn_fwd and the workspace is not touched.
 *   workspace        device buffer of at least attn_fwd_workspace_bytes()
 *                    (which may be 0: then NULL is fine), 16-byte aligned,
 *                    owned by the caller, contents ignored
 * Errors as attn_fwd, plus ERR_WORKSPACE (NULL or too small when needed) and
 * ERR_ALIGN for a misaligned workspace. Enqueues one kernel, or the split
 * kernel and the merge kernel, on `stream`. */
int attn_fwd_ws(const void *q, const void *k, const void *v, void *o, float *lse,
                const int32_t *q_seg, const int32_t *kv_seg,
                int B, int K, int G, int T, int S, int H, int causal,
                void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of device workspace attn_fwd_ws (and attn_fwd_local, attn_fwd_mask)
 * needs for these sizes: 0 when it does not split, else n_splits * B*K*G*T *
 * (H + 1) fp32 rounded up to 256 bytes (partial outputs
 * [n_splits,B,K,G,T,H], then partial lse [n_splits,B,K,G,T]). Returns 0 for
 * invalid sizes. The pages describe no such buffer: it belongs to the
 * split-KV answer to the low-intensity decoding regime of
 * danielwatson6.github.io/fa, "Quick digression: what about inference?". */
size_t attn_fwd_workspace_bytes(int B, int K, int G, int T, int S, int H);

/* Number of key splits attn_fwd_ws uses for these sizes (1: no split; 0 for
 * invalid sizes). Host-only. Library convention (no passage of the pages):
 * it exposes the split plan of the decoding path above for callers and tests. */
int attn_fwd_split_count(int B, int K, int G, int T, int S, int H);

/* Forward pass with a local (sliding) window: key s is visible to query t
 * only when t - window_left <= s <= t + window_right, in addition to the
 * causal rule and segment ids; -1 leaves a side unbounded, and causal = 1
 * already bounds the right side at 0. The pages run splash attention with a
 * FullMask through its block mask processing (danielwatson6.github.io/fa,
 * "Our first kernel": make_splash_fn_nojit); a band of diagonals is the
 * simplest mask whose block classification is not all-full, and here it is
 * applied lazily as the causal mask is: key tiles outside the band are not
 * visited, and only tiles crossing an edge get an element mask. Otherwise as
 * attn_fwd_ws (workspace as there; window_left / window_right below -1 ->
 * ERR_MASK). A side at least as long as the sequence bounds nothing and is
 * treated as unbounded. With both sides unbounded it computes what
 * attn_fwd_ws does. Equal to attn_fwd_mask with prefix 0. */
int attn_fwd_local(const void *q, const void *k, const void *v, void *o, float *lse,
                   const int32_t *q_seg, const int32_t *kv_seg,
                   int B, int K, int G, int T, int S, int H, int causal, int window_left, int window_right,
                   void *workspace, size_t workspace_bytes, void *stream);

/* Host-only validation of attn_fwd_local's arguments. Same return codes; the
 * checks of attn_check_fwd (same passages) plus the window sides. */
int attn_check_fwd_local(const void *q, const void *k, const void *v, const void *o, const float *lse,
                         const int32_t *q_seg, const int32_t *kv_seg,
                         int B, int K, int G, int T, int S, int H, int causal, int window_left, int window_right,
                         const void *workspace, size_t workspace_bytes);

/* Host-only validation of attn_fwd_ws's arguments. Same return codes; the
 * checks of attn_check_fwd (same passages) plus the workspace. */
int attn_check_fwd_ws(const void *q, const void *k, const void *v, const void *o, const float *lse,
                      const int32_t *q_seg, const int32_t *kv_seg,
                      int B, int K, int G, int T, int S, int H, int causal,
                      const void *workspace, size_t workspace_bytes);

/* Forward pass with the general lazy mask of this library. Key s is visible
 * to query t iff
 *     s < prefix  or  (t - window_left <= s <= t + window_right and the
 *                      causal rule holds),
 * and, with segment ids, q_seg[b,t] == kv_seg[b,s]. The pages build their
 * splash baseline from a block mask (danielwatson6.github.io/fa, "Our first
 * kernel": MultiHeadMask handed to process_mask) that classifies every
 * (query block, key block) pair as empty, partial or full, and apple/axlearn
 * PR 845 generates such masks lazily. The same classification is made here
 * from the closed form, per key tile: empty tiles are never visited, full
 * ones take no element mask, only partial ones do.
 *   causal         0, 1 (top-left) or 2 (end-aligned), as for attn_fwd
 *   window_left,
 *   window_right   band sides, -1 = unbounded (as attn_fwd_local)
 *   prefix         keys s < prefix are visible to every query of the row,
 *                  whatever the causal rule and the band say (bidirectional
 *                  over a prefix, causal after it: a prefix-LM; with a band
 *                  it keeps a few leading keys global). 0 = none.
 *   workspace      as attn_fwd_ws (decoding shapes split the key range)
 * Errors as attn_fwd_ws, plus ERR_MASK for an invalid causal mode, window
 * side or prefix. */
int attn_fwd_mask(const void *q, const void *k, const void *v, void *o, float *lse,
                  const int32_t *q_seg, const int32_t *kv_seg,
                  int B, int K, int G, int T, int S, int H, int causal, int window_left, int window_right, int prefix,
                  void *workspace, size_t workspace_bytes, void *stream);

/* Host-only validation of attn_fwd_mask's arguments. Same return codes; the
 * checks of attn_check_fwd (same passages) plus the mask arguments. */
int attn_check_fwd_mask(const void *q, const void *k, const void *v, const void *o, const float *lse,
                        const int32_t *q_seg, const int32_t *kv_seg,
                        int B, int K, int G, int T, int S, int H, int causal, int window_left, int window_right,
                        int prefix, const void *workspace, size_t workspace_bytes);

/* Forward pass with an explicit schedule: attn_fwd_mask with the caller's
 * choice of the two schedule parameters the library otherwise takes from its
 * tuning table (attn_fwd_tuning). The pages' kernels take their block sizes
 * from the caller, with a default getter whose heuristic is left as a TODO
 * (fjformer page, "BlockSizes dataclass": BlockSizes and get_default; the
 * block-size sweep of danielwatson6.github.io/fa, "Optimizing the kernel").
 * Here the tile shapes are fixed per head size and kernel; what varies per
 * shape is:
 *   load_placement  where a ping-pong forward wave issues its K/V tile loads:
 *                   0 in its softmax phase, 1 at the start of its MFMA phase,
 *                   2 spread over its MFMA phase; -1 = the table's choice
 *   split_target    the workgroups the split-KV plan aims for when the grid is
 *                   small (0 = never split, at most 2^20); -1 = the table's
 * Neither changes the arithmetic: every choice gives bitwise the same O and
 * lse. The workspace must hold attn_fwd_tuned_workspace_bytes(...,
 * split_target). Errors as attn_fwd_mask, plus ERR_TUNING for a choice out of
 * range. */
int attn_fwd_tuned(const void *q, const void *k, const void *v, void *o, float *lse,
                   const int32_t *q_seg, const int32_t *kv_seg,
                   int B, int K, int G, int T, int S, int H, int causal, int window_left, int window_right, int prefix,
                   int load_placement, int split_target, void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes of attn_fwd_tuned for a split target (-1: the table's, the
 * same as attn_fwd_workspace_bytes). 0 when the plan does not split or for
 * invalid arguments. Library convention (no passage). */
size_t attn_fwd_tuned_workspace_bytes(int B, int K, int G, int T, int S, int H, int split_target);

/* The tuning table's schedule for a call (host only): the role of get_default
 * in fjformer's BlockSizes dataclass, filled from measured sweeps on MI355X
 * instead of a fixed default. segments: nonzero when segment ids are given.
 * Writes load_placement and split_target; returns 0, or ERR_NULL / ERR_SHAPE /
 * ERR_HEADDIM / ERR_MASK for invalid arguments. */
int attn_fwd_tuning(int B, int K, int G, int T, int S, int H, int causal, int window_left, int window_right,
                    int prefix, int segments, int *load_placement, int *split_target);

/* Bytes of device workspace attn_bwd needs for these sizes: the per-row
 * D = sum_s P[t,s] dP[t,s] vector, fp32 [B,K,G,T], then lse * log2(e) in the
 * same layout (the form the dK/dV kernel consumes), each rounded up to 256
 * bytes. Returns 0 for invalid sizes. The pages give no backward; D is the row
 * quantity of the softmax derivative, kept beside the lse residual that
 * splash attention's save_residuals returns (danielwatson6.github.io/fa,
 * "Our first kernel"). */
size_t attn_bwd_workspace_bytes(int B, int K, int G, int T, int S, int H);

/* Backward pass: gradients of sum(O * dO) with respect to the pre-scaled q,
 * and k, v. The weights are recomputed from the saved lse (the role splash
 * attention's save_residuals plays on the danielwatson6.github.io/fa page);
 * dK/dV and dQ are computed by separate kernels, as the separate *_dkv and
 * *_dq block sizes of the fjformer BlockSizes dataclass suggest.
 *   q, k, v, dO      bf16, layouts above
 *   o                the forward output, or NULL: it is not read. D =
 *                    rowsum(dO * O) is instead summed in fp32 as
 *                    sum_s P dP from the recomputed weights, because the
 *                    bf16 O carries the forward's bf16 rounding of P and a
 *                    D taken from it moves dQ by up to ~1e-1 on early
 *                    causal rows
 *   lse              fp32 [B,K,G,T] from attn_fwd on the same inputs (required)
 *   dq               fp32 [B,K,G,T,H] (written)
 *   dk, dv           fp32 [B,K,S,H]   (written; summed over the G query heads)
 *   workspace        device buffer of at least attn_bwd_workspace_bytes(),
 *                    16-byte aligned, owned by the caller, contents ignored
 * Errors as attn_fwd (with dq in the role of o), plus ERR_NULL for
 * lse/dO/dq/dk/dv, ERR_ALIGN for a misaligned non-NULL o, and ERR_WORKSPACE.
 * Enqueues three kernels on `stream`: the D pass, dQ, then dK/dV. */
int attn_bwd(const void *q, const void *k, const void *v, const void *o, const float *lse,
             const void *dO, float *dq, float *dk, float *dv,
             const int32_t *q_seg, const int32_t *kv_seg,
             int B, int K, int G, int T, int S, int H, int causal,
             void *workspace, size_t workspace_bytes, void *stream);

/* Backward pass of attn_fwd_local: the same window (window_left, window_right,
 * -1 unbounded) restricts every recomputed weight, and the kernels visit only
 * the tiles inside the band. Otherwise as attn_bwd; window sides below -1 ->
 * ERR_MASK. Equal to attn_bwd_mask with prefix 0. */
int attn_bwd_local(const void *q, const void *k, const void *v, const void *o, const float *lse,
                   const void *dO, float *dq, float *dk, float *dv,
                   const int32_t *q_seg, const int32_t *kv_seg,
                   int B, int K, int G, int T, int S, int H, int causal, int window_left, int window_right,
                   void *workspace, size_t workspace_bytes, void *stream);

/* Host-only validation of attn_bwd_local's arguments. Same return codes; the
 * checks of attn_check_bwd plus the window sides. */
int attn_check_bwd_local(const void *q, const void *k, const void *v, const void *o, const float *lse,
                         const void *dO, const float *dq, const float *dk, const float *dv,
                         const int32_t *q_seg, const int32_t *kv_seg,
                         int B, int K, int G, int T, int S, int H, int causal, int window_left, int window_right,
                         const void *workspace, size_t workspace_bytes);

/* Backward pass of attn_fwd_mask: the same mask (causal mode, window sides,
 * prefix) restricts every recomputed weight, and the kernels visit only the
 * tiles that hold a visible pair. Otherwise as attn_bwd; an invalid mask
 * argument -> ERR_MASK. */
int attn_bwd_mask(const void *q, const void *k, const void *v, const void *o, const float *lse,
                  const void *dO, float *dq, float *dk, float *dv,
                  const int32_t *q_seg, const int32_t *kv_seg,
                  int B, int K, int G, int T, int S, int H, int causal, int window_left, int window_right, int prefix,
                  void *workspace, size_t workspace_bytes, void *stream);

/* Host-only validation of attn_bwd_mask's arguments. Same return codes; the
 * checks of attn_check_bwd plus the mask arguments. */
int attn_check_bwd_mask(const void *q, const void *k, const void *v, const void *o, const float *lse,
                        const void *dO, const float *dq, const float *dk, const float *dv,
                        const int32_t *q_seg, const int32_t *kv_seg,
                        int B, int K, int G, int T, int S, int H, int causal, int window_left, int window_right,
                        int prefix, const void *workspace, size_t workspace_bytes);

/* Host-only validation of attn_bwd's arguments. Same return codes. Like
 * attn_check_fwd it stands in for the fused kernel wrapper's shape asserts
 * (danielwatson6.github.io/fa, "Optimizing the kernel") and for the
 * ValueError of fjformer's BlockSizes dataclass, whose separate *_dkv and *_dq
 * block sizes are the two backward kernels validated here. */
int attn_check_bwd(const void *q, const void *k, const void *v, const void *o, const float *lse,
                   const void *dO, const float *dq, const float *dk, const float *dv,
                   const int32_t *q_seg, const int32_t *kv_seg,
                   int B, int K, int G, int T, int S, int H, int causal,
                   const void *workspace, size_t workspace_bytes);

/* Forward pass with a mask per query head: the splash baseline's
 * MultiHeadMask (danielwatson6.github.io/fa, "Our first kernel") holds one
 * mask per head, so that local and global heads, or heads with different
 * prefixes, share one call. Query head (k, g) takes the mask of attn_fwd_mask
 * with its own window sides and prefix from the table; the causal mode and
 * segment ids apply to every head.
 *   head_mask   device int32 [K][G][3], 4-byte aligned, owned by the caller:
 *               head_mask[(k G + g) 3 + 0] window_left, + 1 window_right,
 *               + 2 prefix. A negative side is unbounded; a prefix is
 *               clamped to [0, S]. Every value is accepted (the host cannot
 *               read device memory), normalised in the kernels as the
 *               single-mask calls normalise theirs.
 * Runs the general kernel, one pass (no split, no workspace): it visits a
 * block's key tiles inside the union of its heads' bands and prefixes, and
 * each wave masks with its own head's. Errors as attn_fwd, plus ERR_NULL /
 * ERR_ALIGN for head_mask. */
int attn_fwd_head_masks(const void *q, const void *k, const void *v, void *o, float *lse,
                        const int32_t *q_seg, const int32_t *kv_seg,
                        int B, int K, int G, int T, int S, int H, int causal, const int32_t *head_mask,
                        void *stream);

/* Host-only validation of attn_fwd_head_masks' arguments. Same return codes. */
int attn_check_fwd_head_masks(const void *q, const void *k, const void *v, const void *o, const float *lse,
                              const int32_t *q_seg, const int32_t *kv_seg,
                              int B, int K, int G, int T, int S, int H, int causal, const int32_t *head_mask);

/* Backward pass of attn_fwd_head_masks: every recomputed weight of head
 * (k, g) takes that head's mask. Otherwise as attn_bwd (its workspace
 * included); it runs the general dQ and dK / dV kernels. */
int attn_bwd_head_masks(const void *q, const void *k, const void *v, const void *o, const float *lse,
                        const void *dO, float *dq, float *dk, float *dv,
                        const int32_t *q_seg, const int32_t *kv_seg,
                        int B, int K, int G, int T, int S, int H, int causal, const int32_t *head_mask,
                        void *workspace, size_t workspace_bytes, void *stream);

/* Host-only validation of attn_bwd_head_masks' arguments. Same return codes. */
int attn_check_bwd_head_masks(const void *q, const void *k, const void *v, const void *o, const float *lse,
                              const void *dO, const float *dq, const float *dk, const float *dv,
                              const int32_t *q_seg, const int32_t *kv_seg,
                              int B, int K, int G, int T, int S, int H, int causal, const int32_t *head_mask,
                              const void *workspace, size_t workspace_bytes);

/* Forward pass that allocates nothing, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid hipMalloc. Same arguments and result as
 * attn_fwd_mask minus the workspace: when the shape splits the key range
 * (decoding shapes, as attn_fwd_ws), the partial outputs and lse go to a
 * static device array of the library, 16 MiB per GPU (2^24 bytes), held from
 * the first call on a device until the process ends. A shape whose
 * attn_fwd_workspace_bytes() exceeds 16 MiB returns ERR_WORKSPACE before
 * anything is launched. The call makes no hipMalloc / hipFree or other
 * allocating call; its first call on a device looks up that device's copy of
 * the array (hipGetSymbolAddress). Every call on one GPU shares that GPU's
 * array: calls that overlap on one GPU (concurrent streams) race and must be
 * serialised by the caller. Each split writes every row it owns, so no state
 * carries over from one call to the next. */
int attn_fwd_noalloc(const void *q, const void *k, const void *v, void *o, float *lse,
                     const int32_t *q_seg, const int32_t *kv_seg,
                     int B, int K, int G, int T, int S, int H, int causal, int window_left, int window_right,
                     int prefix, void *stream);

/* Static, NUL-terminated description of a return code. Never NULL. It plays
 * the part of the message text of the BlockSizes ValueError (fjformer page,
 * "BlockSizes dataclass"); the Python binding raises it as a ValueError. */
const char *attn_strerror(int code);

/* The hipError_t behind the calling thread's most recent GQA_ATTN_ERR_HIP
 * (0 if none). Library convention, no passage of the pages. */
int attn_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GQA_ATTN_H */
