// Fused grouped-query flash attention, forward pass, for gfx950 (MI355X).
//
// Method (danielwatson6.github.io/fa): "Chunked attention" gives the
// numerically stable scan over key chunks -- a running row maximum m, a
// running denominator and an output carry rescaled by exp(m_old - m_new) --
// and "Optimizing the kernel" fuses the key loop into one kernel whose carries
// never leave the chip and whose output is written once, in bf16. Masks are
// generated lazily (apple/axlearn PR 845): causal and segment-id visibility
// are evaluated from indices, and whole key tiles that no query of a block
// can see are never visited.
//
// Work decomposition. One workgroup owns one (batch b, kv head k, group of
// gw query heads, block of bq queries) unit: gw*bq query rows, 32 per wave.
// All gw heads of the unit read the same K/V tiles (the page's kernel sees
// the G axis inside each (b, kv head) program), so every K/V tile is staged
// into LDS once per workgroup and consumed by all of its waves.
//
// Per wave, per key tile of BKV keys:
//   S^T = K_tile Q^T  : bf16 MFMA 32x32x16, K from LDS (A operand),
//                       Q^T resident in registers (B operand)
//   each lane owns one query column of S^T (its half of the keys; the other
//   half sits in lane ^ 32), so the row max and row sum are in-lane plus one
//   cross-half exchange
//   P = exp2(S*log2e - m), carries rescaled by exp2(m_old - m_new)
//   O^T += V_tile^T P^T : bf16 MFMA, P^T straight from the S^T registers
//                         (B operand), V^T via the LDS transpose read
#include "gqa_device.h"
#include "gqa_launch.h"

#include <algorithm>
#include <atomic>
#include <climits>
#include <cmath>
#include <type_traits>
#include <utility>

// LDS operand reads run this many MFMAs ahead of their use: in the general
// kernel's dense loop, and in the ping-pong kernel's M phase (in steps)
constexpr int kFwdPrefetch = 2;

namespace gqa {

// Interleave pattern of one dense-loop iteration for the machine scheduler.
// MFMA slot m: the MFMA, the LDS operand reads of MFMA m + D (one b128 read of
// K for each of the N_QK QK^T MFMAs, two transpose reads of V for each PV
// MFMA), then VALU_PER VALU instructions of the weight computation.
template <int M, int N_QK, int N_MFMA>
__device__ __forceinline__ void sched_operand_reads() {
    if constexpr (M < N_MFMA) __builtin_amdgcn_sched_group_barrier(0x100, (M < N_QK) ? 1 : 2, 0);
}
template <int M, int N_QK, int N_MFMA, int D, int VALU_PER>
__device__ __forceinline__ void sched_slot() {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    sched_operand_reads<M + D, N_QK, N_MFMA>();
    __builtin_amdgcn_sched_group_barrier(0x002, VALU_PER, 0);
}
template <int N_QK, int N_MFMA, int D, int VALU_PER, int... P, int... M>
__device__ __forceinline__ void dense_schedule(std::integer_sequence<int, P...>, std::integer_sequence<int, M...>) {
    (sched_operand_reads<P, N_QK, N_MFMA>(), ...);
    (sched_slot<M, N_QK, N_MFMA, D, VALU_PER>(), ...);
}

// DENSE: no segment ids, window or prefix, whole key tiles (S % BKV == 0)
// and, when causal, T + coff == S with one query block per key tile (bq ==
// BKV) and the diagonal offset a whole number of tiles: only the last tile of
// a block (its diagonal) needs an element mask, and the key loop has scalar
// control and a branch-free steady state.
template <int H, int BKV, int NW, int WAVES_PER_SIMD, bool CAUSAL, bool DENSE>
__global__ __launch_bounds__(NW * 64, WAVES_PER_SIMD) void attn_fwd_kernel(FwdArgs a) {
    constexpr int CPR = H / 8;        // 16-byte chunks per K/V row
    constexpr int KSTEPS = H / 16;    // k-steps of the QK^T contraction
    constexpr int MB = BKV / 32;      // 32-key blocks per tile
    constexpr int HB = H / 32;        // 32-wide h blocks of O^T
    constexpr int PK = BKV / 16;      // k-steps of the PV contraction
    using L = TileLayout<H, BKV>;

    // K and V tiles, two buffers each (see the pipeline below), in padded-row
    // layouts that make every MFMA operand read bank-conflict free.
    __shared__ __attribute__((aligned(1024))) __bf16 sk0[L::K_ELEMS];
    __shared__ __attribute__((aligned(1024))) __bf16 sk1[L::K_ELEMS];
    __shared__ __attribute__((aligned(1024))) __bf16 sv0[L::V_ELEMS];
    __shared__ __attribute__((aligned(1024))) __bf16 sv1[L::V_ELEMS];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31, c = lane >> 5;

    // ---- work unit; causal blocks are issued heaviest (last query block) first;
    // with split-KV the grid holds one copy per split
    const int units = a.B * a.K * a.n_gsplit;
    const int per_split = units * a.n_qblocks;
    const int split = a.o_part ? (int)blockIdx.x / per_split : 0;
    const int bid = a.o_part ? (int)blockIdx.x % per_split : (int)blockIdx.x;
    int qb = bid / units;
    if (CAUSAL) qb = a.n_qblocks - 1 - qb;
    const int u = bid % units;
    const int gs = u % a.n_gsplit;
    const int kh = (u / a.n_gsplit) % a.K;
    const int b = u / (a.n_gsplit * a.K);
    const int t0 = qb * a.bq;
    const int T = a.T, S = a.S;

    // ---- this lane's query row (column n of the wave's S^T tile)
    const int rows_wg = a.gw * a.bq;
    const int rho = wave * 32 + n;
    const bool row_in_wg = rho < rows_wg;
    const int g = gs * a.gw + (row_in_wg ? rho / a.bq : 0);
    const int t = t0 + (row_in_wg ? rho % a.bq : 0);
    const bool q_valid = row_in_wg && t < T;
    const bool wave_active = wave * 32 < rows_wg;
    const int tmin_w = t0 + (a.bq >= 32 ? (wave * 32) % a.bq : 0);
    const int tmax_w = tmin_w + (a.bq >= 32 ? 31 : a.bq - 1);

    const size_t bk = (size_t)b * a.K + kh;
    const size_t qrow_off = ((bk * a.G + g) * (size_t)T + t) * H;

    // Q^T operand: lane (n, c), k-step ks holds q[t][16ks + 8c .. +7]
    bf16x8 qf[KSTEPS];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ks++) {
        if (q_valid)
            qf[ks] = *(const bf16x8 *)(a.q + qrow_off + 16 * ks + 8 * c);
        else
            qf[ks] = bf16x8{};
    }

    // K and V of this (b, kv head) as bounds-checked buffers: rows past S read as zero
    const buffer_rsrc krs = make_rsrc(a.k + bk * (size_t)S * H, S * H * 2);
    const buffer_rsrc vrs = make_rsrc(a.v + bk * (size_t)S * H, S * H * 2);

    // ---- segment ids: this lane's query id and the workgroup / wave id ranges
    const bool segs = !DENSE && a.q_seg != nullptr;
    const int32_t *kvs = segs ? a.kv_seg + (size_t)b * S : nullptr;
    int my_qid = 0, wg_qmin = INT_MAX, wg_qmax = INT_MIN, w_qmin = INT_MAX, w_qmax = INT_MIN;
    if (segs) {
        const int32_t *qs = a.q_seg + (size_t)b * T;
        int lo = INT_MAX, hi = INT_MIN;
        for (int i = lane; i < a.bq; i += 64) {
            if (t0 + i < T) {
                int id = qs[t0 + i];
                lo = min(lo, id);
                hi = max(hi, id);
            }
        }
        wg_qmin = wave_min_i(lo);
        wg_qmax = wave_max_i(hi);
        my_qid = q_valid ? qs[t] : 0;
        w_qmin = wave_min_i(q_valid ? my_qid : INT_MAX);
        w_qmax = wave_max_i(q_valid ? my_qid : INT_MIN);
    }

    // ---- the mask sides: WL, WR, PFX of this wave's head (its 32 rows are one
    // head: bq is a multiple of 32), and WLu, WRu, PFXu of the union over the
    // block's heads, which bound its key range. Without per-head masks all are
    // the call's.
    int WL = a.wl, WR = a.wr, PFX = a.prefix;
    int WLu = WL, WRu = WR, PFXu = PFX;
    if (!DENSE && a.head_mask) {
        const HeadMask hw = head_mask_of(a.head_mask, kh, a.G, __builtin_amdgcn_readfirstlane(g), T, S, a.causal,
                                         a.coff);
        WL = hw.wl, WR = hw.wr, PFX = hw.pfx;
        WLu = WRu = INT_MIN;
        PFXu = 0;
        for (int i = 0; i < a.gw; i++) {
            const HeadMask h = head_mask_of(a.head_mask, kh, a.G, gs * a.gw + i, T, S, a.causal, a.coff);
            WLu = max(WLu, h.wl);
            WRu = max(WRu, h.wr);
            PFXu = max(PFXu, h.pfx);
        }
    }

    // ---- key-tile range: the band [t - WLu, t + WRu] of the block's first and
    // last query, and the prefix keys s < PFXu; a split covers its own range
    const int n_tiles = (S + BKV - 1) / BKV;
    const int t_last = min(t0 + a.bq, T) - 1;  // the block's last query
    const int s_last = max(min(t_last + WRu, S - 1), PFXu - 1);
    int j_end = s_last < 0 ? 0 : min(n_tiles, s_last / BKV + 1);
    int j_begin = (PFXu > 0 || t0 - WLu <= 0) ? 0 : (t0 - WLu) / BKV;
    if (!DENSE && a.o_part) {
        j_begin = max(j_begin, split * a.split_tiles);
        j_end = min(j_end, split * a.split_tiles + a.split_tiles);
    }

    // ---- kv ids of the block's key range staged in LDS (8-wave copies, up to
    // KV_CAP keys), with each tile's id range: inside the key loop a global
    // load of ids would be counted behind the tile loads just issued, and
    // waiting for it would wait for them too.
    constexpr int KV_CAP = NW == 8 ? 4096 : 1;
    constexpr int KV_TILES = KV_CAP / BKV > 0 ? KV_CAP / BKV : 1;
    __shared__ int s_kvid[KV_CAP];
    __shared__ int s_tmin[KV_TILES], s_tmax[KV_TILES];
    const int kv_base = j_begin * BKV;
    const bool kv_lds = segs && NW == 8 && j_end > j_begin && (j_end - j_begin) * BKV <= KV_CAP;
    if (kv_lds) {
        for (int jj = j_begin + wave; jj < j_end; jj += NW) {
            const int s = jj * BKV + lane;
            const bool ok = lane < BKV && s < S;
            const int id = ok ? kvs[s] : 0;
            if (ok) s_kvid[s - kv_base] = id;
            const int lo = wave_min_i(ok ? id : INT_MAX);
            const int hi = wave_max_i(ok ? id : INT_MIN);
            if (lane == 0) {
                s_tmin[jj - j_begin] = lo;
                s_tmax[jj - j_begin] = hi;
            }
        }
        __syncthreads();
    }

    // kv-id range of tile j (wave-uniform; every wave computes the same value)
    auto tile_ids = [&](int j, int &kmin, int &kmax) {
        if (kv_lds) {
            kmin = __builtin_amdgcn_readfirstlane(s_tmin[j - j_begin]);
            kmax = __builtin_amdgcn_readfirstlane(s_tmax[j - j_begin]);
            return;
        }
        const int s = j * BKV + lane;
        int id = 0;
        const bool ok = lane < BKV && s < S;
        if (ok) id = kvs[s];
        kmin = wave_min_i(ok ? id : INT_MAX);
        kmax = wave_max_i(ok ? id : INT_MIN);
    };
    // next tile at or after j that some query of the workgroup can see: inside
    // the prefix or the block's band, and (segment ids) sharing an id range
    auto next_tile = [&](int j) {
        if (!segs && PFXu == 0) return j;
        for (; j < j_end; j++) {
            const int s0 = j * BKV;
            if (!(s0 < PFXu || (s0 + BKV - 1 >= t0 - WLu && s0 <= t_last + WRu))) continue;
            if (segs) {
                int kmin, kmax;
                tile_ids(j, kmin, kmax);
                if (kmax < wg_qmin || kmin > wg_qmax) continue;
            }
            break;
        }
        return j;
    };
    // does this wave compute tile j, and does it need an element mask there
    auto tile_flags = [&](int j, bool &run, bool &mask) {
        const int s0 = j * BKV;
        run = j < j_end && wave_active && (s0 < PFX || (s0 <= tmax_w + WR && s0 + BKV - 1 >= tmin_w - WL));
        bool seg_mask = false;
        if (run && segs) {
            int kmin, kmax;
            tile_ids(j, kmin, kmax);
            if (kmax < w_qmin || kmin > w_qmax) run = false;
            seg_mask = !(w_qmin == w_qmax && kmin == kmax && kmin == w_qmin);
        }
        // a tile wholly inside the prefix needs no band mask
        const bool band_mask = s0 + BKV - 1 >= PFX && ((s0 + BKV - 1 > tmin_w + WR) || (s0 < tmax_w - WL));
        mask = band_mask || (s0 + BKV > S) || seg_mask;
    };

    // One tile of K (row stride L::KRS chunks) or V (L::VRS) into LDS, straight
    // from memory (no registers). Wave load blk writes the 64 consecutive
    // 16-byte slots blk*64 .. blk*64+63; slot p holds chunk p % RS of key row
    // p / RS, and the padding slots (chunk >= CPR) repeat the row's last chunk.
    // This wave issues loads blk = wave, wave + NW, ...; their per-lane byte
    // offsets within a tile are fixed, and the tile's own offset is added to
    // them (the range check zero-fills the rows of a last, partial tile past S).
    constexpr int K_PER_WAVE = (L::K_BLOCKS + NW - 1) / NW;
    constexpr int V_PER_WAVE = (L::V_BLOCKS + NW - 1) / NW;
    int k_off[K_PER_WAVE], v_off[V_PER_WAVE];
#pragma unroll
    for (int i = 0; i < K_PER_WAVE; i++) {
        const int p = (wave + i * NW) * 64 + lane;
        k_off[i] = ((p / L::KRS) * H + min(p % L::KRS, CPR - 1) * 8) * 2;
    }
#pragma unroll
    for (int i = 0; i < V_PER_WAVE; i++) {
        const int p = (wave + i * NW) * 64 + lane;
        v_off[i] = ((p / L::VRS) * H + min(p % L::VRS, CPR - 1) * 8) * 2;
    }
    const unsigned wave_slot = wave * 1024;  // this wave's first 1 KiB block
    // Loads i < K_FULL (V_FULL) are issued by every wave; the rest only by the
    // first waves (wave-uniform branches).
    constexpr int K_FULL = L::K_BLOCKS / NW;
    constexpr int V_FULL = L::V_BLOCKS / NW;
    auto issue_k_part = [&](int j, const __bf16 *dst, auto full) {
        const int tile = __builtin_amdgcn_readfirstlane(j * BKV * H * 2);
        char *base = (char *)dst + wave_slot;
#pragma unroll
        for (int i = 0; i < K_PER_WAVE; i++) {
            if constexpr (decltype(full)::value) {
                if (i < K_FULL) lds_load16_to(krs, base + i * NW * 1024, k_off[i] + tile);
            } else {
                if (i >= K_FULL && wave + i * NW < L::K_BLOCKS) lds_load16_to(krs, base + i * NW * 1024, k_off[i] + tile);
            }
        }
    };
    auto issue_v_part = [&](int j, const __bf16 *dst, auto full) {
        const int tile = __builtin_amdgcn_readfirstlane(j * BKV * H * 2);
        char *base = (char *)dst + wave_slot;
#pragma unroll
        for (int i = 0; i < V_PER_WAVE; i++) {
            if constexpr (decltype(full)::value) {
                if (i < V_FULL) lds_load16_to(vrs, base + i * NW * 1024, v_off[i] + tile);
            } else {
                if (i >= V_FULL && wave + i * NW < L::V_BLOCKS) lds_load16_to(vrs, base + i * NW * 1024, v_off[i] + tile);
            }
        }
    };
    using all_waves_t = std::integral_constant<bool, true>;
    using first_waves_t = std::integral_constant<bool, false>;
    auto issue_k = [&](int j, const __bf16 *dst) {
        issue_k_part(j, dst, all_waves_t{});
        issue_k_part(j, dst, first_waves_t{});
    };
    auto issue_v = [&](int j, const __bf16 *dst) {
        issue_v_part(j, dst, all_waves_t{});
        issue_v_part(j, dst, first_waves_t{});
    };

    // S^T = K_tile Q^T for one tile: lane reads row 32mb + n, chunk 2ks + c
    const int k_lane = n * L::KRS * 8 + c * 8;
    auto qk = [&](const __bf16 *kt, f32x16 (&sacc)[MB]) {
#pragma unroll
        for (int mb = 0; mb < MB; mb++) {
            sacc[mb] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ks++) {
                const bf16x8 kf = *(const bf16x8 *)(kt + k_lane + mb * 32 * L::KRS * 8 + ks * 16);
                sacc[mb] = mfma32x32x16(kf, qf[ks], sacc[mb]);
            }
        }
    };

    f32x16 oacc[HB];
#pragma unroll
    for (int hb = 0; hb < HB; hb++) oacc[hb] = f32x16{};
    float m_run = -INFINITY;  // reference max, log2 units
    float l_run = 0.f;        // running denominator over this lane's half of the keys

    // ---- per-tile pieces: lazy mask, row max + rescale, weights, PV
    // Register r of block mb holds key s0 + 32mb + acc_row(r, c); with the lane's
    // half c folded into one limit, every comparison is against a constant.
    auto mask_tile = [&](f32x16 (&sacc)[MB], int s0) {
        const int lim = min(t + WR, S - 1) - s0 - 4 * c;  // last visible key offset
        const int first = t - WL - s0 - 4 * c;           // first visible key offset
        const int plim = PFX - s0 - 4 * c;               // offsets below it are prefix keys (PFX <= S)
#pragma unroll
        for (int mb = 0; mb < MB; mb++) {
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int off = 32 * mb + 8 * (r >> 2) + (r & 3);
                bool vis = (off <= lim && off >= first) || off < plim;
                if (segs && vis) vis = (kv_lds ? s_kvid[s0 + off + 4 * c - kv_base] : kvs[s0 + off + 4 * c]) == my_qid;
                if (!vis) sacc[mb][r] = -INFINITY;
            }
        }
    };
    // Lazy rescale: the reference max m_run moves only when some row of the
    // wave grew by more than 2^kRescaleLog2. Keeping a stale reference is an
    // exact re-association (numerator and denominator carry the same factor).
    // A row's keys are split between lane n and lane n + 32; each checks its
    // own half, so the common case needs no cross-lane exchange. When some row
    // must move, both halves take the full row max, so m_run stays identical in
    // the lane pair.
    auto tile_max = [&](const f32x16 (&sacc)[MB]) {
        // four independent partial maxima (short dependency chains)
        float m4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
        for (int mb = 0; mb < MB; mb++)
#pragma unroll
            for (int r = 0; r < 16; r += 2)
                m4[(r >> 1) & 3] = max_nan(m4[(r >> 1) & 3], max_nan(sacc[mb][r], sacc[mb][r + 1]));
        return max_nan(max_nan(m4[0], m4[1]), max_nan(m4[2], m4[3]));
    };
    auto rescale = [&](float mx) {
        mx = max_nan(mx, __shfl_xor(mx, 32));
        const float m_new = max_nan(m_run, mx * kLog2e);
        const float corr = (m_new == -INFINITY) ? 1.f : exp2_fast(m_run - m_new);
        l_run *= corr;
#pragma unroll
        for (int hb = 0; hb < HB; hb++) oacc[hb] *= corr;
        m_run = m_new;
    };
    // returns the reference the weights are taken against
    auto rowmax_rescale = [&](const f32x16 (&sacc)[MB]) {
        const float mx = tile_max(sacc);
        if (__any(mx * kLog2e > m_run + kRescaleLog2)) rescale(mx);
        return (m_run == -INFINITY) ? 0.f : m_run;
    };
    // P = exp2(S log2e - m) in bf16 (the PV operand); returns this lane's part
    // of the fp32 row sum
    auto weights = [&](const f32x16 (&sacc)[MB], float m_use, bf16x8 (&pf)[PK]) {
        float rs[4] = {0.f, 0.f, 0.f, 0.f};  // independent partial sums
#pragma unroll
        for (int kk = 0; kk < PK; kk++) {
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                const float p0 = exp2_fast(__builtin_fmaf(sacc[kk >> 1][8 * (kk & 1) + e], kLog2e, -m_use));
                const float p1 = exp2_fast(__builtin_fmaf(sacc[kk >> 1][8 * (kk & 1) + e + 1], kLog2e, -m_use));
                pf[kk][e] = (__bf16)p0;
                pf[kk][e + 1] = (__bf16)p1;
                rs[e >> 1] += p0 + p1;
            }
        }
        return (rs[0] + rs[1]) + (rs[2] + rs[3]);
    };
    // O^T += V^T P^T; V^T from two transpose reads per MFMA. Source lane gi of
    // each 16-lane group addresses key row 16kk + 8e + 4c + gi/4 at
    // h = 32hb + 16hh + 4(gi%4), so lane l receives h = 32hb + l%32 for the
    // four keys 16kk + 8e + 4c + (0..3) -- the keys of its P^T slots.
    const int v_lane = (4 * c + ((lane & 15) >> 2)) * L::VRS * 8 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    auto pv = [&](const bf16x8 (&pf)[PK], const __bf16 *vt) {
#pragma unroll
        for (int kk = 0; kk < PK; kk++) {
#pragma unroll
            for (int hb = 0; hb < HB; hb++) {
                const __bf16 *vp = vt + v_lane + kk * 16 * L::VRS * 8 + hb * 32;
                const s16x4 lo = lds_read_tr16(vp);
                const s16x4 hi = lds_read_tr16(vp + 8 * L::VRS * 8);
                oacc[hb] = mfma32x32x16(join_bf16x8(lo, hi), pf[kk], oacc[hb]);
            }
        }
    };
    auto softmax_pv = [&](f32x16 (&sacc)[MB], const __bf16 *vt) {
        const float m_use = rowmax_rescale(sacc);
        bf16x8 pf[PK];
        l_run += weights(sacc, m_use, pf);
        pv(pf, vt);
    };

    if constexpr (DENSE) {
        // ---- dense pipeline over tiles 0 .. n_t-1, two stages deep.
        // Iteration i (0 <= i < n_t - 1) issues the QK^T MFMAs of tile i+1 and the
        // PV MFMAs of tile i-1, and between them computes the weights of tile i,
        // so every MFMA of the iteration has VALU work beside it. Tile i+1's K and
        // tile i-1's V are read from LDS while K(i+2) and V(i) are being loaded
        // into the buffers that held K(i) and V(i-2).
        //
        // Buffer and register roles alternate between iterations; "A" iterations
        // (even i) hold S(i) in sa and P(i) in pa and read (kB, vB), "B" iterations
        // the other halves. The last iteration always runs in the A roles: when
        // n_t - 1 is odd, its S and the previous P are copied over once and the
        // buffer pointers are swapped (uniform values).
        // causal: the diagonal tile qb + coff / BKV is the block's last
        const int n_t = CAUSAL ? qb + 1 + a.coff / BKV : S / BKV;
        f32x16 sa[MB], sb[MB];
        bf16x8 pa[PK], pb[PK];
        const __bf16 *kA = sk0, *kB = sk1, *vA = sv0, *vB = sv1;
        issue_k(0, kA);
        if (n_t > 1) issue_k(1, kB);
        wait_lds_loads();
        __syncthreads();
        qk(kA, sa);

        // Weights of a tile with no masked key. The rescale test needs no row max:
        // weights are >= 0, so a lane whose weights sum to at most 2^kRescaleLog2
        // has none above that bound. Only when some lane's sum exceeds it (or is
        // inf / NaN, as on the first tile, whose reference is -inf) does the wave
        // take the row max, rescale and recompute. A sum can pass the bound while
        // every weight is below it; the rescale is exact either way.
        auto mid = [&](auto with_pv, f32x16 (&s_cur)[MB], f32x16 (&s_nxt)[MB], const bf16x8 (&p_prev)[PK],
                       bf16x8 (&p_cur)[PK], const __bf16 *k_rd, const __bf16 *k_ld, const __bf16 *v_rd,
                       const __bf16 *v_ld, int i) {
            wait_lds_loads();
            __syncthreads();
            // the loads every wave issues go into the MFMA stream below (the
            // scheduler spreads them); K(i+2) past the last tile is a dead load,
            // or a bounds-checked zero read past the end of K
            if (i + 2 < n_t) issue_k_part(i + 2, k_ld, first_waves_t{});
            issue_v_part(i, v_ld, first_waves_t{});
            __builtin_amdgcn_s_setprio(1);
            issue_k_part(i + 2, k_ld, all_waves_t{});
            issue_v_part(i, v_ld, all_waves_t{});
            qk(k_rd, s_nxt);
            if constexpr (decltype(with_pv)::value) pv(p_prev, v_rd);
            float ls = weights(s_cur, m_run, p_cur);
            constexpr int n_qk = MB * KSTEPS;
            constexpr int n_mfma = n_qk + (decltype(with_pv)::value ? PK * HB : 0);
            constexpr int valu_per = (3 * MB * 16 + n_mfma - 1) / n_mfma;
            dense_schedule<n_qk, n_mfma, kFwdPrefetch, valu_per>(std::make_integer_sequence<int, kFwdPrefetch>(),
                                                                        std::make_integer_sequence<int, n_mfma>());
            // a rescale in here multiplies O after the PV above has been added:
            // P(i-1) was taken against the old reference
            if (__any(!(ls <= kRescaleBound))) {
                rescale(tile_max(s_cur));
                ls = weights(s_cur, m_run, p_cur);
            }
            l_run += ls;
            __builtin_amdgcn_s_setprio(0);
        };
        using no_pv = std::integral_constant<bool, false>;
        using do_pv = std::integral_constant<bool, true>;
        if (n_t > 1) {
            mid(no_pv{}, sa, sb, pb, pa, kB, kA, vB, vA, 0);
            int i = 1;
            while (i + 1 < n_t - 1) {
                mid(do_pv{}, sb, sa, pa, pb, kA, kB, vA, vB, i);
                mid(do_pv{}, sa, sb, pb, pa, kB, kA, vB, vA, i + 1);
                i += 2;
            }
            if (i < n_t - 1) mid(do_pv{}, sb, sa, pa, pb, kA, kB, vA, vB, i++);
            if (i & 1) {
#pragma unroll
                for (int mb = 0; mb < MB; mb++) sa[mb] = sb[mb];
#pragma unroll
                for (int kk = 0; kk < PK; kk++) pb[kk] = pa[kk];
                const __bf16 *t = kA;
                kA = kB;
                kB = t;
                t = vA;
                vA = vB;
                vB = t;
            }
            // last tile (the diagonal one when causal): PV of the tile before it,
            // then its own mask, weights and PV
            wait_lds_loads();
            __syncthreads();
            issue_v(n_t - 1, vA);
            __builtin_amdgcn_s_setprio(1);
            pv(pb, vB);
            if (CAUSAL) mask_tile(sa, (n_t - 1) * BKV);
            const float m_use = rowmax_rescale(sa);
            l_run += weights(sa, m_use, pa);
            __builtin_amdgcn_s_setprio(0);
            wait_lds_loads();
            __syncthreads();
            pv(pa, vA);
        } else {
            issue_v(0, vA);
            wait_lds_loads();
            __syncthreads();
            if (CAUSAL) mask_tile(sa, 0);
            softmax_pv(sa, vA);
        }
    } else {
        // ---- software pipeline over the visible tiles n_0 < n_1 < ...
        // Iteration i starts with S^T of n_i in registers, K of n_{i+1} and V of n_i
        // in LDS. After one barrier (every wave finished iteration i-1) it loads K of
        // n_{i+2} into the K buffer of n_i and V of n_{i+1} into the V buffer of
        // n_{i-1}, issues the QK^T MFMAs of n_{i+1} and, while they run, does the
        // softmax and PV of n_i. Even iterations use (sk0 | sk1, sv0 | sv1), odd ones
        // the swapped pairs, so S^T buffers alternate without register copies.
        int j_cur = j_begin < j_end ? next_tile(j_begin) : j_end;
        int j_nxt = j_cur < j_end ? next_tile(j_cur + 1) : j_end;
        if (j_cur < j_end) {
            issue_k(j_cur, sk0);
            issue_v(j_cur, sv0);
        }
        if (j_nxt < j_end) issue_k(j_nxt, sk1);
        wait_lds_loads();
        __syncthreads();
        f32x16 sa[MB], sb[MB];
        bool run_cur, mask_cur;
        tile_flags(j_cur, run_cur, mask_cur);
        if (run_cur) qk(sk0, sa);

        auto iteration = [&](f32x16 (&s_cur)[MB], f32x16 (&s_nxt)[MB], __bf16 *k_cur, __bf16 *k_nxt,
                             __bf16 *v_cur, __bf16 *v_nxt) {
            const int j_nn = j_nxt < j_end ? next_tile(j_nxt + 1) : j_end;
            wait_lds_loads();
            __syncthreads();
            if (j_nn < j_end) issue_k(j_nn, k_cur);
            if (j_nxt < j_end) issue_v(j_nxt, v_nxt);
            bool run_nxt, mask_nxt;
            tile_flags(j_nxt, run_nxt, mask_nxt);
            if (run_cur && mask_cur) mask_tile(s_cur, j_cur * BKV);
            if (run_cur && run_nxt) {
                // common case, one basic block: the QK^T MFMAs of the next tile are
                // interleaved with the exponentials of this one, so the matrix pipe
                // and the VALU work at the same time
                const float m_use = rowmax_rescale(s_cur);
                bf16x8 pf[PK];
                    __builtin_amdgcn_s_setprio(1);
                qk(k_nxt, s_nxt);
                l_run += weights(s_cur, m_use, pf);
                    pv(pf, v_cur);
                __builtin_amdgcn_s_setprio(0);
                    // schedule: K operand reads run two MFMAs ahead; each QK^T MFMA is
                // followed by a share of the weight computation; then the PV MFMAs
                // with their V transpose reads two MFMAs ahead
            } else {
                if (run_nxt) qk(k_nxt, s_nxt);
                if (run_cur) softmax_pv(s_cur, v_cur);
            }
            j_cur = j_nxt;
            j_nxt = j_nn;
            run_cur = run_nxt;
            mask_cur = mask_nxt;
            return j_cur < j_end;
        };
        if (j_cur < j_end) {
            while (iteration(sa, sb, sk0, sk1, sv0, sv1) && iteration(sb, sa, sk1, sk0, sv1, sv0)) {
            }
        }
    }

    // ---- finalize: O = acc / l in bf16, lse = ln(sum exp(logits)); a split
    // writes both in fp32 to its part of the workspace
    l_run += __shfl_xor(l_run, 32);  // the two halves of each row
    if (!DENSE && a.o_part) {
        if (q_valid) {
            const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
            const size_t row = (bk * a.G + g) * (size_t)T + t;
            const size_t rows = (size_t)a.B * a.K * a.G * T;
            float *orow = a.o_part + ((size_t)split * rows + row) * H;
#pragma unroll
            for (int hb = 0; hb < HB; hb++)
#pragma unroll
                for (int q4 = 0; q4 < 4; q4++)
                    *(f32x4 *)(orow + 32 * hb + 8 * q4 + 4 * c) =
                        f32x4{oacc[hb][4 * q4] * inv, oacc[hb][4 * q4 + 1] * inv, oacc[hb][4 * q4 + 2] * inv,
                              oacc[hb][4 * q4 + 3] * inv};
            if (c == 0) a.lse_part[(size_t)split * rows + row] = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
        }
        return;
    }
    if (q_valid) {
        const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
        __bf16 *orow = a.o + qrow_off;
#pragma unroll
        for (int hb = 0; hb < HB; hb++)
#pragma unroll
            for (int q4 = 0; q4 < 4; q4++) {
                bf16x4 val;
#pragma unroll
                for (int e = 0; e < 4; e++) val[e] = (__bf16)(oacc[hb][4 * q4 + e] * inv);
                *(bf16x4 *)(orow + 32 * hb + 8 * q4 + 4 * c) = val;
            }
        if (c == 0 && a.lse)
            a.lse[(bk * a.G + g) * (size_t)T + t] = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
    }
}



// Interleave pattern of one M phase of the ping-pong kernel: NX steps of
// NM MFMAs each (one QK^T and / or one PV MFMA), the LDS operand reads of a
// step (R reads: one b128 read of K, two transpose reads of V) issued D steps
// ahead.
template <int X, int NX, int R>
__device__ __forceinline__ void sched_m_reads() {
    if constexpr (X < NX) __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
}
template <int X, int NX, int NM, int R, int D>
__device__ __forceinline__ void sched_m_step() {
    __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
    sched_m_reads<X + D, NX, R>();
}
template <int NX, int NM, int R, int D, int... P, int... X>
__device__ __forceinline__ void m_phase_schedule(std::integer_sequence<int, P...>, std::integer_sequence<int, X...>) {
    (sched_m_reads<P, NX, R>(), ...);
    (sched_m_step<X, NX, NM, R, D>(), ...);
}

// ---------------------------------------------------------------------------
// Ping-pong forward for dense shapes (the conditions of DENSE above, 8 waves,
// one workgroup per CU): H <= 128 with 64-key tiles, and H = 256 with 32-key
// tiles when G is a multiple of 8 (8 heads by 32 queries per workgroup).
//
// The two waves of each SIMD take turns: waves 0-3 (group A) and waves 4-7
// (group B) run the same sequence of phases, B one phase behind A, with a
// workgroup barrier between phases. A wave alternates
//   M(i): the QK^T MFMAs of tile i+1 and the PV MFMAs of tile i (MFMA only)
//   V(i): the weights of tile i (exp / fma / add / convert, VALU only)
// so while one wave of a SIMD keeps the matrix pipe busy, the other does its
// softmax beside it, and a wave needs one S^T and one P^T tile of registers.
//
// Tiles move through LDS in three slots: slot i % 3 holds K(i+1) and V(i),
// the operands of M(i). During V(i) group A loads K(i+2) and group B loads
// V(i+1) into slot (i+1) % 3, whose previous contents (read by M(i-2)) are
// dead by then. Every wave waits for its own loads at the end of each of its
// M phases, one barrier before any wave reads them.
//
// Where a wave issues its tile loads (MLD): 0 in its V phase; 1 all at the
// start of its M phase; 2 spread among its M phase's MFMAs. 1 and 2 issue them
// from assembly, so that the compiler adds no wait before the phase's operand
// reads. M(i) then loads tile i+2: group A its K into slot (i+1) % 3, group B
// its V into slot (i+2) % 3, and each wave waits for them at the end of its
// next V phase. K(i+2) is first read by M(i+1), which group A starts right
// after that wait; V(i+2) by M(i+2), two phases after group B's wait. The
// slots' previous contents were last read by M(i-2) (K(i-1)) and M(i-1)
// (V(i-1)), which both groups have finished. The V phase is the longer one
// when the MFMAs per tile are few (H = 64) or the blocks short (segment ids),
// and there moving the loads out of it pays.
//
// PF (a persistent grid without segment ids, loads in the V phase): the next
// block's Q and first tiles are loaded during this block's last V phase
// (next_bid >= 0), and this block's came from the previous one (prefetched).
// The blocks of a workgroup rotate the slots: a block starts at slot base and
// leaves base + n_t (mod 3) to the next. In the last V phases the phases still
// to run read K slot base + n_t - 2 (group B's M(n_t - 2)) and V slots
// base + n_t - 2 and base + n_t - 1, so the next block's K(0) (K slot
// base + n_t - 1), K(1) and V(0) (slot base + n_t) are free. Q's registers
// are dead after each group's last QK^T.
//
// RAG: S is not a multiple of BKV. The last key tile is partial: every tile
// then loads with its whole offset per lane, so that the range check reads
// zeros past S, and the partial tile's keys at or past S are masked. Loads in
// the V phase only (the M-phase placements put the tile offset in the scalar
// offset, which the range check does not cover).
//
// SPL: split-KV. The grid is n_splits copies of the blocks; copy j covers the
// key tiles [j split_tiles, (j + 1) split_tiles) of each block's range and
// writes its normalised fp32 O and lse to o_part[j] and lse_part[j], which the
// merge kernel combines. Only the copy holding a block's diagonal tile masks
// it; a copy whose range misses the block's keys writes O = 0, lse = -inf.
template <int H, int BKV, bool CAUSAL, bool WIN, bool SEG, int MLD, bool PF, bool RAG = false, bool SPL = false>
__device__ __forceinline__ void pp_block(const FwdArgs &a, const int bid, const int next_bid, int &base,
                                         bf16x8 (&qf)[H / 16], const bool prefetched) {
    static_assert(!SPL || (!PF && !SEG && !WIN && MLD == 0), "split-KV: dense shapes, loads in the V phase");
    static_assert(!PF || (MLD == 0 && !SEG), "prefetch: loads in the V phase, no segment ids");
    static_assert(!RAG || (MLD == 0 && !SEG), "partial key tiles: loads in the V phase, no segment ids");
    constexpr int NG = 4;  // waves per group (8 per workgroup)
    constexpr int CPR = H / 8;
    constexpr int KSTEPS = H / 16;
    constexpr int MB = BKV / 32;
    constexpr int HB = H / 32;
    constexpr int PK = BKV / 16;
    constexpr int NQK = MB * KSTEPS, NPV = PK * HB;
    static_assert(NQK == NPV, "M phase pairs one QK^T MFMA with one PV MFMA");
    using L = TileLayout<H, BKV>;
    constexpr int NSLOT = 3;
    __shared__ __attribute__((aligned(1024))) __bf16 sk[NSLOT][L::K_ELEMS];
    __shared__ __attribute__((aligned(1024))) __bf16 sv[NSLOT][L::V_ELEMS];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave / NG, gwv = wave % NG;
    const int n = lane & 31, c = lane >> 5;

    // ---- work unit (causal: heaviest query block first) and this lane's row
    const int units = a.B * a.K * a.n_gsplit;
    const int per_split = units * a.n_qblocks;
    const int split = SPL ? bid / per_split : 0;
    const int bidb = SPL ? bid % per_split : bid;
    int qb = bidb / units;
    if (CAUSAL) qb = a.n_qblocks - 1 - qb;
    const int u = bidb % units;
    const int gs = u % a.n_gsplit;
    const int kh = (u / a.n_gsplit) % a.K;
    const int b = u / (a.n_gsplit * a.K);
    const int t0 = qb * a.bq;
    const int T = a.T, S = a.S;
    const int rho = wave * 32 + n;  // gw * bq == 32 * NW: every row belongs to the unit
    const int g = gs * a.gw + rho / a.bq;
    const int t = t0 + rho % a.bq;
    const bool q_valid = t < T;
    const size_t bk = (size_t)b * a.K + kh;
    const size_t qrow_off = ((bk * a.G + g) * (size_t)T + t) * H;

    // SEG: every segment id the prologue needs (the lane's query, the block's
    // queries, the keys of the tiles this wave stages) is loaded before Q and
    // before any of them is used, so that the loads' latencies overlap
    // instead of adding up.
    constexpr int KV_CAP = SEG ? 8192 : 1;
    constexpr int NT_CAP = SEG ? KV_CAP / BKV : 1;
    constexpr int KV_PW = SEG ? NT_CAP / 8 : 1;  // key tiles a wave stages, at most
    [[maybe_unused]] const int nt_all = CAUSAL ? qb + 1 + a.coff / BKV : S / BKV;
    int pre_q = 0, pre_qb[4] = {}, pre_kv[KV_PW] = {};
    if constexpr (SEG) {
        const int32_t *qs = a.q_seg + (size_t)b * T;
        const int32_t *kvs = a.kv_seg + (size_t)b * S;
        // (loads from clamped in-range indices; the validity tests come at
        // the uses, so that no select waits on a load here)
        pre_q = qs[min(t, T - 1)];
        // the block's queries t0 .. t0 + bq - 1 (bq <= 256: gw * bq == 256)
#pragma unroll
        for (int m = 0; m < 4; m++) pre_qb[m] = qs[min(t0 + lane + 64 * m, T - 1)];
        // key tiles wave, wave + 8, ... (whole tiles: jj * BKV + lane < S)
#pragma unroll
        for (int m = 0; m < KV_PW; m++) {
            const int jj = wave + 8 * m;
            if (jj < nt_all) pre_kv[m] = kvs[jj * BKV + lane];
        }
    }

    // Q^T. SEG: a row past T (a ragged last block) reads row T - 1 instead;
    // its query column is computed but never stored, and no other column
    // depends on it. Unconditional loads keep the compiler's waits exact, so
    // that the id loads above and these are all in flight before the first
    // use.
    if constexpr (SEG) {
        const size_t qload_off = ((bk * a.G + g) * (size_t)T + min(t, T - 1)) * H;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ks++) qf[ks] = *(const bf16x8 *)(a.q + qload_off + 16 * ks + 8 * c);
        sched_fence();
    } else if (!(PF && prefetched)) {
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ks++)
            qf[ks] = q_valid ? *(const bf16x8 *)(a.q + qrow_off + 16 * ks + 8 * c) : bf16x8{};
    }

    const buffer_rsrc krs = make_rsrc(a.k + bk * (size_t)S * H, S * H * 2);
    const buffer_rsrc vrs = make_rsrc(a.v + bk * (size_t)S * H, S * H * 2);

    // ---- segment ids (SEG, S <= KV_CAP): the kv ids of the block's key tiles
    // staged in LDS with each tile's id range, and the list of the tiles whose
    // range meets the block's query-id range (in increasing order; the others
    // hold no visible pair). The loop walks that list; it is the same for
    // every wave, so both groups stay in step.
    __shared__ __attribute__((aligned(16))) int s_kvid[KV_CAP];
    __shared__ int s_tmin[NT_CAP], s_tmax[NT_CAP], s_jlist[NT_CAP];
    __shared__ int s_nvis;
    int my_qid = 0, w_qmin = 0, w_qmax = 0, n_vis = 0;
    if constexpr (SEG) {
        my_qid = q_valid ? pre_q : 0;
        w_qmin = wave_min_i(q_valid ? my_qid : INT_MAX);
        w_qmax = wave_max_i(q_valid ? my_qid : INT_MIN);
        // id range of the block's queries t0 .. t0 + bq - 1 (bq may exceed
        // the wave's 64 lanes: 128 or 256 queries when a unit holds one or
        // two heads)
        int qlo = INT_MAX, qhi = INT_MIN;
#pragma unroll
        for (int m = 0; m < 4; m++) {
            const int i = lane + 64 * m;
            if (i < a.bq && t0 + i < T) {
                qlo = min(qlo, pre_qb[m]);
                qhi = max(qhi, pre_qb[m]);
            }
        }
        const int wg_qmin = wave_min_i(qlo), wg_qmax = wave_max_i(qhi);
        static_assert(!SEG || BKV == 64, "one key per lane");
#pragma unroll
        for (int m = 0; m < KV_PW; m++) {
            const int jj = wave + 8 * m;
            if (jj < nt_all) {
                const int id = pre_kv[m];
                s_kvid[jj * BKV + lane] = id;
                const int lo = wave_min_i(id), hi = wave_max_i(id);
                if (lane == 0) {
                    s_tmin[jj] = lo;
                    s_tmax[jj] = hi;
                }
            }
        }
        __syncthreads();
        if (wave == 0) {
            int cnt = 0;
            for (int jb = 0; jb < nt_all; jb += 64) {
                const int j = jb + lane;
                const bool vis = j < nt_all && !(s_tmax[j] < wg_qmin || s_tmin[j] > wg_qmax);
                const unsigned long long m = __ballot(vis);
                if (vis) s_jlist[cnt + __popcll(m & ((1ull << lane) - 1))] = j;
                cnt += __popcll(m);
            }
            if (lane == 0) s_nvis = cnt;
        }
        __syncthreads();
        n_vis = __builtin_amdgcn_readfirstlane(s_nvis);
        if (n_vis == 0) {
            // no query of the block shares an id with any key it may see
            if (q_valid) {
#pragma unroll
                for (int k2 = 0; k2 < H / 16; k2++) *(bf16x8 *)(a.o + qrow_off + 8 * (2 * k2 + c)) = bf16x8{};
                if (c == 0 && a.lse) a.lse[(bk * a.G + g) * (size_t)T + t] = -INFINITY;
            }
            return;
        }
    }

    // key tiles j0 .. j0 + n_t - 1 (SEG: the n_vis tiles of the list); a left
    // window (causal only, WIN) starts the block's range at the first tile its
    // first query can see
    const int WL = a.wl;
    // causal: the block's diagonal tile qb + coff / BKV comes last (j_end is
    // one past it); SPL: the copy's part of the range
    const int j_end = CAUSAL ? qb + 1 + a.coff / BKV : (RAG ? (S + BKV - 1) / BKV : S / BKV);
    const int j0_blk = WIN && t0 - WL > 0 ? (t0 - WL) / BKV : 0;
    const int j0 = SPL ? max(j0_blk, split * a.split_tiles) : j0_blk;
    const int n_t = SEG ? n_vis : (SPL ? min(j_end, (split + 1) * a.split_tiles) : j_end) - j0;
    // SPL: does the copy hold the block's last tile (the diagonal, or the
    // partial one)?
    const bool holds_last = !SPL || j0 + n_t == j_end;
    if constexpr (SPL) {
        if (n_t <= 0) {
            // none of the block's keys: O = 0, lse = -inf
            if (q_valid) {
                const size_t row = (bk * a.G + g) * (size_t)T + t;
                const size_t rows = (size_t)a.B * a.K * a.G * T;
                float *orow = a.o_part + ((size_t)split * rows + row) * H;
#pragma unroll
                for (int hb = 0; hb < H / 32; hb++)
#pragma unroll
                    for (int q4 = 0; q4 < 4; q4++) *(f32x4 *)(orow + 32 * hb + 8 * q4 + 4 * c) = f32x4{};
                if (c == 0) a.lse_part[(size_t)split * rows + row] = -INFINITY;
            }
            return;
        }
    }
    // key tile of loop step i
    auto tile_of = [&](int i) { return SEG ? __builtin_amdgcn_readfirstlane(s_jlist[i]) : j0 + i; };

    // ---- global -> LDS loads: group A loads K tiles, group B V tiles; wave gwv
    // of a group issues 1 KiB blocks gwv, gwv + NG, ... (padding slots repeat
    // the row's last chunk, as in TileLayout)
    constexpr int KL = (L::K_BLOCKS + NG - 1) / NG, VL = (L::V_BLOCKS + NG - 1) / NG;
    constexpr int NL = KL > VL ? KL : VL;
    const int rs = grp == 0 ? L::KRS : L::VRS;
    int ld_off[NL];
#pragma unroll
    for (int i = 0; i < NL; i++) {
        const int pslot = (gwv + i * NG) * 64 + lane;
        // slots past the tile's last padded row (the last K block at H = 256)
        // re-read row BKV - 1 into the slot's tail
        ld_off[i] = (min(pslot / rs, BKV - 1) * H + min(pslot % rs, CPR - 1) * 8) * 2;
    }
    // Without RAG, tiles j < n_t lie wholly inside K and V (S % BKV == 0,
    // rows < BKV), so the tile offset may go in the scalar offset, which the
    // range check does not cover. With RAG it goes into each lane's offset.
    auto issue_tile_from = [&](const buffer_rsrc &kr, const buffer_rsrc &vr, int jt, int slot) {
        const int tile = __builtin_amdgcn_readfirstlane(jt * BKV * H * 2);
        auto load = [&](const buffer_rsrc &r, char *dst, int off) {
            if constexpr (RAG)
                lds_load16_to(r, dst, off + tile);
            else
                lds_load16_to(r, dst, off, tile);
        };
        if (grp == 0) {
#pragma unroll
            for (int i = 0; i < KL; i++)
                if (gwv + i * NG < L::K_BLOCKS) load(kr, (char *)sk[slot] + (gwv + i * NG) * 1024, ld_off[i]);
        } else {
#pragma unroll
            for (int i = 0; i < VL; i++)
                if (gwv + i * NG < L::V_BLOCKS) load(vr, (char *)sv[slot] + (gwv + i * NG) * 1024, ld_off[i]);
        }
    };
    auto issue_tile = [&](int j, int slot) { issue_tile_from(krs, vrs, tile_of(j), slot); };
    // the tile load an M phase issues (slot < 0: none)
    struct MLd {
        int bytes, slot;
    };
    // MLD 1: the loads of issue_tile from assembly, with the tile's byte
    // offset (wave-uniform) in the scalar offset
    const i32x4 my_rs = grp == 0 ? make_rsrc_words(a.k + bk * (size_t)S * H, S * H * 2)
                                 : make_rsrc_words(a.v + bk * (size_t)S * H, S * H * 2);
    const int my_blocks = grp == 0 ? L::K_BLOCKS : L::V_BLOCKS;
    // LDS addresses as wave-uniform integers, so that the M phase computes
    // the destinations on the scalar unit
    const unsigned my_base0 = __builtin_amdgcn_readfirstlane(grp == 0 ? lds_addr(sk[0]) : lds_addr(sv[0]));
    const unsigned my_slot_bytes = grp == 0 ? L::K_ELEMS * 2 : L::V_ELEMS * 2;
    auto issue_tile_asm = [&](MLd ld) {
        const unsigned base = my_base0 + (unsigned)ld.slot * my_slot_bytes;
        const int tb = __builtin_amdgcn_readfirstlane(ld.bytes);
#pragma unroll
        for (int i = 0; i < NL; i++)
            if (gwv + i * NG < my_blocks)
                lds_dma16_so(my_rs, __builtin_amdgcn_readfirstlane(base + (unsigned)(gwv + i * NG) * 1024u), ld_off[i], tb);
    };
    // MLD 2: every wave issues NL loads per M phase without branches; a block
    // past the tile gets an out-of-range offset (no memory is read) and the
    // dummy destination
    __shared__ __attribute__((aligned(1024))) char s_ldummy[MLD == 2 ? 1024 : 16];
    const unsigned dummy_dst = __builtin_amdgcn_readfirstlane(lds_addr(s_ldummy));
    if constexpr (MLD == 2) {
#pragma unroll
        for (int i = 0; i < NL; i++)
            if (gwv + i * NG >= my_blocks) ld_off[i] = (int)0x80000000u;
    }
    auto issue_one = [&](int i, MLd ld) {
        const unsigned base = my_base0 + (unsigned)ld.slot * my_slot_bytes;
        const unsigned dst = gwv + i * NG < my_blocks ? base + (unsigned)(gwv + i * NG) * 1024u : dummy_dst;
        lds_dma16_so(my_rs, __builtin_amdgcn_readfirstlane(dst), ld_off[i], __builtin_amdgcn_readfirstlane(ld.bytes));
    };

    f32x16 sacc[MB];
    bf16x8 pf[PK];
    f32x16 oacc[HB];
#pragma unroll
    for (int hb = 0; hb < HB; hb++) oacc[hb] = f32x16{};
    float m_run = -INFINITY;  // reference max, log2 units (identical in a lane pair)
    float l_run = 0.f;        // denominator over this lane's half of the keys

    // ---- M phase: QK^T MFMA x and PV MFMA x alternate (independent chains)
    const int k_lane = n * L::KRS * 8 + c * 8;
    const int v_lane = (4 * c + ((lane & 15) >> 2)) * L::VRS * 8 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    auto m_phase = [&](auto do_qk, auto do_pv, int kslot, int vslot, MLd ld, auto loads) {
        const __bf16 *kt = sk[kslot];
        const __bf16 *vt = sv[vslot];
        __builtin_amdgcn_s_setprio(1);
        if constexpr (MLD == 1) {
            if (ld.slot >= 0) issue_tile_asm(ld);
            sched_fence();
        }
        constexpr int LSTEP = NQK / NL > 0 ? NQK / NL : 1;
#pragma unroll
        for (int x = 0; x < NQK; x++) {
            if constexpr (decltype(do_qk)::value) {
                const int mb = x % MB, ks = x / MB;
                const bf16x8 kf = *(const bf16x8 *)(kt + k_lane + mb * 32 * L::KRS * 8 + ks * 16);
                sacc[mb] = mfma32x32x16(kf, qf[ks], ks == 0 ? f32x16{} : sacc[mb]);
            }
            if constexpr (decltype(do_pv)::value) {
                const int kk = x / HB, hb = x % HB;
                const __bf16 *vp = vt + v_lane + kk * 16 * L::VRS * 8 + hb * 32;
                const s16x4 lo = lds_read_tr16(vp);
                const s16x4 hi = lds_read_tr16(vp + 8 * L::VRS * 8);
                oacc[hb] = mfma32x32x16(join_bf16x8(lo, hi), pf[kk], oacc[hb]);
            }
            if constexpr (MLD == 2 && decltype(loads)::value)
                if (x % LSTEP == LSTEP / 2 && x / LSTEP < NL) issue_one(x / LSTEP, ld);
        }
        constexpr bool QK = decltype(do_qk)::value, PV = decltype(do_pv)::value;
        constexpr int D = kFwdPrefetch < NQK ? kFwdPrefetch : NQK;
        m_phase_schedule<NQK, (QK ? 1 : 0) + (PV ? 1 : 0), (QK ? 1 : 0) + (PV ? 2 : 0), D>(
            std::make_integer_sequence<int, D>(), std::make_integer_sequence<int, NQK>());
        __builtin_amdgcn_s_setprio(0);
        if constexpr (MLD == 0) wait_lds_loads();
    };

    // ---- V phase pieces (as in the kernel above)
    auto mask_tile = [&](int s0) {
        const int lim = min(CAUSAL ? t + a.coff : INT_MAX, S - 1) - s0 - 4 * c;  // last visible key offset
        const int first = WIN ? t - WL - s0 - 4 * c : INT_MIN;          // first visible key offset
#pragma unroll
        for (int mb = 0; mb < MB; mb++)
#pragma unroll
            for (int q4 = 0; q4 < 4; q4++) {
                // SEG: the ids of keys s0 + 32 mb + 8 q4 + 4 c + 0..3
                i32x4 ids{};
                if constexpr (SEG) ids = *(const i32x4 *)&s_kvid[s0 + 32 * mb + 8 * q4 + 4 * c];
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int r = 4 * q4 + e, off = 32 * mb + 8 * q4 + e;
                    bool hide = off > lim || off < first;
                    if constexpr (SEG) hide = hide || ids[e] != my_qid;
                    if (hide) sacc[mb][r] = -INFINITY;
                }
            }
    };
    // SEG: does tile j need the element mask for this wave's rows (not every
    // id of the tile and of the wave's queries the same)?
    auto seg_mask = [&](int j) {
        const int kmin = __builtin_amdgcn_readfirstlane(s_tmin[j]), kmax = __builtin_amdgcn_readfirstlane(s_tmax[j]);
        return !(w_qmin == w_qmax && kmin == kmax && kmin == w_qmin);
    };
    auto tile_max = [&]() {
        float m4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
        for (int mb = 0; mb < MB; mb++)
#pragma unroll
            for (int r = 0; r < 16; r += 2)
                m4[(r >> 1) & 3] = max_nan(m4[(r >> 1) & 3], max_nan(sacc[mb][r], sacc[mb][r + 1]));
        return max_nan(max_nan(m4[0], m4[1]), max_nan(m4[2], m4[3]));
    };
    auto rescale = [&](float mx) {
        mx = max_nan(mx, __shfl_xor(mx, 32));
        const float m_new = max_nan(m_run, mx * kLog2e);
        const float corr = (m_new == -INFINITY) ? 1.f : exp2_fast(m_run - m_new);
        l_run *= corr;
#pragma unroll
        for (int hb = 0; hb < HB; hb++) oacc[hb] *= corr;
        m_run = m_new;
    };
    // all scaled logits before all exponentials: a lone VALU wave would
    // otherwise wait on each fma before its exp
    auto weights = [&](float m_use) {
        float w[PK * 8];
#pragma unroll
        for (int kk = 0; kk < PK; kk++)
#pragma unroll
            for (int e = 0; e < 8; e++) w[kk * 8 + e] = __builtin_fmaf(sacc[kk >> 1][8 * (kk & 1) + e], kLog2e, -m_use);
        sched_fence();
#pragma unroll
        for (int j = 0; j < PK * 8; j++) w[j] = exp2_fast(w[j]);
        sched_fence();
#pragma unroll
        for (int kk = 0; kk < PK; kk++)
#pragma unroll
            for (int e = 0; e < 8; e++) pf[kk][e] = (__bf16)w[kk * 8 + e];
        // pairwise tree: short dependency chains for a lone VALU wave
#pragma unroll
        for (int n2 = PK * 8 / 2; n2 >= 1; n2 /= 2)
#pragma unroll
            for (int j = 0; j < n2; j++) w[j] = w[2 * j] + w[2 * j + 1];
        return w[0];
    };
    // Weights of a tile with no masked key: the rescale test needs no row max
    // (weights are >= 0, so a lane whose weights sum to at most 2^kRescaleLog2
    // has none above it); the first tile (reference -inf) always rescales.
    auto v_phase_open = [&]() {
        float ls = weights(m_run);
        if (__any(!(ls <= kRescaleBound))) {
            rescale(tile_max());
            ls = weights(m_run);
        }
        l_run += ls;
    };
    // The diagonal tile: element mask, row max, weights.
    auto v_phase_masked = [&](int s0) {
        mask_tile(s0);
        const float mx = tile_max();
        if (__any(mx * kLog2e > m_run + kRescaleLog2)) rescale(mx);
        l_run += weights(m_run == -INFINITY ? 0.f : m_run);
    };

    using yes = std::integral_constant<bool, true>;
    using no = std::integral_constant<bool, false>;

    // MLD > 0: the load M(i) issues
    auto mload = [&](int i, int nslot) {
        const int nnslot = nslot == NSLOT - 1 ? 0 : nslot + 1;
        return MLD > 0 && i + 2 < n_t ? MLd{tile_of(i + 2) * BKV * H * 2, grp == 0 ? nslot : nnslot} : MLd{0, -1};
    };

    // ---- prologue: K(0) -> slot base - 1, K(1) and V(0) -> slot base (MLD >
    // 0: K(1) and V(1) come from M(-1)); base is 0 without PF. A prefetched
    // block's loads have landed: each wave waited for its own at the end of
    // the previous block's last M phase.
    const int slot_m1 = base == 0 ? NSLOT - 1 : base - 1;
    if (!(PF && prefetched)) {
        issue_tile(0, grp == 0 ? slot_m1 : base);
        if (MLD == 0 && grp == 0 && n_t > 1) issue_tile(1, base);
        wait_lds_loads();
    }
    barrier_no_drain();

    if (grp == 1) barrier_no_drain();  // group B runs one phase behind
    {                                  // M(-1): S^T of tile 0
        const MLd ld = mload(-1, base);
        if (MLD == 2 && ld.slot >= 0)
            m_phase(yes{}, no{}, slot_m1, base, ld, yes{});
        else
            m_phase(yes{}, no{}, slot_m1, base, ld, no{});
    }
    int slot = base;                   // slot of tile set i: K(i+1), V(i)
    // MLD > 0: round i = V(i), the wait for the loads of M(i-1), M(i) with
    // its loads (rounds 0 .. n_t - 3; MLD 2 keeps the branch out of M by
    // peeling the last round). VK: how V(i) masks (0: no element mask, 1: the
    // element mask, 2: segment ids decide per tile).
    using v_open = std::integral_constant<int, 0>;
    using v_masked = std::integral_constant<int, 1>;
    using v_seg = std::integral_constant<int, 2>;
    auto round_ld = [&](int i, auto vk, auto ld_tag) {
        const int nslot = slot == NSLOT - 1 ? 0 : slot + 1;
        barrier_no_drain();
        if constexpr (decltype(vk)::value == 2) {
            const int j = tile_of(i);
            if (seg_mask(j))
                v_phase_masked(j * BKV);
            else
                v_phase_open();
        } else if constexpr (decltype(vk)::value == 1) {
            v_phase_masked((j0 + i) * BKV);
        } else {
            v_phase_open();
        }
        const MLd ld = mload(i, nslot);
        wait_lds_loads();
        barrier_no_drain();
        m_phase(yes{}, yes{}, slot, slot, ld, ld_tag);
        slot = nslot;
    };
    auto rounds_from = [&](int i, auto vk) {
        for (; i < n_t - 2; i++) round_ld(i, vk, yes{});
        for (; i < n_t - 1; i++) round_ld(i, vk, no{});
    };
    if constexpr (MLD == 0) {
        // one round: V(i) then M(i); MASKED: tile i needs the element mask
        auto round = [&](int i, auto masked) {
            const int nslot = slot == NSLOT - 1 ? 0 : slot + 1;
            barrier_no_drain();
            // V(i)
            if (grp == 0 ? i + 2 < n_t : true) issue_tile(grp == 0 ? i + 2 : i + 1, nslot);
            if constexpr (decltype(masked)::value)
                v_phase_masked((j0 + i) * BKV);
            else
                v_phase_open();
            barrier_no_drain();
            // M(i)
            m_phase(yes{}, yes{}, slot, slot, MLd{0, -1}, no{});
            slot = nslot;
        };
        if constexpr (WIN) {
            // The window's left edge, t - WL over the block's BKV queries, spans at
            // most two tiles: those before the first tile every query sees whole
            // take the element mask.
            int i = 0;
            for (; i < 2 && i < n_t - 1 && (j0 + i) * BKV < t0 + BKV - 1 - WL; i++) round(i, yes{});
            for (; i < n_t - 1; i++) round(i, no{});
        } else if constexpr (SEG) {
            for (int i = 0; i < n_t - 1; i++) {
                const int nslot = slot == NSLOT - 1 ? 0 : slot + 1;
                barrier_no_drain();
                if (grp == 0 ? i + 2 < n_t : true) issue_tile(grp == 0 ? i + 2 : i + 1, nslot);
                const int j = tile_of(i);
                if (seg_mask(j))
                    v_phase_masked(j * BKV);
                else
                    v_phase_open();
                barrier_no_drain();
                m_phase(yes{}, yes{}, slot, slot, MLd{0, -1}, no{});
                slot = nslot;
            }
        } else {
            for (int i = 0; i < n_t - 1; i++) {
                const int nslot = slot == NSLOT - 1 ? 0 : slot + 1;
                barrier_no_drain();
                if (grp == 0 ? i + 2 < n_t : true) issue_tile(grp == 0 ? i + 2 : i + 1, nslot);
                v_phase_open();
                barrier_no_drain();
                m_phase(yes{}, yes{}, slot, slot, MLd{0, -1}, no{});
                slot = nslot;
            }
        }
    } else if constexpr (WIN) {
        int i = 0;
        for (; i < 2 && i < n_t - 1 && (j0 + i) * BKV < t0 + BKV - 1 - WL; i++) {
            if (i < n_t - 2)
                round_ld(i, v_masked{}, yes{});
            else
                round_ld(i, v_masked{}, no{});
        }
        rounds_from(i, v_open{});
    } else if constexpr (SEG) {
        rounds_from(0, v_seg{});
    } else {
        rounds_from(0, v_open{});
    }
    // the last tile (the diagonal one when causal): nothing left to load or to
    // multiply with K. SEG masks it always (its ids and, when causal, the
    // diagonal). PF: the next block's loads go out first.
    const int base_next = (base + n_t) % NSLOT;
    barrier_no_drain();
    if constexpr (PF) {
        if (next_bid >= 0) {
            const int qb_n = CAUSAL ? a.n_qblocks - 1 - next_bid / units : next_bid / units;
            const int u_n = next_bid % units;
            const int kh_n = (u_n / a.n_gsplit) % a.K;
            const int b_n = u_n / (a.n_gsplit * a.K);
            const int t0_n = qb_n * a.bq;
            const size_t bk_n = (size_t)b_n * a.K + kh_n;
            // Q^T of the lane's next row, through a descriptor over its head's
            // rows (wave-uniform: a wave's 32 rows belong to one head); a row
            // past T reads zeros without a select
            const int g_n = (u_n % a.n_gsplit) * a.gw + rho / a.bq;
            const int t_n = t0_n + rho % a.bq;
            const buffer_rsrc qrs = make_rsrc(a.q + (bk_n * a.G + g_n) * (size_t)T * H, T * H * 2);
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ks++)
                qf[ks] = __builtin_bit_cast(
                    bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qrs, (t_n * H + 16 * ks + 8 * c) * 2, 0, 0));
            const int j0_n = WIN && t0_n - WL > 0 ? (t0_n - WL) / BKV : 0;
            const int n_t_n = (CAUSAL ? qb_n + 1 + a.coff / BKV : (RAG ? (S + BKV - 1) / BKV : S / BKV)) - j0_n;
            const buffer_rsrc krs_n = make_rsrc(a.k + bk_n * (size_t)S * H, S * H * 2);
            const buffer_rsrc vrs_n = make_rsrc(a.v + bk_n * (size_t)S * H, S * H * 2);
            if (grp == 0) {
                issue_tile_from(krs_n, vrs_n, j0_n, base_next == 0 ? NSLOT - 1 : base_next - 1);
                if (n_t_n > 1) issue_tile_from(krs_n, vrs_n, j0_n + 1, base_next);
            } else {
                issue_tile_from(krs_n, vrs_n, j0_n, base_next);
            }
        }
    }
    if constexpr (CAUSAL || SEG) {
        if (holds_last)
            v_phase_masked(tile_of(n_t - 1) * BKV);
        else
            v_phase_open();  // SPL: a tile before the diagonal one
    } else {
        // a partial last tile: its keys at or past S out, then the usual
        // weights (a lane whose keys are all out sums zero)
        if constexpr (RAG)
            if (holds_last) mask_tile(tile_of(n_t - 1) * BKV);
        v_phase_open();
    }
    if (MLD > 0) wait_lds_loads();
    barrier_no_drain();
    m_phase(no{}, yes{}, slot, slot, MLd{0, -1}, no{});
    if (grp == 0) barrier_no_drain();  // group A's trailing phase

    // ---- finalize: O = acc / l in bf16 through LDS, so that the wave's 32 rows
    // (consecutive queries of one head: 8 KiB contiguous in o) leave in eight
    // fully coalesced 1 KiB stores; lse = ln(sum exp(logits)).
    l_run += __shfl_xor(l_run, 32);
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    // Staging region of this wave: 32 rows of H * 2 + 16 bytes (padded:
    // conflict-free 8-byte writes), two waves per K slot and the last two in a
    // V slot. Every K slot and V slot n_t % 3 are dead here: the only phase
    // still running is group B's last PV, which reads V slot (n_t - 1) % 3,
    // and all loads have landed (each M phase ends with a wait). At H = 256
    // the rows do not fit and O leaves straight from registers. PF: the next
    // block's tiles hold K slots base + n_t - 1 and base + n_t and V slot
    // base + n_t, so group A stages in K and V slot base + n_t + 1 (dead since
    // group B's M(n_t - 2)) and group B in a region of its own.
    constexpr int OROW = H * 2 + 16;
    constexpr bool kStage = 2 * 32 * OROW <= L::K_ELEMS * 2 && 2 * 32 * OROW <= L::V_ELEMS * 2;
    __shared__ __attribute__((aligned(16))) char s_ostage[PF && kStage ? 4 * 32 * OROW : 16];
    if constexpr (SPL) {
        // the copy's normalised O in fp32 and its lse, straight from registers
        if (q_valid) {
            const size_t row = (bk * a.G + g) * (size_t)T + t;
            const size_t rows = (size_t)a.B * a.K * a.G * T;
            float *orow = a.o_part + ((size_t)split * rows + row) * H;
#pragma unroll
            for (int hb = 0; hb < HB; hb++)
#pragma unroll
                for (int q4 = 0; q4 < 4; q4++)
                    *(f32x4 *)(orow + 32 * hb + 8 * q4 + 4 * c) =
                        f32x4{oacc[hb][4 * q4] * inv, oacc[hb][4 * q4 + 1] * inv, oacc[hb][4 * q4 + 2] * inv,
                              oacc[hb][4 * q4 + 3] * inv};
            if (c == 0)
                a.lse_part[(size_t)split * rows + row] = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
        }
    } else if constexpr (kStage) {
        char *stage;
        if constexpr (PF) {
            const int fs = base_next == NSLOT - 1 ? 0 : base_next + 1;
            stage = grp == 1 ? s_ostage + (wave - 4) * 32 * OROW
                             : (wave < 2 ? (char *)sk[fs] : (char *)sv[fs]) + (wave & 1) * 32 * OROW;
        } else {
            stage = (wave < 6 ? (char *)sk[wave >> 1] : (char *)sv[n_t % NSLOT]) + (wave & 1) * 32 * OROW;
        }
#pragma unroll
        for (int hb = 0; hb < HB; hb++)
#pragma unroll
            for (int q4 = 0; q4 < 4; q4++) {
                bf16x4 val;
#pragma unroll
                for (int e = 0; e < 4; e++) val[e] = (__bf16)(oacc[hb][4 * q4 + e] * inv);
                *(bf16x4 *)(stage + n * OROW + (32 * hb + 8 * q4 + 4 * c) * 2) = val;
            }
        // rows of this wave: queries t_w .. t_w + 31 of head g (all lanes agree)
        const int t_w = t - n;
        __bf16 *orows = a.o + ((bk * a.G + g) * (size_t)T + t_w) * H;
        constexpr int CPR16 = H / 8;  // 16-byte chunks per row
#pragma unroll
        for (int j = 0; j < 32 * CPR16 / 64; j++) {
            const int idx = j * 64 + lane;
            const int r = idx / CPR16, ch = idx % CPR16;
            const bf16x8 val = *(const bf16x8 *)(stage + r * OROW + ch * 16);
            if (t_w + r < T) *(bf16x8 *)(orows + (size_t)r * H + ch * 8) = val;
        }
        if (q_valid && c == 0 && a.lse)
            a.lse[(bk * a.G + g) * (size_t)T + t] = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
    } else {
        if (q_valid) {
            __bf16 *orow = a.o + qrow_off;
#pragma unroll
            for (int hb = 0; hb < HB; hb++)
#pragma unroll
                for (int q4 = 0; q4 < 4; q4++) {
                    bf16x4 val;
#pragma unroll
                    for (int e = 0; e < 4; e++) val[e] = (__bf16)(oacc[hb][4 * q4 + e] * inv);
                    *(bf16x4 *)(orow + 32 * hb + 8 * q4 + 4 * c) = val;
                }
            if (c == 0 && a.lse)
                a.lse[(bk * a.G + g) * (size_t)T + t] = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
        }
    }
    if constexpr (PF) base = base_next;
}

// The kernel: one query block per workgroup, or (PERSIST: H <= 128 without
// segment ids, more blocks than compute units) a persistent grid of one
// workgroup per compute unit walking the blocks in snake order (w, 2G - 1 -
// w, 2G + w, ... for a grid of G): each round of G blocks is covered once,
// and the heaviest causal blocks (first in the numbering) pair with the
// lightest. This saves the dispatch of a new workgroup per block. With
// segment ids the blocks' costs are unknown in advance and the hardware's
// dynamic dispatch balances them better.
template <int H, int BKV, bool CAUSAL, bool WIN, bool SEG, int MLD, bool PERSIST, bool RAG>
__device__ __forceinline__ void pp_run(const FwdArgs &a) {
    bf16x8 qf[H / 16];
    int base = 0;
    if constexpr (PERSIST) {
        const int total = a.B * a.K * a.n_gsplit * a.n_qblocks;
        const int g2 = 2 * (int)gridDim.x;
        auto bid_of = [&](int r) { return (r / 2) * g2 + ((r & 1) ? g2 - 1 - (int)blockIdx.x : (int)blockIdx.x); };
        // loads in the V phase, no segment ids: each block prefetches the next
        constexpr bool PF = MLD == 0 && !SEG;
        for (int r = 0;; r++) {
            const int bid = bid_of(r);
            if (bid >= total) break;
            const int next = bid_of(r + 1) < total ? bid_of(r + 1) : -1;
            pp_block<H, BKV, CAUSAL, WIN, SEG, MLD, PF, RAG>(a, bid, next, base, qf, r > 0);
            // without the prefetch the next block's prologue reuses the LDS
            // slots; with it the prologue's barrier orders the blocks
            if constexpr (!PF) __syncthreads();
        }
    } else {
        pp_block<H, BKV, CAUSAL, WIN, SEG, MLD, false, RAG>(a, blockIdx.x, -1, base, qf, false);
    }
}

template <int H, int BKV, bool CAUSAL, bool WIN, bool SEG = false, int MLD = 0, bool PERSIST = false>
__global__ __launch_bounds__(512, 2) void attn_fwd_pp_kernel(FwdArgs a) {
    pp_run<H, BKV, CAUSAL, WIN, SEG, MLD, PERSIST, false>(a);
}

// Split-KV on the ping-pong kernel (dense shapes without a window; RAG: a
// partial last key tile): one workgroup per (split, block).
template <int H, int BKV, bool CAUSAL, bool RAG>
__global__ __launch_bounds__(512, 2) void attn_fwd_pp_split_kernel(FwdArgs a) {
    bf16x8 qf[H / 16];
    int base = 0;
    pp_block<H, BKV, CAUSAL, false, false, 0, false, RAG, true>(a, blockIdx.x, -1, base, qf, false);
}

// The same with a partial last key tile (S not a multiple of BKV): loads in
// the V phase, no segment ids.
template <int H, int BKV, bool CAUSAL, bool WIN, bool PERSIST>
__global__ __launch_bounds__(512, 2) void attn_fwd_pp_ragged_kernel(FwdArgs a) {
    pp_run<H, BKV, CAUSAL, WIN, false, 0, PERSIST, true>(a);
}

// The ping-pong kernel with the call's load placement (a runtime choice; the
// three variants compute bitwise the same outputs).
// Compute units of the current device, read once per device (1 if the query
// fails, which leaves a persistent grid correct, only serial).
static unsigned device_cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 1;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return (unsigned)n;
}

template <int H, int BKV, bool CAUSAL, bool WIN, bool SEG>
static void launch_pp(const FwdArgs &a, unsigned grid, hipStream_t stream) {
    // a partial last key tile: the ragged kernel (loads in the V phase, the
    // same arithmetic as every placement)
    if constexpr (!SEG) {
        if (a.S % BKV != 0) {
            if constexpr (H <= 128) {
                const unsigned cus = device_cu_count();
                if (grid > cus) {
                    hipLaunchKernelGGL((attn_fwd_pp_ragged_kernel<H, BKV, CAUSAL, WIN, true>), dim3(cus), dim3(512),
                                       0, stream, a);
                    return;
                }
            }
            hipLaunchKernelGGL((attn_fwd_pp_ragged_kernel<H, BKV, CAUSAL, WIN, false>), dim3(grid), dim3(512), 0,
                               stream, a);
            return;
        }
    }
    // H <= 128 without segment ids and more blocks than compute units: the
    // persistent grid, one workgroup per CU (the kernel's LDS and registers
    // allow one per CU)
    if constexpr (H <= 128 && !SEG) {
        const unsigned cus = device_cu_count();
        if (grid > cus) {
            switch (a.load_placement) {
                case 1: hipLaunchKernelGGL((attn_fwd_pp_kernel<H, BKV, CAUSAL, WIN, SEG, 1, true>), dim3(cus), dim3(512), 0, stream, a); break;
                case 2: hipLaunchKernelGGL((attn_fwd_pp_kernel<H, BKV, CAUSAL, WIN, SEG, 2, true>), dim3(cus), dim3(512), 0, stream, a); break;
                default: hipLaunchKernelGGL((attn_fwd_pp_kernel<H, BKV, CAUSAL, WIN, SEG, 0, true>), dim3(cus), dim3(512), 0, stream, a); break;
            }
            return;
        }
    }
    switch (a.load_placement) {
        case 1: hipLaunchKernelGGL((attn_fwd_pp_kernel<H, BKV, CAUSAL, WIN, SEG, 1>), dim3(grid), dim3(512), 0, stream, a); break;
        case 2: hipLaunchKernelGGL((attn_fwd_pp_kernel<H, BKV, CAUSAL, WIN, SEG, 2>), dim3(grid), dim3(512), 0, stream, a); break;
        default: hipLaunchKernelGGL((attn_fwd_pp_kernel<H, BKV, CAUSAL, WIN, SEG, 0>), dim3(grid), dim3(512), 0, stream, a); break;
    }
}

template <int H, int BKV, int NW, int WPS>
static hipError_t launch_fwd_t(const FwdArgs &a, hipStream_t stream) {
    const unsigned grid = (unsigned)(a.B * a.K * a.n_gsplit * a.n_qblocks * (a.o_part ? a.n_splits : 1));
    const bool all_waves = a.gw * a.bq == 32 * NW;
    const MaskSpec m{a.causal, a.coff, a.wl, a.wr, a.prefix};
    // causal: every block's diagonal lies in its last key tile (one query
    // block per key tile, the diagonal offset a whole number of tiles)
    const bool diag_tiles = !a.causal || (a.coff >= 0 && a.coff % BKV == 0 && a.T + a.coff == a.S && a.bq == BKV);
    // per-head masks: the general kernel (it alone reads the table)
    const bool uniform = a.head_mask == nullptr;
    const bool dense = uniform && a.o_part == nullptr && a.q_seg == nullptr && all_waves && a.S % BKV == 0 &&
                       !mask_extra(m) && diag_tiles;
    if constexpr (H <= 128 && NW == 8) {
        // the ping-pong kernel, also with a partial last key tile
        const bool pp_dense =
            uniform && a.o_part == nullptr && a.q_seg == nullptr && all_waves && !mask_extra(m) && diag_tiles;
        if (pp_dense) {
            if (a.causal)
                launch_pp<H, BKV, true, false, false>(a, grid, stream);
            else
                launch_pp<H, BKV, false, false, false>(a, grid, stream);
            return hipGetLastError();
        }
        // segment ids on an otherwise dense shape with at most 8192 keys: the
        // ping-pong kernel over each block's list of tiles that share an id
        const bool dense_seg = uniform && a.o_part == nullptr && a.q_seg != nullptr && all_waves && a.S % BKV == 0 &&
                               a.S <= 8192 && !mask_extra(m) && diag_tiles;
        if (dense_seg) {
            if (a.causal)
                launch_pp<H, BKV, true, false, true>(a, grid, stream);
            else
                launch_pp<H, BKV, false, false, true>(a, grid, stream);
            return hipGetLastError();
        }
        // a causal left window on an otherwise dense shape: the ping-pong kernel
        // starting at each block's first visible tile
        const bool dense_win = uniform && a.o_part == nullptr && a.q_seg == nullptr && all_waves &&
                               mask_left_window_only(m) && diag_tiles;
        if (dense_win) {
            launch_pp<H, BKV, true, true, false>(a, grid, stream);
            return hipGetLastError();
        }
    }
    if (a.causal && dense)
        hipLaunchKernelGGL((attn_fwd_kernel<H, BKV, NW, WPS, true, true>), dim3(grid), dim3(NW * 64), 0, stream, a);
    else if (a.causal)
        hipLaunchKernelGGL((attn_fwd_kernel<H, BKV, NW, WPS, true, false>), dim3(grid), dim3(NW * 64), 0, stream, a);
    else if (dense)
        hipLaunchKernelGGL((attn_fwd_kernel<H, BKV, NW, WPS, false, true>), dim3(grid), dim3(NW * 64), 0, stream, a);
    else
        hipLaunchKernelGGL((attn_fwd_kernel<H, BKV, NW, WPS, false, false>), dim3(grid), dim3(NW * 64), 0, stream, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Split-KV decoding: few query rows per (b, kv head), R = G * T <= 16 (one new
// token of each of the G query heads, say), against a long context. At T = 1
// the work per byte is about G FLOP, so the call is bound by reading K and V.
// The R rows of a unit all read the same K and V, so they are folded into the
// 16 columns of one 16 x 16 MFMA tile: with 32 x 32 tiles and one wave per
// head, each key would cost 32 times the MFMA work it needs.
//
// One workgroup per (b, kv head, split), 4 waves (one per SIMD). The split's
// keys are cut into 16-key tiles; wave w takes tiles w, w + 4, ... and streams
// them through its own ring of NST LDS stages (a K and a V tile per stage,
// unpadded, 16-byte chunks XOR-swizzled by row), NST - 1 tiles ahead of its
// compute. A wave reads only what it loaded, so it waits for its own loads
// and the loop has no barrier.
//   S^T = K Q^T     v_mfma_f32_16x16x32_bf16: A = K rows, B = Q^T (registers)
//   O^T += V^T P^T  v_mfma_f32_16x16x16_bf16: A = V^T (LDS transpose read),
//                   B = P^T, which is the S^T accumulator's own layout
// Lane l holds keys 4 (l / 16) + i (i < 4) of query column l % 16 of S^T, and
// rows h = 16 hb + 4 (l / 16) + i of that column of O^T. The online softmax is
// the forward's (exp2 domain, lazy rescale). At the end the 4 waves' running
// max, sum and O merge through LDS into the split's normalised O and lse
// (o_part, lse_part), which attn_fwd_merge_kernel combines across splits.
template <int H, int NST>
__global__ __launch_bounds__(256, 1) void attn_fwd_decode_kernel(FwdArgs a) {
    constexpr int NW = 4, TK = 16;   // waves, keys per tile
    constexpr int CPR = H / 8;       // 16-byte chunks per row
    constexpr int TILE = TK * H;     // elements per K or V tile
    constexpr int NLD = TILE / 512;  // 1 KiB loads per K or V tile
    constexpr int KS = H / 32;       // k-steps of S^T = K Q^T
    constexpr int HB = H / 16;       // 16-row blocks of O^T
    constexpr int RPB = H <= 128 ? 128 / H : 1;  // rows per 256 bytes (64 banks), at least 1
    constexpr int KSW = CPR < 16 ? CPR - 1 : 15, VSW = CPR / 2 < 8 ? CPR / 2 - 1 : 7;
    static_assert(NLD >= 1 && TILE % 512 == 0, "whole 1 KiB loads");
    // K: chunk slot p of row r holds chunk p ^ kswz(r), so that a row read
    // (16 lanes: 16 rows, one chunk) meets 16 distinct slots of 16 bytes mod
    // 256. V: 32-byte pair slot p holds pair p ^ vswz(r), so that a transpose
    // read (32 lanes: 8 rows of 32 bytes) meets 8 distinct 32-byte slots.
    auto kswz = [](int r) { return (r / RPB) & KSW; };
    auto vswz = [](int r) { return (r / RPB) & VSW; };
    __shared__ __attribute__((aligned(1024))) __bf16 sk[NW][NST][TILE];
    __shared__ __attribute__((aligned(1024))) __bf16 sv[NW][NST][TILE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, grp4 = lane >> 4;  // query column, key / h quad
    const int R = a.G * a.T;                       // query rows of the unit
    const int split = (int)blockIdx.x % a.n_splits;
    const int unit = (int)blockIdx.x / a.n_splits;  // b * K + kv head
    const int S = a.S;
    const size_t rows_total = (size_t)a.B * a.K * R;

    // the split's keys [k_begin, k_end) and this wave's 16-key tiles
    // (split_tiles counts the split plan's key tiles: fwd_config_split's bkv)
    constexpr int PLAN_BKV = H == 256 ? 32 : 64;
    const int k_begin = split * a.split_tiles * PLAN_BKV;
    const int k_end = min(S, k_begin + a.split_tiles * PLAN_BKV);
    const int n16 = max(0, (k_end - k_begin + TK - 1) / TK);
    const int n_mine = n16 > wave ? (n16 - wave + NW - 1) / NW : 0;

    // Q^T: column col is query row col of the unit (rows g T + t are
    // contiguous in q); columns past R are zero and never stored
    bf16x8 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ks++)
        qf[ks] = col < R ? *(const bf16x8 *)(a.q + ((size_t)unit * R + col) * H + 32 * ks + 8 * grp4) : bf16x8{};

    const buffer_rsrc krs = make_rsrc(a.k + (size_t)unit * S * H, S * H * 2);
    const buffer_rsrc vrs = make_rsrc(a.v + (size_t)unit * S * H, S * H * 2);
    // per-lane byte offsets within a tile of the loads (load j: chunk slots
    // 64 j + lane of the tile), and element offsets of the operand reads
    int ld_k[NLD], ld_v[NLD];
#pragma unroll
    for (int j = 0; j < NLD; j++) {
        const int p = 64 * j + lane, r = p / CPR, slot = p % CPR;
        ld_k[j] = (r * H + 8 * (slot ^ kswz(r))) * 2;
        const int pair = (slot >> 1) ^ vswz(r);
        ld_v[j] = (r * H + 8 * (2 * pair + (slot & 1))) * 2;
    }
    int k_rd[KS], v_rd[HB];
#pragma unroll
    for (int ks = 0; ks < KS; ks++) k_rd[ks] = col * H + 8 * ((4 * ks + grp4) ^ kswz(col));
    {
        // transpose read: lane 16 g + m addresses key 4 g + m / 4, columns
        // 16 hb + 4 (m % 4) .. + 3, and receives V[4 g + i][16 hb + m], i < 4
        const int r = 4 * grp4 + col / 4;
#pragma unroll
        for (int hb = 0; hb < HB; hb++)
            v_rd[hb] = r * H + 16 * (hb ^ vswz(r)) + 8 * ((col & 3) >> 1) + 4 * (col & 1);
    }
    auto issue = [&](int i) {  // this wave's tile i into stage i % NST
        const int key0 = k_begin + (wave + NW * i) * TK;
        const int st = i % NST;
#pragma unroll
        for (int j = 0; j < NLD; j++) lds_load16_to(krs, (char *)sk[wave][st] + j * 1024, key0 * H * 2 + ld_k[j]);
#pragma unroll
        for (int j = 0; j < NLD; j++) lds_load16_to(vrs, (char *)sv[wave][st] + j * 1024, key0 * H * 2 + ld_v[j]);
    };
    // wait until tile i has landed: the loads of the k tiles issued after it
    // may stay in flight
    // (k < NST; the counts of k >= NST, never used, are clamped to compile)
    constexpr auto cnt = [](int k) { return 2 * NLD * k < 64 ? 2 * NLD * k : 63; };
    auto wait_tile = [&](int k) {
        switch (k) {
            case 0: wait_lds_loads(); break;
            case 1: wait_lds_loads_but<cnt(1)>(); break;
            case 2: wait_lds_loads_but<cnt(2)>(); break;
            case 3: wait_lds_loads_but<cnt(3)>(); break;
            default: wait_lds_loads_but<cnt(4)>(); break;
        }
    };
    static_assert(NST <= 5 && 2 * NLD * (NST - 1) < 64, "wait_tile covers the ring within vmcnt");

    f32x4 oacc[HB];
#pragma unroll
    for (int hb = 0; hb < HB; hb++) oacc[hb] = f32x4{};
    float m_run = -INFINITY;  // reference max of column col, log2 units (same in its 4 lanes)
    float l_run = 0.f;        // sum over this lane's keys of the column

    for (int i = 0; i < min(NST - 1, n_mine); i++) issue(i);
    for (int i = 0; i < n_mine; i++) {
        if (i + NST - 1 < n_mine) {
            // stage (i - 1) % NST: tile i - 1's reads are done (its MFMAs
            // consumed them); make sure before the loads overwrite it
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
            issue(i + NST - 1);
        }
        wait_tile(min(NST - 1, n_mine - 1 - i));
        const int st = i % NST;
        const __bf16 *kt = sk[wave][st];
        const __bf16 *vt = sv[wave][st];
        f32x4 s = f32x4{};
#pragma unroll
        for (int ks = 0; ks < KS; ks++)
            s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8 *)(kt + k_rd[ks]), qf[ks], s, 0, 0, 0);
        const int key0 = k_begin + (wave + NW * i) * TK + 4 * grp4;
        if (key0 + 3 >= k_end) {  // keys past the split (or past S) in the tile
#pragma unroll
            for (int e = 0; e < 4; e++)
                if (key0 + e >= k_end) s[e] = -INFINITY;
        }
        float p[4];
        auto weights = [&](float m_use) {
            float sum = 0.f;
#pragma unroll
            for (int e = 0; e < 4; e++) {
                p[e] = exp2_fast(__builtin_fmaf(s[e], kLog2e, -m_use));
                sum += p[e];
            }
            return sum;
        };
        float ls = weights(m_run);
        if (__any(!(ls <= kRescaleBound))) {
            // the tile's max per column (its 16 keys are in lanes col + 16 j)
            float mx = max_nan(max_nan(s[0], s[1]), max_nan(s[2], s[3]));
            mx = max_nan(mx, __shfl_xor(mx, 16));
            mx = max_nan(mx, __shfl_xor(mx, 32));
            const float m_new = max_nan(m_run, mx * kLog2e);
            const float corr = m_new == -INFINITY ? 1.f : exp2_fast(m_run - m_new);
            l_run *= corr;
#pragma unroll
            for (int hb = 0; hb < HB; hb++) oacc[hb] *= corr;
            m_run = m_new;
            ls = weights(m_run == -INFINITY ? 0.f : m_run);
        }
        l_run += ls;
        s16x4 pt;
#pragma unroll
        for (int e = 0; e < 4; e++) pt[e] = __builtin_bit_cast(short, (__bf16)p[e]);
#pragma unroll
        for (int hb = 0; hb < HB; hb++)
            oacc[hb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(lds_read_tr16(vt + v_rd[hb]), pt, oacc[hb], 0, 0, 0);
    }

    // ---- merge the 4 waves: column sums, then (m, l, O) of every wave in LDS
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
    __syncthreads();  // every wave is done with its ring (and its loads have landed)
    float *mo = (float *)&sk[0][0][0];  // [NW][16][H] partial O^T columns
    float *ml = (float *)&sv[0][0][0];  // [NW][16] max, then [NW][16] sum
    static_assert(NW * 16 * H * 4 <= (int)sizeof(sk) && 2 * NW * 16 * 4 <= (int)sizeof(sv), "merge buffers fit");
#pragma unroll
    for (int hb = 0; hb < HB; hb++)
        *(f32x4 *)(mo + (wave * 16 + col) * H + 16 * hb + 4 * grp4) = oacc[hb];
    if (grp4 == 0) {
        ml[wave * 16 + col] = m_run;
        ml[NW * 16 + wave * 16 + col] = l_run;
    }
    __syncthreads();
    // thread t: column t / 16, h = (t % 16) * H / 16 .. + H / 16
    constexpr int HPT = H / 16;
    const int q = tid >> 4, h0 = (tid & 15) * HPT;
    if (q < R) {
        float m = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; w++) m = max_nan(m, ml[w * 16 + q]);
        float wt[NW], L = 0.f;
#pragma unroll
        for (int w = 0; w < NW; w++) {
            wt[w] = m == -INFINITY ? 0.f : exp2_fast(ml[w * 16 + q] - m);
            L += wt[w] * ml[NW * 16 + w * 16 + q];
        }
        const float inv = L > 0.f ? 1.f / L : 0.f;
        const size_t row = (size_t)unit * R + q;
        float *orow = a.o_part + ((size_t)split * rows_total + row) * H + h0;
#pragma unroll
        for (int e = 0; e < HPT; e += 4) {
            f32x4 v = f32x4{};
#pragma unroll
            for (int w = 0; w < NW; w++) v += wt[w] * *(const f32x4 *)(mo + (w * 16 + q) * H + h0 + e);
            *(f32x4 *)(orow + e) = v * inv;
        }
        if (h0 == 0) a.lse_part[(size_t)split * rows_total + row] = L > 0.f ? (m + log2f(L)) * kLn2 : -INFINITY;
    }
}

// Whether a split-KV call runs attn_fwd_decode_kernel: at most 16 query rows
// per (b, kv head), no segment ids and no mask.
static bool fwd_decode_applies(int G, int T, int H, const MaskSpec &m, bool segments) {
    return (H == 64 || H == 128 || H == 256) && G * T <= 16 && !segments && !m.causal && !mask_extra(m);
}

// Split-KV copies of the general kernel run 4 waves per workgroup at every
// head size, so that at H <= 128 two workgroups share a CU (a decoding
// workgroup has few query rows, and two of them keep twice the K/V bytes in
// flight). H = 256 keeps one wave per SIMD (its O^T carry needs the registers).
template <int H, int BKV, int WPS>
static hipError_t launch_fwd_split_t(const FwdArgs &a, hipStream_t stream) {
    const unsigned grid = (unsigned)(a.B * a.K * a.n_gsplit * a.n_qblocks * a.n_splits);
    if (a.causal)
        hipLaunchKernelGGL((attn_fwd_kernel<H, BKV, 4, WPS, true, false>), dim3(grid), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((attn_fwd_kernel<H, BKV, 4, WPS, false, false>), dim3(grid), dim3(256), 0, stream, a);
    return hipGetLastError();
}

FwdConfig fwd_config_split(int G, int T, int H) {
    FwdConfig cfg;
    cfg.nw = 4;
    cfg.bkv = (H == 256) ? 32 : 64;
    int gw = 1;
    for (int d = 1; d <= cfg.nw && d <= G; d++)
        if (G % d == 0) gw = d;
    cfg.gw = gw;
    cfg.bq = 32 * (cfg.nw / gw);
    (void)T;
    return cfg;
}

FwdConfig fwd_config(int G, int T, int H) {
    // 32 query rows per wave. H <= 128: 8 waves (2 per SIMD, <= 256 registers
    // each). H = 256: the O^T carry alone is 128 registers per lane, so 4 waves
    // (1 per SIMD, up to 512 registers). gw query heads (the largest divisor of
    // G that is <= the wave count) share each K/V tile.
    FwdConfig cfg;
    cfg.nw = (H == 256) ? 4 : 8;
    cfg.bkv = (H == 256) ? 32 : 64;
    int gw = 1;
    for (int d = 1; d <= cfg.nw && d <= G; d++)
        if (G % d == 0) gw = d;
    cfg.gw = gw;
    cfg.bq = 32 * (cfg.nw / gw);
    (void)T;
    return cfg;
}

// ---------------------------------------------------------------------------
// Split-KV merge. The splits of a row hold normalised partial outputs O_j and
// log-sum-exps lse_j over disjoint key ranges; the whole row's result is
//   lse = ln sum_j exp(lse_j),   O = sum_j exp(lse_j - lse) O_j,
// which is the online-softmax combination applied across the splits. A split
// that sees no key has lse_j = -inf and weight 0; a row that sees none gets
// O = 0 and lse = -inf. One pass over the splits with a running maximum, so
// that no load waits on another (the kernel is bound by the latency of its
// loads, not their bytes); each wave takes kMergeRows rows, each lane H / 64
// elements of a row.
constexpr int kMergeRows = 2;
template <int H>
__global__ __launch_bounds__(256) void attn_fwd_merge_kernel(FwdArgs a, int rows) {
    constexpr int EPL = H / 64;  // elements per lane
    constexpr int RPW = kMergeRows;
    const int lane = threadIdx.x & 63;
    const int row0 = ((int)blockIdx.x * 4 + (int)(threadIdx.x >> 6)) * RPW;
    if (row0 >= rows) return;
    float m[RPW], wsum[RPW], acc[RPW][EPL];
#pragma unroll
    for (int r = 0; r < RPW; r++) {
        m[r] = -INFINITY;
        wsum[r] = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; e++) acc[r][e] = 0.f;
    }
    // splits in groups of four, all loads of a group issued before any use
    // (a split past n_splits reads the last one again and counts as -inf)
    constexpr int NJ = 4;
    for (int j0 = 0; j0 < a.n_splits; j0 += NJ) {
        float lj[NJ][RPW], oj[NJ][RPW][EPL];
#pragma unroll
        for (int q = 0; q < NJ; q++)
#pragma unroll
            for (int r = 0; r < RPW; r++) {
                const size_t pr = (size_t)min(j0 + q, a.n_splits - 1) * rows + min(row0 + r, rows - 1);
                lj[q][r] = a.lse_part[pr];
                const float *op = a.o_part + pr * H + lane * EPL;
#pragma unroll
                for (int e = 0; e < EPL; e++) oj[q][r][e] = op[e];
            }
#pragma unroll
        for (int q = 0; q < NJ; q++)
#pragma unroll
            for (int r = 0; r < RPW; r++) {
                const float l = j0 + q < a.n_splits ? lj[q][r] : -INFINITY;
                // running maximum; what was summed is rescaled to it (by 0
                // while the maximum was -inf), without a branch
                const float m_new = max_nan(m[r], l);
                const float corr = m_new == -INFINITY ? 1.f : exp2_fast((m[r] - m_new) * kLog2e);
                const float w = l == -INFINITY ? 0.f : exp2_fast((l - m_new) * kLog2e);
                wsum[r] = wsum[r] * corr + w;
#pragma unroll
                for (int e = 0; e < EPL; e++) acc[r][e] = acc[r][e] * corr + w * oj[q][r][e];
                m[r] = m_new;
            }
    }
#pragma unroll
    for (int r = 0; r < RPW; r++) {
        const int row = row0 + r;
        if (row >= rows) break;
        const float inv = wsum[r] > 0.f ? 1.f / wsum[r] : 0.f;
        __bf16 *orow = a.o + (size_t)row * H + lane * EPL;
#pragma unroll
        for (int e = 0; e < EPL; e++) orow[e] = (__bf16)(acc[r][e] * inv);
        if (lane == 0 && a.lse) a.lse[row] = wsum[r] > 0.f ? m[r] + logf(wsum[r]) : -INFINITY;
    }
}

hipError_t launch_fwd_merge(const FwdArgs &a, int H, hipStream_t stream) {
    const int rows = a.B * a.K * a.G * a.T;
    const int waves = (rows + kMergeRows - 1) / kMergeRows;
    const dim3 grid((unsigned)((waves + 3) / 4));
    switch (H) {
        case 64: hipLaunchKernelGGL((attn_fwd_merge_kernel<64>), grid, dim3(256), 0, stream, a, rows); break;
        case 128: hipLaunchKernelGGL((attn_fwd_merge_kernel<128>), grid, dim3(256), 0, stream, a, rows); break;
        case 256: hipLaunchKernelGGL((attn_fwd_merge_kernel<256>), grid, dim3(256), 0, stream, a, rows); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// Split-KV pays when the usual grid leaves the GPU idle (few (b, kv head)
// units and query blocks, as in decoding with T << S): the key range is then
// cut into splits of whole tiles until the grid has about split_target
// workgroups, keeping at least kMinSplitTiles tiles per split.
SplitPlan fwd_split_plan(int B, int K, int G, int T, int S, int H, int split_target) {
    const long long kTargetBlocks = split_target;
    constexpr int kMinSplitTiles = 4;
    const FwdConfig full = fwd_config(G, T, H);
    const long long base_full = (long long)B * K * (G / full.gw) * ((T + full.bq - 1) / full.bq);
    const FwdConfig cfg = fwd_config_split(G, T, H);
    const long long base = (long long)B * K * (G / cfg.gw) * ((T + cfg.bq - 1) / cfg.bq);
    const int n_tiles = (S + cfg.bkv - 1) / cfg.bkv;
    SplitPlan p{1, n_tiles};
    if (split_target <= 0 || base_full >= kTargetBlocks / 2 || n_tiles < 2 * kMinSplitTiles) return p;
    int want = (int)((kTargetBlocks + base - 1) / base);
    want = min(want, n_tiles / kMinSplitTiles);
    if (want < 2) return p;
    p.split_tiles = (n_tiles + want - 1) / want;
    p.n_splits = (n_tiles + p.split_tiles - 1) / p.split_tiles;
    return p;
}

// ---------------------------------------------------------------------------
// The runtime tuning table (tuning/mi355x.json, via the generated
// tuning_table.inc): the first row that matches a call gives its choice.
namespace {
struct LoadPlacementRow {
    int H, causal, segments, window, g8, t_min, t_max, s_min, s_max, value;
};
struct SplitTargetRow {
    int H, t_min, t_max, s_min, s_max, value;
};
#include "tuning_table.inc"
inline bool hit(int want, int have) { return want < 0 || want == have; }
}  // namespace

int fwd_split_target(int T, int S, int H) {
    for (const SplitTargetRow &r : kSplitTargetRows)
        if (hit(r.H, H) && T >= r.t_min && T <= r.t_max && S >= r.s_min && S <= r.s_max) return r.value;
    return 1024;
}

FwdTuning fwd_tuning(int G, int T, int S, int H, const MaskSpec &m, bool segments) {
    FwdTuning t{0, fwd_split_target(T, S, H)};
    // the window column: 0 nothing beyond the causal diagonal, 1 a causal left
    // window only, 2 anything else (prefix keys, right windows)
    const int window = !mask_extra(m) ? 0 : (mask_left_window_only(m) ? 1 : 2);
    for (const LoadPlacementRow &r : kLoadPlacementRows) {
        if (hit(r.H, H) && hit(r.causal, m.causal) && hit(r.segments, segments ? 1 : 0) && hit(r.window, window) &&
            hit(r.g8, G % 8 == 0 ? 1 : 0) && T >= r.t_min && T <= r.t_max && S >= r.s_min && S <= r.s_max) {
            t.load_placement = r.value;
            break;
        }
    }
    return t;
}

// H = 256 on the ping-pong kernel: 8 waves of 32 query rows (gw = 8 heads by
// bq = 32 queries) over 32-key tiles, for dense shapes: no segment ids, no
// window or prefix, whole key tiles, and when causal T + coff == S with the
// diagonal offset coff a whole number of tiles (the diagonal tile is then
// each block's last).
bool fwd_pp256_applies(int G, int T, int S, const MaskSpec &m, bool segments) {
    return G % 8 == 0 && !segments && !mask_extra(m) &&
           (!m.causal || (m.coff >= 0 && m.coff % 32 == 0 && T + m.coff == S));
}

FwdConfig fwd_config_pp256() {
    FwdConfig cfg;
    cfg.nw = 8;
    cfg.gw = 8;
    cfg.bq = 32;
    cfg.bkv = 32;
    return cfg;
}

static hipError_t launch_fwd_pp256(const FwdArgs &a, hipStream_t stream) {
    const unsigned grid = (unsigned)(a.B * a.K * a.n_gsplit * a.n_qblocks);
    if (a.causal)
        launch_pp<256, 32, true, false, false>(a, grid, stream);
    else
        launch_pp<256, 32, false, false, false>(a, grid, stream);
    return hipGetLastError();
}

// Split-KV on the ping-pong kernel: H <= 128, no segment ids, no window or
// prefix, and when causal the dense kernel's diagonal structure (one query
// block per key tile, the diagonal offset a whole number of tiles). The call
// then uses fwd_config's 8-wave blocks.
bool fwd_pp_split_applies(int G, int T, int S, int H, const MaskSpec &m, bool segments) {
    if (H > 128 || segments || mask_extra(m)) return false;
    const FwdConfig cfg = fwd_config(G, T, H);
    return !m.causal || (m.coff >= 0 && m.coff % cfg.bkv == 0 && T + m.coff == S && cfg.bq == cfg.bkv);
}

template <int H>
static hipError_t launch_fwd_pp_split(const FwdArgs &a, hipStream_t stream) {
    const dim3 grid((unsigned)(a.B * a.K * a.n_gsplit * a.n_qblocks * a.n_splits));
    const bool rag = a.S % 64 != 0;
    if (a.causal && rag)
        hipLaunchKernelGGL((attn_fwd_pp_split_kernel<H, 64, true, true>), grid, dim3(512), 0, stream, a);
    else if (a.causal)
        hipLaunchKernelGGL((attn_fwd_pp_split_kernel<H, 64, true, false>), grid, dim3(512), 0, stream, a);
    else if (rag)
        hipLaunchKernelGGL((attn_fwd_pp_split_kernel<H, 64, false, true>), grid, dim3(512), 0, stream, a);
    else
        hipLaunchKernelGGL((attn_fwd_pp_split_kernel<H, 64, false, false>), grid, dim3(512), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_fwd(const FwdArgs &a, int H, hipStream_t stream) {
    if (a.o_part) {
        const MaskSpec m{a.causal, a.coff, a.wl, a.wr, a.prefix};
        if (fwd_decode_applies(a.G, a.T, H, m, a.q_seg != nullptr)) {
            const unsigned grid = (unsigned)(a.B * a.K * a.n_splits);
            if (H == 64)
                hipLaunchKernelGGL((attn_fwd_decode_kernel<64, 5>), dim3(grid), dim3(256), 0, stream, a);
            else if (H == 128)
                hipLaunchKernelGGL((attn_fwd_decode_kernel<128, 4>), dim3(grid), dim3(256), 0, stream, a);
            else
                hipLaunchKernelGGL((attn_fwd_decode_kernel<256, 2>), dim3(grid), dim3(256), 0, stream, a);
            return hipGetLastError();
        }
        // the ping-pong kernel's blocks (the call's configuration is fwd_config's)
        if (a.gw * a.bq == 256 && fwd_pp_split_applies(a.G, a.T, a.S, H, m, a.q_seg != nullptr)) {
            if (H == 64) return launch_fwd_pp_split<64>(a, stream);
            if (H == 128) return launch_fwd_pp_split<128>(a, stream);
        }
        switch (H) {
            case 64: return launch_fwd_split_t<64, 64, 2>(a, stream);
            case 128: return launch_fwd_split_t<128, 64, 2>(a, stream);
            case 256: return launch_fwd_split_t<256, 32, 1>(a, stream);
            default: return hipErrorInvalidValue;
        }
    }
    switch (H) {
        case 64: return launch_fwd_t<64, 64, 8, 2>(a, stream);
        case 128: return launch_fwd_t<128, 64, 8, 2>(a, stream);
        case 256:
            // a configuration from fwd_config_pp256 (all 8 waves hold rows)
            if (a.gw * a.bq == 256) return launch_fwd_pp256(a, stream);
            return launch_fwd_t<256, 32, 4, 1>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gqa
