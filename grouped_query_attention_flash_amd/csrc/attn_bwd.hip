// Fused grouped-query flash attention, backward pass, for gfx950 (MI355X).
//
// The pages give no backward math; this is the standard calculus of softmax
// attention, recomputing the weights from the forward's saved logsumexp
// (the residual that splash attention's save_residuals option keeps,
// danielwatson6.github.io/fa, "Our first kernel"), split into a dK/dV
// kernel and a dQ kernel as the separate *_dkv and *_dq block sizes of the
// fjformer BlockSizes dataclass do:
//   P  = exp(S - lse),  S = q.k (no scale)
//   dP = dO V^T,  D = rowsum(P * dP)                          (bwd_dq<DELTA>)
//   dS = P * (dP - D)
//   dV = sum_{g,t} P^T dO,  dK = sum_{g,t} dS^T Q             (bwd_dkv)
//   dQ = dS K                                                 (bwd_dq)
// All contractions run on the 32x32x16 bf16 MFMA with fp32 accumulation;
// P and dS are rounded to bf16 as MFMA operands, except that dS enters the
// dQ product as a bf16 hi + lo pair (in the ping-pong dQ kernel, on the tiles
// where |dS| is large enough for the lo part to matter). Gradients are written in fp32. The G-sum
// of dK/dV stays inside one workgroup: no atomics, and the result is
// deterministic. The D pass also stores lse * log2(e) per row beside D, the
// form in which the dK/dV kernel takes it.
//
// D equals rowsum(dO * O) in exact arithmetic, but the forward's O carries
// the rounding of P to bf16 in its PV product; D taken from it moves dQ by
// up to ~1e-1 on early causal rows (where |dS| ~ 10). D is therefore summed
// in fp32 from the recomputed weights, in a pass of its own over K and V.
#include "gqa_device.h"
#include "gqa_launch.h"

#include <climits>
#include <cmath>
#include <type_traits>
#include <utility>

// LDS operand reads of the ping-pong M phases (D pass and dQ) are issued this
// many MFMA steps ahead of their use
constexpr int kBwdPrefetch = 2;

// The ping-pong dQ kernel adds the bf16 lo part of dS (dS - bf16(dS)) into
// dQ only on a wave's tiles where some |dS| exceeds this bound. The dropped
// part of an element is at most 2^-8 of it, and on a skipped tile every |dS|
// is at most 1/4. On N(0, 1) inputs with causal T = S = 8192, |dS| on a tile
// falls roughly as 200 / t, so rows past t ~ 800 skip it; dQ then moves by at
// most 4.9e-3 against the hi + lo sum (5.2e-3 with a 1024-key window), where
// dropping it on every tile moves it by 0.11 on the early rows.
constexpr float kDsLoMin = 0.25f;

namespace gqa {

// Interleave pattern of a ping-pong M phase for the machine scheduler: NX
// steps of NM MFMAs, the R LDS operand reads of step X issued after the
// MFMAs of step X - D (the first D steps' reads up front).
template <int X, int NX, int R>
__device__ __forceinline__ void pp_sched_reads() {
    if constexpr (X < NX) __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
}
template <int X, int NX, int NM, int R, int D>
__device__ __forceinline__ void pp_sched_step() {
    __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
    pp_sched_reads<X + D, NX, R>();
}
template <int NX, int NM, int R, int D, int... P, int... X>
__device__ __forceinline__ void pp_schedule(std::integer_sequence<int, P...>, std::integer_sequence<int, X...>) {
    (pp_sched_reads<P, NX, R>(), ...);
    (pp_sched_step<X, NX, NM, R, D>(), ...);
}

// Segment ids for the ping-pong D and dQ kernels (512 threads, at most 8192
// keys): stages the kv ids of key tiles 0 .. nt - 1 (BKV keys each) in s_kvid
// with each tile's id range, and lists in s_jlist, in increasing order, the
// tiles whose range meets the id range of the block's queries t0 .. t0 + bq
// - 1 (the others hold no visible pair). Returns the list's length, the same
// in every wave. Every id load is in flight before the first use.
constexpr int kSegKeyCap = 8192;
template <int BKV>
__device__ __forceinline__ int seg_tile_list(const int32_t *qs, const int32_t *kvs, int t0, int bq, int T, int nt,
                                             int *s_kvid, int *s_tmin, int *s_tmax, int *s_jlist, int *s_cnt) {
    static_assert(BKV == 32 || BKV == 64, "a tile is one wave or half of one");
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    constexpr int PER = kSegKeyCap / 512;
    const int nkeys = nt * BKV;  // >= BKV
    int id[PER], qb_id[4];
#pragma unroll
    for (int m = 0; m < 4; m++) qb_id[m] = qs[min(t0 + lane + 64 * m, T - 1)];
#pragma unroll
    for (int m = 0; m < PER; m++) id[m] = kvs[min(tid + 512 * m, nkeys - 1)];
    int qlo = INT_MAX, qhi = INT_MIN;
#pragma unroll
    for (int m = 0; m < 4; m++) {
        const int i = lane + 64 * m;
        if (i < bq && t0 + i < T) {
            qlo = min(qlo, qb_id[m]);
            qhi = max(qhi, qb_id[m]);
        }
    }
    qlo = wave_min_i(qlo);
    qhi = wave_max_i(qhi);
#pragma unroll
    for (int m = 0; m < PER; m++) {
        const int k = tid + 512 * m;
        if (512 * m + 64 * wave < nkeys) {  // wave-uniform; whole tiles below nkeys
            const bool ok = k < nkeys;
            if (ok) s_kvid[k] = id[m];
            int lo = ok ? id[m] : INT_MAX, hi = ok ? id[m] : INT_MIN;
#pragma unroll
            for (int o = BKV / 2; o >= 1; o >>= 1) {
                lo = min(lo, __shfl_xor(lo, o));
                hi = max(hi, __shfl_xor(hi, o));
            }
            if (ok && (lane & (BKV - 1)) == 0) {
                s_tmin[k / BKV] = lo;
                s_tmax[k / BKV] = hi;
            }
        }
    }
    __syncthreads();
    if (wave == 0) {
        int cnt = 0;
        for (int jb = 0; jb < nt; jb += 64) {
            const int j = jb + lane;
            const bool vis = j < nt && !(s_tmax[j] < qlo || s_tmin[j] > qhi);
            const unsigned long long m = __ballot(vis);
            if (vis) s_jlist[cnt + __popcll(m & ((1ull << lane) - 1))] = j;
            cnt += __popcll(m);
        }
        if (lane == 0) *s_cnt = cnt;
    }
    __syncthreads();
    return __builtin_amdgcn_readfirstlane(*s_cnt);
}

// Per-head masks on the ping-pong D and dQ kernels: the block's key tiles are
// the union of its gw heads' ranges, [first, last] of BKV-key tiles (each
// wave computes it from the table, one lane per head), and a wave masks with
// its own head's sides and prefix. Whole tiles (S % BKV == 0).
template <int BKV>
struct HmRange {
    int first, last;
};
template <int BKV>
__device__ __forceinline__ HmRange<BKV> hm_union(const BwdArgs &a, int kh, int g0, int gw, int t0, int bq) {
    const int lane = threadIdx.x & 63;
    int f = INT_MAX, l = INT_MIN;
    if (lane < gw) {
        const HeadMask h = head_mask_of(a.head_mask, kh, a.G, g0 + lane, a.T, a.S, a.causal, a.coff);
        f = h.pfx > 0 ? 0 : max(0, t0 - h.wl) / BKV;
        l = min(a.S / BKV - 1, max(h.pfx - 1, t0 + bq - 1 + h.wr) / BKV);
    }
    return HmRange<BKV>{wave_min_i(f), wave_max_i(l)};
}


// ---------------------------------------------------------------------------
// dK, dV. One workgroup per (b, kv head, block of 32*NW keys); wave w owns
// keys [s0 + 32w, s0 + 32w + 32). The workgroup walks every query head g
// and every query tile of BQ = 32 rows that can see its keys; Q, dO, lse
// and D of the tile are staged in LDS and shared by the waves.
//
// Per wave and query tile (M = queries, N = the wave's 32 keys):
//   S  = Q K^T    A: Q rows (LDS)         B: K^T (registers)
//   dP = dO V^T   A: dO rows (LDS)        B: V^T (registers)
//   lane (n, c) holds key n and the 16 queries acc_row(r, c) of S, P, dP, dS
//   dV^T += dO^T P   A: dO^T (LDS transpose read)   B: P  (registers, bf16)
//   dK^T += Q^T dS   A: Q^T  (LDS transpose read)   B: dS (registers, bf16)
// PART: 0 computes dK and dV; 1 only dV (S, P, dV^T); 2 only dK (S, dP, dS,
// dK^T). At H = 256 the two accumulators of one pass would fill a wave's
// registers, so two passes run, one per part.
template <int H, int NW, int PART>
__global__ __launch_bounds__(NW * 64) void attn_bwd_dkv_kernel(BwdArgs a, int n_kblocks) {
    constexpr bool DO_DV = PART != 2, DO_DK = PART != 1;
    constexpr int BQ = 32;
    constexpr int CPR = H / 8;
    constexpr int KSTEPS = H / 16;
    constexpr int HB = H / 32;
    constexpr int NT = NW * 64;
    constexpr int TILE_CHUNKS = BQ * CPR;                 // per tensor (Q or dO)
    constexpr int LOADS = (2 * TILE_CHUNKS + NT - 1) / NT;

    __shared__ __attribute__((aligned(16))) __bf16 sq[BQ * H];
    __shared__ __attribute__((aligned(16))) __bf16 sdo[BQ * H];
    __shared__ __attribute__((aligned(16))) float slse[BQ];  // lse * log2(e); +inf for empty rows
    __shared__ __attribute__((aligned(16))) float sdel[BQ];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 31, c = lane >> 5;
    const int T = a.T, S = a.S, G = a.G;

    // heaviest first: with causal masking the first key blocks see the most queries
    const int units = a.B * a.K;
    const int kb_idx = blockIdx.x / units;
    const int u = blockIdx.x % units;
    const int kh = u % a.K, b = u / a.K;
    const int s0_wg = kb_idx * 32 * NW;
    const int s_w = s0_wg + 32 * wave;      // first key of this wave
    const int s = s_w + n;                   // this lane's key
    const bool k_valid = s < S;
    const bool wave_active = s_w < S;
    const size_t bk = (size_t)b * a.K + kh;

    // K^T and V^T operands (B operands): lane (n, c), k-step ks holds row s, h = 16ks + 8c .. +7.
    // VLDS (H = 256): the V^T operands wait in LDS, in the wave's 32 rows of
    // svw (swizzled as the Q / dO tiles), and are read back per k-step: K^T,
    // V^T and both accumulators do not fit in one wave's registers together.
    constexpr bool VLDS = H > 128 && DO_DK;
    __shared__ __attribute__((aligned(16))) __bf16 svw[VLDS ? NW * 32 * H : 8];
    const int vrow_l = 32 * wave + n;  // the lane's row of svw
    bf16x8 kf[KSTEPS], vf[VLDS ? 1 : KSTEPS];
    {
        const __bf16 *krow = a.k + (bk * S + s) * H;
        const __bf16 *vrow = a.v + (bk * S + s) * H;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ks++) {
            kf[ks] = k_valid ? *(const bf16x8 *)(krow + 16 * ks + 8 * c) : bf16x8{};
            const bf16x8 vv = k_valid ? *(const bf16x8 *)(vrow + 16 * ks + 8 * c) : bf16x8{};
            if constexpr (VLDS)
                *(bf16x8 *)(svw + vrow_l * H + (((2 * ks + c) ^ swz<CPR>(vrow_l)) << 3)) = vv;
            else
                vf[ks] = vv;
        }
    }

    const bool segs = a.q_seg != nullptr;
    const int32_t *qsb = segs ? a.q_seg + (size_t)b * T : nullptr;
    int my_kid = 0, wg_kmin = INT_MAX, wg_kmax = INT_MIN, w_kmin = INT_MAX, w_kmax = INT_MIN;
    if (segs) {
        const int32_t *kvs = a.kv_seg + (size_t)b * S;
        int lo = INT_MAX, hi = INT_MIN;
        for (int i = lane; i < 32 * NW; i += 64) {
            if (s0_wg + i < S) {
                const int id = kvs[s0_wg + i];
                lo = min(lo, id);
                hi = max(hi, id);
            }
        }
        wg_kmin = wave_min_i(lo);
        wg_kmax = wave_max_i(hi);
        my_kid = k_valid ? kvs[s] : 0;
        w_kmin = wave_min_i(k_valid ? my_kid : INT_MAX);
        w_kmax = wave_max_i(k_valid ? my_kid : INT_MIN);
    }

    // query tiles that can see the block's keys: t in [s - R, s + L] for the
    // band sides L, R, or every query for a block that starts in the prefix.
    // Per-head masks: the range of the union over the kv head's G heads, and
    // each step takes its own head's sides (head_sides).
    int WLu = a.wl, WRu = a.wr, PFXu = a.prefix;
    if (a.head_mask) {
        WLu = WRu = INT_MIN;
        PFXu = 0;
        for (int i = 0; i < G; i++) {
            const HeadMask h = head_mask_of(a.head_mask, kh, G, i, T, S, a.causal, a.coff);
            WLu = max(WLu, h.wl);
            WRu = max(WRu, h.wr);
            PFXu = max(PFXu, h.pfx);
        }
    }
    auto head_sides = [&](int g, int &wl, int &wr, int &pfx) {
        if (a.head_mask) {
            const HeadMask h = head_mask_of(a.head_mask, kh, G, g, T, S, a.causal, a.coff);
            wl = h.wl, wr = h.wr, pfx = h.pfx;
        } else {
            wl = a.wl, wr = a.wr, pfx = a.prefix;
        }
    };
    const int n_qt_all = (T + BQ - 1) / BQ;
    const bool blk_pfx = s0_wg < PFXu;
    const int qt_begin = blk_pfx ? 0 : min(n_qt_all, max(0, s0_wg - WRu) / BQ);
    const int n_qt = blk_pfx ? n_qt_all
                             : max(qt_begin, min(n_qt_all, (s0_wg + 32 * NW - 1 + WLu) / BQ + 1));  // end of the tile range
    const int n_steps = G * (n_qt - qt_begin);  // (g, query tile) pairs, g outer

    auto q_ids = [&](int qt, int &qmin, int &qmax) {
        const int t = qt * BQ + lane;
        const bool ok = lane < BQ && t < T;
        const int id = ok ? qsb[t] : 0;
        qmin = wave_min_i(ok ? id : INT_MAX);
        qmax = wave_max_i(ok ? id : INT_MIN);
    };
    auto next_step = [&](int st) {
        if (!segs && !a.head_mask) return st;
        for (; st < n_steps; st++) {
            const int qt = qt_begin + st % (n_qt - qt_begin);
            if (a.head_mask) {
                // the step's head sees none of the block's keys from this tile
                int wl, wr, pfx;
                head_sides(st / (n_qt - qt_begin), wl, wr, pfx);
                const int t0 = qt * BQ;
                if (!(s0_wg < pfx || (t0 + BQ - 1 >= s0_wg - wr && t0 <= s0_wg + 32 * NW - 1 + wl))) continue;
            }
            if (segs) {
                int qmin, qmax;
                q_ids(qt, qmin, qmax);
                if (qmax < wg_kmin || qmin > wg_kmax) continue;
            }
            break;
        }
        return st;
    };

    i32x4 pre[LOADS];
    float pre_lse = 0.f, pre_del = 0.f;
    auto load_step = [&](int st) {
        const int g = st / (n_qt - qt_begin);
        const int t0 = (qt_begin + st % (n_qt - qt_begin)) * BQ;
        const size_t rowbase = (bk * G + g) * (size_t)T;
#pragma unroll
        for (int i = 0; i < LOADS; i++) {
            const int ci = tid + i * NT;
            if (ci < 2 * TILE_CHUNKS) {
                const int tensor = ci / TILE_CHUNKS;
                const int cc = ci % TILE_CHUNKS;
                const int r = cc / CPR, ch = cc % CPR;
                const int t = t0 + r;
                const __bf16 *src = (tensor ? a.dout : a.q) + (rowbase + t) * H + ch * 8;
                pre[i] = t < T ? *(const i32x4 *)src : i32x4{0, 0, 0, 0};
            }
        }
        if (tid < BQ) {
            const int t = t0 + tid;
            float l = INFINITY, d = 0.f;
            if (t < T) {
                l = a.lse[rowbase + t];
                l = (l == -INFINITY) ? INFINITY : l * kLog2e;  // empty row: every P is 0
                d = a.delta[rowbase + t];
            }
            pre_lse = l;
            pre_del = d;
        }
    };
    auto store_step = [&]() {
#pragma unroll
        for (int i = 0; i < LOADS; i++) {
            const int ci = tid + i * NT;
            if (ci < 2 * TILE_CHUNKS) {
                const int tensor = ci / TILE_CHUNKS;
                const int cc = ci % TILE_CHUNKS;
                const int r = cc / CPR, ch = cc % CPR;
                *(i32x4 *)((tensor ? sdo : sq) + r * H + ((ch ^ swz<CPR>(r)) << 3)) = pre[i];
            }
        }
        if (tid < BQ) {
            slse[tid] = pre_lse;
            sdel[tid] = pre_del;
        }
    };

    f32x16 dv_acc[HB], dk_acc[HB];
#pragma unroll
    for (int hb = 0; hb < HB; hb++) {
        dv_acc[hb] = f32x16{};
        dk_acc[hb] = f32x16{};
    }

    int st = next_step(0);
    if (st < n_steps) load_step(st);
    while (st < n_steps) {
        __syncthreads();
        store_step();
        __syncthreads();
        const int st_next = next_step(st + 1);
        if (st_next < n_steps) load_step(st_next);

        const int t0 = (qt_begin + st % (n_qt - qt_begin)) * BQ;
        int WL, WR, PFX;  // the step's head
        head_sides(st / (n_qt - qt_begin), WL, WR, PFX);
        bool run = wave_active && (s_w < PFX || (t0 + BQ - 1 >= s_w - WR && t0 <= s_w + 31 + WL));
        bool seg_mask = false;
        if (run && segs) {
            int qmin, qmax;
            q_ids(t0 / BQ, qmin, qmax);
            if (qmax < w_kmin || qmin > w_kmax) run = false;
            seg_mask = !(w_kmin == w_kmax && qmin == qmax && qmin == w_kmin);
        }
        if (run) {
            // S = Q K^T and dP = dO V^T, both 32 queries x 32 keys
            f32x16 sacc = f32x16{}, pacc = f32x16{};
            {
                const __bf16 *qrow = sq + n * H;
                const __bf16 *drow = sdo + n * H;
                const int sw = swz<CPR>(n);
#pragma unroll
                for (int ks = 0; ks < KSTEPS; ks++) {
                    const int off = ((2 * ks + c) ^ sw) << 3;
                    sacc = mfma32x32x16(*(const bf16x8 *)(qrow + off), kf[ks], sacc);
                    if constexpr (DO_DK) {
                        bf16x8 vk;
                        if constexpr (VLDS)
                            vk = *(const bf16x8 *)(svw + vrow_l * H + (((2 * ks + c) ^ swz<CPR>(vrow_l)) << 3));
                        else
                            vk = vf[ks];
                        pacc = mfma32x32x16(*(const bf16x8 *)(drow + off), vk, pacc);
                    }
                }
            }
            // keys wholly inside the prefix need no band mask
            const bool band_mask = s_w + 31 >= PFX && ((s_w + 31 > t0 + WR) || (s_w < t0 + BQ - 1 - WL));
            const bool need_mask = band_mask || (s_w + 32 > S) || (t0 + BQ > T) || seg_mask;
            // P = exp2(S log2e - lse log2e); dS = P (dP - D)
#pragma unroll
            for (int q4 = 0; q4 < 4; q4++) {
                const int r0 = 8 * q4 + 4 * c;  // queries r0 .. r0+3 of the tile
                const f32x4 l4 = *(const f32x4 *)(slse + r0);
                const f32x4 d4 = *(const f32x4 *)(sdel + r0);
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int r = 4 * q4 + e;
                    float x = sacc[r];
                    if (need_mask) {
                        const int t = t0 + r0 + e;
                        bool vis = k_valid && t < T && ((s <= t + WR && s >= t - WL) || s < PFX);
                        if (segs && vis) vis = qsb[t] == my_kid;
                        if (!vis) x = -INFINITY;
                    }
                    const float p = exp2_fast(__builtin_fmaf(x, kLog2e, -l4[e]));
                    sacc[r] = p;
                    if constexpr (DO_DK) pacc[r] = p * (pacc[r] - d4[e]);
                }
            }
            // dV^T += dO^T P ; dK^T += Q^T dS   (k = queries, 2 k-steps of 16)
            const int gi = lane & 15, hh = (lane >> 4) & 1;
#pragma unroll
            for (int kk = 0; kk < 2; kk++) {
                bf16x8 pf, sf;
#pragma unroll
                for (int e = 0; e < 8; e++) {
                    pf[e] = (__bf16)sacc[8 * kk + e];
                    sf[e] = (__bf16)pacc[8 * kk + e];
                }
                const int r0 = 16 * kk + 4 * c + (gi >> 2);
                const int r1 = r0 + 8;
                const int sw0 = swz<CPR>(r0), sw1 = swz<CPR>(r1);
#pragma unroll
                for (int hb = 0; hb < HB; hb++) {
                    const int hcol = 32 * hb + 16 * hh + 4 * (gi & 3);
                    const int ch = hcol >> 3, within = hcol & 7;
                    const int o0 = r0 * H + ((ch ^ sw0) << 3) + within;
                    const int o1 = r1 * H + ((ch ^ sw1) << 3) + within;
                    if constexpr (DO_DV) {
                        const bf16x8 dot = join_bf16x8(lds_read_tr16(sdo + o0), lds_read_tr16(sdo + o1));
                        dv_acc[hb] = mfma32x32x16(dot, pf, dv_acc[hb]);
                    }
                    if constexpr (DO_DK) {
                        const bf16x8 qt = join_bf16x8(lds_read_tr16(sq + o0), lds_read_tr16(sq + o1));
                        dk_acc[hb] = mfma32x32x16(qt, sf, dk_acc[hb]);
                    }
                }
            }
        }
        st = st_next;
    }

    // dK, dV rows (fp32): lane (n, c) holds h = 32hb + acc_row(r, c) of key s
    if (k_valid) {
        float *dkrow = a.dk + (bk * S + s) * H;
        float *dvrow = a.dv + (bk * S + s) * H;
#pragma unroll
        for (int hb = 0; hb < HB; hb++)
#pragma unroll
            for (int q4 = 0; q4 < 4; q4++) {
                const int h = 32 * hb + 8 * q4 + 4 * c;
                if constexpr (DO_DK)
                    *(f32x4 *)(dkrow + h) = f32x4{dk_acc[hb][4 * q4], dk_acc[hb][4 * q4 + 1], dk_acc[hb][4 * q4 + 2],
                                                  dk_acc[hb][4 * q4 + 3]};
                if constexpr (DO_DV)
                    *(f32x4 *)(dvrow + h) = f32x4{dv_acc[hb][4 * q4], dv_acc[hb][4 * q4 + 1], dv_acc[hb][4 * q4 + 2],
                                                  dv_acc[hb][4 * q4 + 3]};
            }
    }
    (void)n_kblocks;
}

// ---------------------------------------------------------------------------
// dK, dV for shapes without segment ids at H <= 128, with the work of each
// 32-key block split over a pair of waves so that two waves share every SIMD
// (one wave per SIMD would leave its own VALU work in the way of its MFMAs).
// One workgroup per (b, kv head, 128 keys), 8 waves: wave p (p < 4, "A") and
// wave p + 4 ("B") own keys [s0 + 32p, s0 + 32p + 32). Per 32-query step
// (the same (g, query tile) walk as the kernel above):
//   A:  S = Q K^T (K^T in registers), P = exp2(S log2e - lse log2e) with the
//       mask, dV^T += dO^T P; P also goes to LDS in fp32 for B
//   B:  dP = dO V^T (V^T in registers), dS = P (dP - D) with P from A,
//       dK^T += Q^T dS
// Lane (n, c) holds key n and queries acc_row(r, c) of S, P, dP, dS in both
// waves, so A's P reaches B lane to lane.
//
// Iteration i has two phases (workgroup barriers between), so that the two
// waves of a SIMD alternate between MFMA and VALU work:
//   phase 1: A  MFMAs S(i+2), dV(i)    B  VALU dS(i) from dP(i) and P(i)
//   phase 2: A  VALU P(i+1) from S(i+1), written to exchange buffer (i+1) % 2
//            B  MFMAs dP(i+1), dK(i)
// B reads P(i) from exchange buffer i % 2, written by A in the iteration
// before. Q, dO, lse and D of each step go straight from memory into a
// five-stage LDS ring: A waves load the Q tile and lse, B waves the dO tile
// and D. Iteration i reads steps i .. i+2 and loads step i+4 into the stage of
// step i-1, whose last readers finished in iteration i-1; every wave waits for
// its own loads one iteration later, a barrier before anyone reads them.
//
// SEG (segment ids, T <= 8192): the walk covers only the query tiles whose id
// range meets the ids of the block's keys (a list built at the start, the
// same for every wave), and a step whose ids are not all one value takes the
// element mask, which compares the lane's key id with the step's query ids
// (loaded beside lse, lanes 0-7 of one A wave).
//
// HM (per-head masks, G <= 64): each head walks its own query tile range,
// from its window sides and prefix (head_mask_of), and masks with them.
template <int H, bool CAUSAL, bool SEG = false, bool HM = false>
__global__ __launch_bounds__(512, 1) void attn_bwd_dkv3_kernel(BwdArgs a) {
    static_assert(!(SEG && HM), "segment ids or per-head masks");
    constexpr int NP = 4, BQ = 32;  // wave pairs, queries per step
    constexpr int CPR = H / 8;
    constexpr int KSTEPS = H / 16;
    constexpr int HB = H / 32;
    // Q / dO tile layout (16-byte chunks): rows RS = CPR + 4 chunks apart,
    // one more chunk after every 4 rows (group stride GS). The row reads (16
    // lanes: 16 rows, one chunk each) and the transposed reads (32 lanes: 4
    // rows, 4 chunks each) then both meet 16 distinct 4-bank groups of the
    // 64 banks, so neither has bank conflicts, and every read's offset is a
    // constant added to one base address per lane.
    constexpr int RS = CPR + 4;
    constexpr int GS = 4 * RS + 1;
    constexpr int TBLK = (BQ / 4 * GS + 63) / 64;  // 1 KiB wave loads per tile
    constexpr int TILE = TBLK * 512;
    constexpr int TBW = (TBLK + NP - 1) / NP;   // tile loads per wave and step
    constexpr int NLD = TBW + 1;                // + lse (wave 0) or D (wave 4)
    constexpr int NSTAGE = 5;
    __shared__ __attribute__((aligned(1024))) __bf16 sq[NSTAGE][TILE];
    __shared__ __attribute__((aligned(1024))) __bf16 sdo[NSTAGE][TILE];
    __shared__ __attribute__((aligned(1024))) float sld[NSTAGE][2][256];  // lse (SEG: + query ids), D (32 used)
    __shared__ __attribute__((aligned(1024))) f32x4 sp[2][NP][4][64];      // P exchange: [buf][pair][q4][lane]
    __shared__ __attribute__((aligned(1024))) char sdummy[1024];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool is_a = wave < NP;
    const int pair = wave & (NP - 1);
    const int n = lane & 31, c = lane >> 5;
    const int T = a.T, S = a.S, G = a.G;

    const int units = a.B * a.K;
    const int kb_idx = blockIdx.x / units;  // heaviest (causal) key block first
    const int u = blockIdx.x % units;
    const int kh = u % a.K, b = u / a.K;
    const int s0_wg = kb_idx * 32 * NP;
    const int s_w = s0_wg + 32 * pair;
    const int s = s_w + n;
    const bool k_valid = s < S;
    const size_t bk = (size_t)b * a.K + kh;

    // A: K^T, B: V^T (the B operands of S and dP): lane (n, c), k-step ks holds
    // row s, h = 16 ks + 8 c .. + 7
    bf16x8 kv[KSTEPS];
    {
        const __bf16 *row = (is_a ? a.k : a.v) + (bk * S + s) * H;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ks++) kv[ks] = k_valid ? *(const bf16x8 *)(row + 16 * ks + 8 * c) : bf16x8{};
    }

    // query tiles that can see the block's keys (as in the kernel above)
    const int WL = a.wl, WR = a.wr;
    const int n_qt = (T + BQ - 1) / BQ;
    const bool blk_pfx = s0_wg < a.prefix;
    const int qt_begin = blk_pfx ? 0 : min(n_qt, max(0, s0_wg - WR) / BQ);
    const int qt_end = blk_pfx ? n_qt : max(qt_begin, min(n_qt, (s0_wg + 32 * NP - 1 + WL) / BQ + 1));

    // HM: each head's window sides, prefix and query tile range, and the
    // number of steps over all heads, from wave 0 (one lane per head)
    constexpr int HM_CAP = HM ? 64 : 1;
    __shared__ int s_hwl[HM_CAP], s_hwr[HM_CAP], s_hpf[HM_CAP], s_hlo[HM_CAP], s_hhi[HM_CAP], s_hsteps;
    if constexpr (HM) {
        if (wave == 0) {
            int cnt = 0;
            if (lane < G) {
                const HeadMask h = head_mask_of(a.head_mask, kh, G, lane, T, S, a.causal, a.coff);
                const bool bp = s0_wg < h.pfx;
                const int lo = bp ? 0 : min(n_qt, max(0, s0_wg - h.wr) / BQ);
                const int hi = bp ? n_qt : max(lo, min(n_qt, (s0_wg + 32 * NP - 1 + h.wl) / BQ + 1));
                s_hwl[lane] = h.wl;
                s_hwr[lane] = h.wr;
                s_hpf[lane] = h.pfx;
                s_hlo[lane] = lo;
                s_hhi[lane] = hi;
                cnt = hi - lo;
            }
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) cnt += __shfl_xor(cnt, o);
            if (lane == 0) s_hsteps = cnt;
        }
        __syncthreads();
    }

    // SEG: the key's id, the pair's id range, and the list of the query tiles
    // in [qt_begin, qt_end) whose id range meets the block's (s_qtl[0 ..
    // n_vis)); otherwise the walk is [qt_begin, qt_end)
    constexpr int QT_CAP = SEG ? 8192 / BQ : 1;
    __shared__ int s_tmin[QT_CAP], s_tmax[QT_CAP], s_qtl[QT_CAP];
    __shared__ int s_krange[2 * NP + 1];
    int my_kid = 0, p_kmin = 0, p_kmax = 0;
    int q_lo = qt_begin, q_hi = qt_end;
    if constexpr (SEG) {
        const int32_t *qs = a.q_seg + (size_t)b * T;
        const int32_t *kvs = a.kv_seg + (size_t)b * S;
        // ids of the query tiles qt_begin + 2 wave + (lane >> 5) + 16 m, all
        // loads in flight before the first use (clamped in-range indices)
        constexpr int QM = QT_CAP / 16;
        int qid[QM];
#pragma unroll
        for (int m = 0; m < QM; m++) {
            const int qt = qt_begin + 2 * wave + (lane >> 5) + 16 * m;
            qid[m] = qs[min(qt * BQ + n, T - 1)];
        }
        my_kid = kvs[min(s, S - 1)];
        p_kmin = wave_min_i(k_valid ? my_kid : INT_MAX);
        p_kmax = wave_max_i(k_valid ? my_kid : INT_MIN);
        if (is_a && lane == 0) {
            s_krange[2 * pair] = p_kmin;
            s_krange[2 * pair + 1] = p_kmax;
        }
#pragma unroll
        for (int m = 0; m < QM; m++) {
            const int qt = qt_begin + 2 * wave + (lane >> 5) + 16 * m;
            if (qt < qt_end) {  // wave-uniform per half: both halves' tiles below qt_end, or one
                const bool ok = qt * BQ + n < T;
                int lo = ok ? qid[m] : INT_MAX, hi = ok ? qid[m] : INT_MIN;
#pragma unroll
                for (int o = 16; o >= 1; o >>= 1) {
                    lo = min(lo, __shfl_xor(lo, o));
                    hi = max(hi, __shfl_xor(hi, o));
                }
                if (n == 0) {
                    s_tmin[qt] = lo;
                    s_tmax[qt] = hi;
                }
            }
        }
        __syncthreads();
        if (wave == 0) {
            int bmin = INT_MAX, bmax = INT_MIN;
#pragma unroll
            for (int p = 0; p < NP; p++) {
                bmin = min(bmin, s_krange[2 * p]);
                bmax = max(bmax, s_krange[2 * p + 1]);
            }
            int cnt = 0;
            for (int jb = qt_begin; jb < qt_end; jb += 64) {
                const int qt = jb + lane;
                const bool vis = qt < qt_end && !(s_tmax[qt] < bmin || s_tmin[qt] > bmax);
                const unsigned long long m = __ballot(vis);
                if (vis) s_qtl[cnt + __popcll(m & ((1ull << lane) - 1))] = qt;
                cnt += __popcll(m);
            }
            if (lane == 0) s_krange[2 * NP] = cnt;
        }
        __syncthreads();
        q_lo = 0;
        q_hi = __builtin_amdgcn_readfirstlane(s_krange[2 * NP]);
    }
    const int n_steps = HM ? __builtin_amdgcn_readfirstlane(s_hsteps) : G * (q_hi - q_lo);

    // loads: A waves the Q tile (blocks pair, pair + 4, ...) and, wave 0, lse;
    // B waves the dO tile and, wave 4, D. Every wave issues NLD loads per step
    // without branches; a load with nothing to fetch gets an out-of-range
    // offset (reads nothing) and the dummy destination.
    const i32x4 trs = is_a ? make_rsrc_words(a.q + bk * G * (size_t)T * H, G * T * H * 2)
                           : make_rsrc_words(a.dout + bk * G * (size_t)T * H, G * T * H * 2);
    // SEG: wave 1 (an A wave) loads the step's query ids instead of nothing
    const bool ids_wave = SEG && is_a && pair == 1;
    const i32x4 lrs = ids_wave ? make_rsrc_words(a.q_seg + (size_t)b * T, T * 4)
                      : is_a   ? make_rsrc_words(a.lse2 + bk * G * (size_t)T, G * T * 4)
                               : make_rsrc_words(a.delta + bk * G * (size_t)T, G * T * 4);
    constexpr unsigned kOutOfRange = 0x80000000u;
    int t_off[TBW];
#pragma unroll
    for (int i = 0; i < TBW; i++) {
        // chunk p of the tile: row 4 (p / GS) + (p % GS) / RS; padding chunks
        // (and those past the last row) re-read an in-range chunk
        const int p = (pair + i * NP) * 64 + lane;
        const int rem = p % GS;
        const int row = min(4 * (p / GS) + min(rem / RS, 3), BQ - 1);
        t_off[i] = (row * H + min(rem % RS, CPR - 1) * 8) * 2;
    }
    const unsigned t_dst0 = (is_a ? lds_addr(sq[0]) : lds_addr(sdo[0])) + pair * 1024;
    // (offsets from sld's base as wave-uniform integers: lse at 0, the ids 32
    // floats on, D one row of 256 on)
    const unsigned l_dst0 =
        __builtin_amdgcn_readfirstlane(lds_addr(sld[0][0]) + (ids_wave ? 32u * 4u : is_a ? 0u : 256u * 4u));
    const unsigned dummy = lds_addr(sdummy);
    // row0: the step's first row g T + t (-1: none); t_row: its first query t
    auto issue_load = [&](int j, int row0, int t_row, int stage) {
        if (j < TBW) {
            const bool ok = row0 >= 0 && pair + j * NP < TBLK;
            const unsigned voff = ok ? (unsigned)(row0 * H * 2 + t_off[j]) : kOutOfRange;
            const unsigned dst = ok ? t_dst0 + stage * (TILE * 2) + j * NP * 1024 : dummy;
            lds_dma16(trs, __builtin_amdgcn_readfirstlane(dst), voff);
        } else if constexpr (SEG) {
            // 32 values, lanes 0-7 only: lse (wave 0) into sld[stage][0][0
            // .. 31], the query ids (wave 1) into [32 .. 63], D (wave 4)
            const bool ok = row0 >= 0 && (pair == 0 || ids_wave);
            const unsigned voff = ok ? (unsigned)((ids_wave ? t_row : row0) * 4 + (lane & 7) * 16) : kOutOfRange;
            const unsigned dst = __builtin_amdgcn_readfirstlane(ok ? l_dst0 + stage * (2 * 256 * 4) : dummy);
            if (lane < 8) lds_dma16(lrs, dst, voff);
        } else {
            // 32 floats: lanes 0-7 fetch them, the others repeat in-range
            // addresses into slots that are not read
            const bool ok = row0 >= 0 && pair == 0;
            const unsigned voff = ok ? (unsigned)(row0 * 4 + (lane & 7) * 16) : kOutOfRange;
            const unsigned dst = ok ? l_dst0 + stage * (2 * 256 * 4) : dummy;
            lds_dma16(lrs, __builtin_amdgcn_readfirstlane(dst), voff);
        }
        (void)t_row;
    };
    // (g, qi): head g, query tile qi (SEG: entry qi of the list; HM: hi is
    // the end of head g's range, and heads with an empty range are skipped)
    struct Cursor {
        int g, qi, hi;
    };
    auto hm_lo = [&](int g) { return __builtin_amdgcn_readfirstlane(s_hlo[g]); };
    auto hm_hi = [&](int g) { return __builtin_amdgcn_readfirstlane(s_hhi[g]); };
    // HM: the cursor at the first step of head g or the next head with steps
    auto hm_seek = [&](int g) {
        while (g < G && hm_lo(g) == hm_hi(g)) ++g;
        return g < G ? Cursor{g, hm_lo(g), hm_hi(g)} : Cursor{G, 0, 0};
    };
    auto first_cursor = [&]() {
        if constexpr (HM)
            return hm_seek(0);
        else
            return Cursor{0, q_lo, 0};
    };
    auto advance = [&](Cursor &cu) {
        if constexpr (HM) {
            if (++cu.qi >= cu.hi) cu = hm_seek(cu.g + 1);
        } else if (++cu.qi == q_hi) {
            cu.qi = q_lo;
            ++cu.g;
        }
    };
    auto qt_of = [&](const Cursor &cu) {
        if constexpr (SEG)
            return __builtin_amdgcn_readfirstlane(s_qtl[cu.g < G ? cu.qi : 0]);
        else
            return cu.qi;
    };
    auto row_of = [&](const Cursor &cu) { return cu.g < G ? cu.g * T + qt_of(cu) * BQ : -1; };

    f32x16 acc[HB];  // A: dV^T, B: dK^T
#pragma unroll
    for (int hb = 0; hb < HB; hb++) acc[hb] = f32x16{};

    const int row_lane = ((n >> 2) * GS + (n & 3) * RS) * 8 + c * 8;  // row n, chunk c
    const int gi = lane & 15, hh = (lane >> 4) & 1;
    // row 4 c + gi / 4 (group c, row gi / 4 of it), column 16 hh + 4 (gi & 3)
    const int tr_lane = c * GS * 8 + (gi >> 2) * RS * 8 + 16 * hh + 4 * (gi & 3);
    // S (A) or dP (B) of the step in `stage`: 32 queries x the pair's 32 keys
    auto sdp = [&](int stage, f32x16 &x) {
        const __bf16 *rowp = (is_a ? sq[stage] : sdo[stage]) + row_lane;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ks++) x = mfma32x32x16(*(const bf16x8 *)(rowp + 16 * ks), kv[ks], ks == 0 ? f32x16{} : x);
    };
    // visibility of (t, s): u = t - s + R in [0, min(L + R + 1, T - s + R)), as
    // in the kernel above (a prefix key takes unbounded sides)
    const bool k_pfx = s < a.prefix;
    const int LL = k_pfx ? kNoWindow : WL, RR = k_pfx ? kNoWindow : WR;
    const unsigned vis_bound = k_valid ? (unsigned)max(0, min(LL + RR + 1, T - s + RR)) : 0u;
    // lse * log2(e) (A) or D (B) of the lane's 16 query rows of the step in
    // `stage`, read into registers a phase before their use
    auto read_rows = [&](int stage, f32x4 (&r4)[4]) {
#pragma unroll
        for (int q4 = 0; q4 < 4; q4++) r4[q4] = *(const f32x4 *)(&sld[stage][is_a ? 0 : 1][8 * q4 + 4 * c]);
    };
    // A: P of a step from its S, its lse * log2(e) and first query t0; returns
    // the bf16 dV operand, writes fp32 P to exchange buffer `buf` and issues
    // one of the wave's loads after each group of four weights (ld(j)). The
    // lane's 16 rows are t0 + 4 c + {0..3, 8..11, 16..19, 24..27}; a step where
    // every lane sees all of them skips the mask.
    // SEG: st_ids is the stage holding the step's query ids.
    // HM: g_step is the step's head, whose sides and prefix replace the
    // call's.
    auto weights_a = [&](const f32x4 (&l4s)[4], int t0, const f32x16 &sx, bf16x8 (&pf)[2], int buf, auto ld,
                         int st_ids, int g_step) {
        int rr = RR;
        unsigned vbound = vis_bound;
        if constexpr (HM) {
            const int hpf = __builtin_amdgcn_readfirstlane(s_hpf[g_step]);
            const int hwl = __builtin_amdgcn_readfirstlane(s_hwl[g_step]);
            const int hwr = __builtin_amdgcn_readfirstlane(s_hwr[g_step]);
            const bool kp = s < hpf;
            const int l2 = kp ? kNoWindow : hwl;
            rr = kp ? kNoWindow : hwr;
            vbound = k_valid ? (unsigned)max(0, min(l2 + rr + 1, T - s + rr)) : 0u;
        }
        (void)g_step;
        const int tb = t0 + 4 * c - s + rr;
        auto body = [&](auto masked) {
#pragma unroll
            for (int q4 = 0; q4 < 4; q4++) {
                f32x4 p4;
                i32x4 qi4{};
                if constexpr (SEG && decltype(masked)::value)
                    qi4 = *(const i32x4 *)(&sld[st_ids][0][32 + 8 * q4 + 4 * c]);
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int r = 4 * q4 + e;
                    float p = exp2_fast(__builtin_fmaf(sx[r], kLog2e, -l4s[q4][e]));
                    if constexpr (decltype(masked)::value) {
                        bool vis = (unsigned)(tb + 8 * q4 + e) < vbound;
                        if constexpr (SEG) vis = vis && qi4[e] == my_kid;
                        p = vis ? p : 0.f;
                    }
                    p4[e] = p;
                    pf[r >> 3][r & 7] = (__bf16)p;
                }
                sp[buf][pair][q4][lane] = p4;
                if (q4 < NLD) ld(q4);
            }
        };
        // SEG: the step's ids and the pair's keys' ids all one value
        bool seg_open = true;
        if constexpr (SEG) {
            const int qt = t0 / BQ;
            const int qmn = __builtin_amdgcn_readfirstlane(s_tmin[qt]), qmx = __builtin_amdgcn_readfirstlane(s_tmax[qt]);
            seg_open = qmn == qmx && p_kmin == p_kmax && qmn == p_kmin;
        }
        (void)st_ids;
        if (seg_open && __all(tb >= 0 && tb + 27 < (int)vbound))
            body(std::integral_constant<bool, false>{});
        else
            body(std::integral_constant<bool, true>{});
        pin_value(pf[0]);
        pin_value(pf[1]);
    };
    // B: dS = P (dP - D) of a step, P from exchange buffer `buf`, loads
    // spread as in weights_a
    auto weights_b = [&](const f32x4 (&d4s)[4], const f32x16 &dpx, bf16x8 (&sf)[2], int buf, auto ld) {
        f32x4 p4s[4];
#pragma unroll
        for (int q4 = 0; q4 < 4; q4++) p4s[q4] = sp[buf][pair][q4][lane];
#pragma unroll
        for (int q4 = 0; q4 < 4; q4++) {
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int r = 4 * q4 + e;
                sf[r >> 3][r & 7] = (__bf16)(p4s[q4][e] * (dpx[r] - d4s[q4][e]));
            }
            if (q4 < NLD) ld(q4);
        }
        // formed here, in the VALU phase, not sunk into the MFMA phase that reads them
        pin_value(sf[0]);
        pin_value(sf[1]);
    };
    // M phase: the row product of the step in st_row (A: S = Q K^T, B: dP =
    // dO V^T) into x, and the outer product of the step in st_tr (A: dV^T +=
    // dO^T P, B: dK^T += Q^T dS) with the weights w, one of each per step x,
    // their LDS operand reads pinned two steps ahead
    auto m_phase = [&](int st_row, int st_tr, f32x16 &x, const bf16x8 (&w)[2], int st_rows, f32x4 (&r4)[4]) {
        const __bf16 *rowp = (is_a ? sq[st_row] : sdo[st_row]) + row_lane;
        const __bf16 *trp = (is_a ? sdo[st_tr] : sq[st_tr]) + tr_lane;
        // the next VALU phase's per-row values first (they land during the MFMAs)
        read_rows(st_rows, r4);
        sched_fence();
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int xs = 0; xs < KSTEPS; xs++) {
            x = mfma32x32x16(*(const bf16x8 *)(rowp + 16 * xs), kv[xs], xs == 0 ? f32x16{} : x);
            const int kk = xs / HB, hb = xs % HB;
            // rows 16 kk + ... (4 groups per 16 rows) and 8 rows (2 groups) further
            const __bf16 *base = trp + kk * 4 * GS * 8 + 32 * hb;
            acc[hb] = mfma32x32x16(join_bf16x8(lds_read_tr16(base), lds_read_tr16(base + 2 * GS * 8)), w[kk], acc[hb]);
        }
        pp_schedule<KSTEPS, 2, 3, 2>(std::make_integer_sequence<int, 2>(), std::make_integer_sequence<int, KSTEPS>());
        // the row product is read only in the next phase: keep the compiler
        // from sinking its MFMAs past the barrier into the VALU phase
        pin_value(x);
        __builtin_amdgcn_s_setprio(0);
    };

    // The whole walk for one role (ROLE_A: the A waves), so that the two roles'
    // registers never meet at a branch inside the loop.
    auto walk = [&](auto role) {
        constexpr bool ROLE_A = decltype(role)::value;
        // prologue: steps 0 .. 3 into stages 0 .. 3; A: P(0) (exchange buffer
        // 0) and S(1); B: dP(0)
        Cursor c_ld = first_cursor();
#pragma unroll
        for (int st = 0; st < 4; st++) {
            const int row_p = row_of(c_ld), t_p = qt_of(c_ld) * BQ;
#pragma unroll
            for (int j = 0; j < NLD; j++) issue_load(j, row_p, t_p, st);
            advance(c_ld);
        }
        wait_lds_loads();
        __syncthreads();
        f32x16 sa;     // A: S(i+1), B: dP(i) at the top of iteration i
        f32x16 sb;     // A: S(i+2), computed in phase 1
        bf16x8 w[2];   // A: P(i) (dV operand); B: dS(i) (dK operand)
        f32x4 r4[4];   // A: lse * log2(e) of step i+1; B: D of step i
        auto no_load = [](int) {};
        if constexpr (ROLE_A) {
            sdp(0, sb);
            read_rows(0, r4);
            const Cursor c0 = first_cursor();
            weights_a(r4, qt_of(c0) * BQ, sb, w, 0, no_load, 0, c0.g);
            sdp(1, sa);
        } else {
            sdp(0, sa);
            read_rows(0, r4);
        }
        Cursor c_w = first_cursor();  // A: step i+1 in iteration i
        advance(c_w);
        int st0 = 0, st1 = 1, st2 = 2, st4 = 4;  // stages of steps i, i+1, i+2, i+4
        // Two phases per iteration, separated by workgroup barriers, so that
        // on every SIMD one wave issues MFMAs while the other does its VALU
        // work:
        //   phase 1: A  S(i+2), dV(i)        B  dS(i); loads of step i+4
        //   phase 2: A  P(i+1); loads        B  dP(i+1), dK(i)
        // Each wave issues its loads of step i+4 in its VALU phase and then
        // waits for those of step i+3, one barrier before their first reader.
        for (int i = 0; i < n_steps; i++) {
            const int row_ld = row_of(c_ld), t_ld = qt_of(c_ld) * BQ;
            advance(c_ld);
            const int t1 = qt_of(c_w) * BQ, g1 = c_w.g;
            advance(c_w);
            auto ld = [&](int j) { issue_load(j, row_ld, t_ld, st4); };
            barrier_no_drain();
            if constexpr (ROLE_A) {
                m_phase(st2, st0, sb, w, st1, r4);  // and lse of step i+1
            } else {
                pin_value(sa);  // no weight work hoisted above the barrier
                weights_b(r4, sa, w, i & 1, ld);
                wait_lds_loads_but<NLD>();
            }
            barrier_no_drain();
            if constexpr (ROLE_A) {
                pin_value(sa);  // no weight work hoisted above the barrier
                weights_a(r4, t1, sa, w, (i + 1) & 1, ld, st1, g1);
                wait_lds_loads_but<NLD>();
                sa = sb;
            } else {
                m_phase(st1, st0, sa, w, st1, r4);  // and D of step i+1
            }
            st0 = st1;
            st1 = st2;
            st2 = st2 == NSTAGE - 1 ? 0 : st2 + 1;
            st4 = st4 == NSTAGE - 1 ? 0 : st4 + 1;
        }
        wait_lds_loads();
    };
    if (n_steps > 0) {
        if (is_a)
            walk(std::integral_constant<bool, true>{});
        else
            walk(std::integral_constant<bool, false>{});
    }

    // rows of key s (fp32): A writes dV, B dK; lane (n, c) holds h = 32 hb + acc_row(r, c)
    if (k_valid) {
        float *orow = (is_a ? a.dv : a.dk) + (bk * S + s) * H;
#pragma unroll
        for (int hb = 0; hb < HB; hb++)
#pragma unroll
            for (int q4 = 0; q4 < 4; q4++)
                *(f32x4 *)(orow + 32 * hb + 8 * q4 + 4 * c) =
                    f32x4{acc[hb][4 * q4], acc[hb][4 * q4 + 1], acc[hb][4 * q4 + 2], acc[hb][4 * q4 + 3]};
    }
}

// ---------------------------------------------------------------------------
// dQ. Same decomposition as the forward: one workgroup per (b, kv head,
// gw heads, bq queries), 32 query rows per wave, K/V tiles in LDS.
// Per wave and key tile (M = keys, N = the wave's 32 queries):
//   S^T  = K Q^T    A: K rows (LDS)    B: Q^T (registers)
//   dP^T = V dO^T   A: V rows (LDS)    B: dO^T (registers)
//   lane (n, c) holds query n: lse and D are one value per lane
//   dQ^T += K^T dS^T   A: K^T (LDS transpose read)   B: dS^T (registers, bf16)
//
// With DELTA set the kernel only computes D = rowsum(P * dP) in fp32 (the
// S^T and dP^T products and the weights) and writes it to the workspace.
template <int H, int BKV, int NW, bool DELTA>
__global__ __launch_bounds__(NW * 64) void attn_bwd_dq_kernel(BwdArgs a, int gw, int bq, int n_gsplit,
                                                              int n_qblocks) {
    constexpr int CPR = H / 8;
    constexpr int KSTEPS = H / 16;
    constexpr int MB = BKV / 32;
    constexpr int HB = H / 32;
    constexpr int PK = BKV / 16;
    constexpr int NT = NW * 64;
    constexpr int TILE_CHUNKS = BKV * CPR;
    static_assert(TILE_CHUNKS % NT == 0, "K and V loads must not share a step");
    constexpr int LOADS = 2 * TILE_CHUNKS / NT;

    __shared__ __attribute__((aligned(16))) __bf16 sk[BKV * H];
    __shared__ __attribute__((aligned(16))) __bf16 sv[BKV * H];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 31, c = lane >> 5;
    const int T = a.T, S = a.S;

    const int units = a.B * a.K * n_gsplit;
    int qb = blockIdx.x / units;
    if (a.causal) qb = n_qblocks - 1 - qb;
    const int u = blockIdx.x % units;
    const int gs = u % n_gsplit;
    const int kh = (u / n_gsplit) % a.K;
    const int b = u / (n_gsplit * a.K);
    const int t0 = qb * bq;

    const int rows_wg = gw * bq;
    const int rho = wave * 32 + n;
    const bool row_in_wg = rho < rows_wg;
    const int g = gs * gw + (row_in_wg ? rho / bq : 0);
    const int t = t0 + (row_in_wg ? rho % bq : 0);
    const bool q_valid = row_in_wg && t < T;
    const bool wave_active = wave * 32 < rows_wg;
    const int tmin_w = t0 + (bq >= 32 ? (wave * 32) % bq : 0);
    const int tmax_w = tmin_w + (bq >= 32 ? 31 : bq - 1);

    const size_t bk = (size_t)b * a.K + kh;
    const size_t row = (bk * a.G + g) * (size_t)T + t;

    bf16x8 qf[KSTEPS], df[KSTEPS];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ks++) {
        qf[ks] = q_valid ? *(const bf16x8 *)(a.q + row * H + 16 * ks + 8 * c) : bf16x8{};
        df[ks] = q_valid ? *(const bf16x8 *)(a.dout + row * H + 16 * ks + 8 * c) : bf16x8{};
    }
    float lse2 = INFINITY, dlt = 0.f;
    if (q_valid) {
        const float l = a.lse[row];
        lse2 = (l == -INFINITY) ? INFINITY : l * kLog2e;
        if constexpr (!DELTA) dlt = a.delta[row];
    }
    float d_acc = 0.f;  // DELTA: running sum of P * dP over this lane's keys

    const __bf16 *kbase = a.k + bk * (size_t)S * H;
    const __bf16 *vbase = a.v + bk * (size_t)S * H;

    const bool segs = a.q_seg != nullptr;
    const int32_t *kvs = segs ? a.kv_seg + (size_t)b * S : nullptr;
    int my_qid = 0, wg_qmin = INT_MAX, wg_qmax = INT_MIN, w_qmin = INT_MAX, w_qmax = INT_MIN;
    if (segs) {
        const int32_t *qs = a.q_seg + (size_t)b * T;
        int lo = INT_MAX, hi = INT_MIN;
        for (int i = lane; i < bq; i += 64) {
            if (t0 + i < T) {
                const int id = qs[t0 + i];
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

    // mask sides: WL, WR, PFX of this wave's head (its 32 rows are one head),
    // WLu, WRu, PFXu of the union over the block's heads (the call's own
    // without per-head masks)
    int WL = a.wl, WR = a.wr, PFX = a.prefix;
    int WLu = WL, WRu = WR, PFXu = PFX;
    if (a.head_mask) {
        const HeadMask hw = head_mask_of(a.head_mask, kh, a.G, __builtin_amdgcn_readfirstlane(g), T, S, a.causal,
                                         a.coff);
        WL = hw.wl, WR = hw.wr, PFX = hw.pfx;
        WLu = WRu = INT_MIN;
        PFXu = 0;
        for (int i = 0; i < gw; i++) {
            const HeadMask h = head_mask_of(a.head_mask, kh, a.G, gs * gw + i, T, S, a.causal, a.coff);
            WLu = max(WLu, h.wl);
            WRu = max(WRu, h.wr);
            PFXu = max(PFXu, h.pfx);
        }
    }

    // key tiles: the band of the block's first and last query, and the
    // prefix keys s < PFXu
    const int n_tiles = (S + BKV - 1) / BKV;
    const int t_last = min(t0 + bq, T) - 1;
    const int s_last = max(min(t_last + WRu, S - 1), PFXu - 1);
    const int j_end = s_last < 0 ? 0 : min(n_tiles, s_last / BKV + 1);
    const int j_begin = (PFXu > 0 || t0 - WLu <= 0) ? 0 : (t0 - WLu) / BKV;

    auto tile_ids = [&](int j, int &kmin, int &kmax) {
        const int ss = j * BKV + lane;
        const bool ok = lane < BKV && ss < S;
        const int id = ok ? kvs[ss] : 0;
        kmin = wave_min_i(ok ? id : INT_MAX);
        kmax = wave_max_i(ok ? id : INT_MIN);
    };
    // next tile at or after j inside the prefix or the block's band, and
    // (segment ids) sharing an id range with the block
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

    i32x4 pre[LOADS];
    auto load_tile = [&](int j) {
#pragma unroll
        for (int i = 0; i < LOADS; i++) {
            const int ci = tid + i * NT;
            const int tensor = ci / TILE_CHUNKS;
            const int cc = ci % TILE_CHUNKS;
            const int r = cc / CPR, ch = cc % CPR;
            const int ss = j * BKV + r;
            const __bf16 *src = (tensor ? vbase : kbase) + (size_t)ss * H + ch * 8;
            pre[i] = ss < S ? *(const i32x4 *)src : i32x4{0, 0, 0, 0};
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int i = 0; i < LOADS; i++) {
            const int ci = tid + i * NT;
            const int tensor = ci / TILE_CHUNKS;
            const int cc = ci % TILE_CHUNKS;
            const int r = cc / CPR, ch = cc % CPR;
            *(i32x4 *)((tensor ? sv : sk) + r * H + ((ch ^ swz<CPR>(r)) << 3)) = pre[i];
        }
    };

    f32x16 dq_acc[HB];
#pragma unroll
    for (int hb = 0; hb < HB; hb++) dq_acc[hb] = f32x16{};

    int j = j_begin < j_end ? next_tile(j_begin) : j_end;
    if (j < j_end) load_tile(j);
    while (j < j_end) {
        __syncthreads();
        store_tile();
        __syncthreads();
        const int jn = next_tile(j + 1);
        if (jn < j_end) load_tile(jn);

        const int s0 = j * BKV;
        bool run = wave_active && (s0 < PFX || (s0 <= tmax_w + WR && s0 + BKV - 1 >= tmin_w - WL));
        bool seg_mask = false;
        if (run && segs) {
            int kmin, kmax;
            tile_ids(j, kmin, kmax);
            if (kmax < w_qmin || kmin > w_qmax) run = false;
            seg_mask = !(w_qmin == w_qmax && kmin == kmax && kmin == w_qmin);
        }
        if (run) {
            f32x16 sacc[MB], pacc[MB];
#pragma unroll
            for (int mb = 0; mb < MB; mb++) {
                sacc[mb] = f32x16{};
                pacc[mb] = f32x16{};
                const int r = 32 * mb + n;
                const int sw = swz<CPR>(r);
#pragma unroll
                for (int ks = 0; ks < KSTEPS; ks++) {
                    const int off = r * H + (((2 * ks + c) ^ sw) << 3);
                    sacc[mb] = mfma32x32x16(*(const bf16x8 *)(sk + off), qf[ks], sacc[mb]);
                    pacc[mb] = mfma32x32x16(*(const bf16x8 *)(sv + off), df[ks], pacc[mb]);
                }
            }
            // a tile wholly inside the prefix needs no band mask
            const bool band_mask = s0 + BKV - 1 >= PFX && ((s0 + BKV - 1 > tmin_w + WR) || (s0 < tmax_w - WL));
            const bool need_mask = band_mask || (s0 + BKV > S) || seg_mask;
#pragma unroll
            for (int mb = 0; mb < MB; mb++)
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    float x = sacc[mb][r];
                    if (need_mask) {
                        const int ss = s0 + 32 * mb + acc_row(r, c);
                        bool vis = ss < S && ((ss <= t + WR && ss >= t - WL) || ss < PFX);
                        if (segs && vis) vis = kvs[ss] == my_qid;
                        if (!vis) x = -INFINITY;
                    }
                    const float p = exp2_fast(__builtin_fmaf(x, kLog2e, -lse2));
                    if constexpr (DELTA)
                        d_acc += p * pacc[mb][r];
                    else
                        pacc[mb][r] = p * (pacc[mb][r] - dlt);
                }
            if constexpr (DELTA) {
                j = jn;
                continue;
            }
            // dQ^T += K^T dS^T, with dS^T split into bf16 hi + lo parts: early causal rows
            // have |dS| of order 10, where one bf16 rounding alone costs ~1e-1 in dQ
            const int gi = lane & 15, hh = (lane >> 4) & 1;
#pragma unroll
            for (int kk = 0; kk < PK; kk++) {
                bf16x8 sf, sf_lo;
#pragma unroll
                for (int e = 0; e < 8; e++) {
                    const float x = pacc[kk >> 1][8 * (kk & 1) + e];
                    const __bf16 hi = (__bf16)x;
                    sf[e] = hi;
                    sf_lo[e] = (__bf16)(x - (float)hi);
                }
                const int r0 = 16 * kk + 4 * c + (gi >> 2);
                const int r1 = r0 + 8;
                const int sw0 = swz<CPR>(r0), sw1 = swz<CPR>(r1);
#pragma unroll
                for (int hb = 0; hb < HB; hb++) {
                    const int hcol = 32 * hb + 16 * hh + 4 * (gi & 3);
                    const int ch = hcol >> 3, within = hcol & 7;
                    const bf16x8 kt = join_bf16x8(lds_read_tr16(sk + r0 * H + ((ch ^ sw0) << 3) + within),
                                                  lds_read_tr16(sk + r1 * H + ((ch ^ sw1) << 3) + within));
                    dq_acc[hb] = mfma32x32x16(kt, sf, dq_acc[hb]);
                    dq_acc[hb] = mfma32x32x16(kt, sf_lo, dq_acc[hb]);
                }
            }
        }
        j = jn;
    }

    if constexpr (DELTA) {
        d_acc += __shfl_xor(d_acc, 32);
        if (q_valid && c == 0) {
            a.delta[row] = d_acc;
            a.lse2[row] = lse2;
        }
        return;
    }
    if (q_valid) {
        float *dqrow = a.dq + row * H;
#pragma unroll
        for (int hb = 0; hb < HB; hb++)
#pragma unroll
            for (int q4 = 0; q4 < 4; q4++)
                *(f32x4 *)(dqrow + 32 * hb + 8 * q4 + 4 * c) =
                    f32x4{dq_acc[hb][4 * q4], dq_acc[hb][4 * q4 + 1], dq_acc[hb][4 * q4 + 2], dq_acc[hb][4 * q4 + 3]};
    }
}

// ---------------------------------------------------------------------------
// D pass for dense shapes (no segments, no window, whole tiles; causal needs
// T = S and query blocks of BKV): the ping-pong scheme of the forward kernel.
// D[t] = sum_s P[t,s] dP[t,s] with P = exp(S - lse) and dP = dO V^T in fp32.
//
// 8 waves, 32 query rows each (the unit's gw heads x BKV queries). Waves 0-3
// (group A) and 4-7 (group B) alternate, B one phase behind A, with a
// workgroup barrier between phases:
//   M(i): S^T = K(i) Q^T and dP^T = V(i) dO^T (MFMA only)
//   V(i): P and the running sum of P * dP for tile i (VALU only)
// so each SIMD runs one wave's MFMAs beside the other wave's VALU work.
// K and V tiles share one row layout (both are A operands read by rows) and
// move through three LDS slots: tile i sits in slot i % 3. Group A loads the
// K tiles and group B the V tiles, each two tiles ahead during its V phase,
// into the slot that M(i-1) of both groups has finished reading; every wave
// waits for its own loads at the end of its next M phase, a barrier before
// any wave reads them.
//
// SEG (segment ids, S <= 8192): the tiles are those of the block's list
// (seg_tile_list); a tile whose ids and the wave's query ids are not all one
// value takes the element mask, and so does the list's last tile.
//
// HM (per-head masks): the block walks the union of its heads' tile ranges
// (hm_union) and each wave masks with its own head's sides and prefix.
template <int H, int BKV, bool CAUSAL, bool WIN = false, bool SEG = false, bool HM = false>
__global__ __launch_bounds__(512, 2) void attn_bwd_delta_pp_kernel(BwdArgs a, int gw, int bq, int n_gsplit,
                                                                   int n_qblocks) {
    static_assert(!(HM && (WIN || SEG)), "per-head masks alone");
    constexpr int NG = 4;  // waves per group
    constexpr int KSTEPS = H / 16;
    constexpr int MB = BKV / 32;
    constexpr int NX = MB * KSTEPS;
    constexpr int CPR = H / 8;
    constexpr int RS = CPR + 1;  // row stride in 16-byte chunks (conflict-free row reads)
    constexpr int BLOCKS = (BKV * RS + 63) / 64;
    constexpr int ELEMS = BLOCKS * 512;
    constexpr int NSLOT = 3;
    __shared__ __attribute__((aligned(1024))) __bf16 sk[NSLOT][ELEMS];
    __shared__ __attribute__((aligned(1024))) __bf16 sv[NSLOT][ELEMS];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave / NG, gwv = wave % NG;
    const int n = lane & 31, c = lane >> 5;

    // work unit (causal: heaviest query block first) and this lane's row
    const int units = a.B * a.K * n_gsplit;
    int qb = blockIdx.x / units;
    if (CAUSAL) qb = n_qblocks - 1 - qb;
    const int u = blockIdx.x % units;
    const int gs = u % n_gsplit;
    const int kh = (u / n_gsplit) % a.K;
    const int b = u / (n_gsplit * a.K);
    const int t0 = qb * bq;
    const int T = a.T, S = a.S;
    const int rho = wave * 32 + n;  // gw * bq == 256: every row belongs to the unit
    const int g = gs * gw + rho / bq;
    const int t = t0 + rho % bq;    // t < T: T is a whole number of query blocks
    const size_t bk = (size_t)b * a.K + kh;
    const size_t row = (bk * a.G + g) * (size_t)T + t;

    bf16x8 qf[KSTEPS], df[KSTEPS];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ks++) {
        qf[ks] = *(const bf16x8 *)(a.q + row * H + 16 * ks + 8 * c);
        df[ks] = *(const bf16x8 *)(a.dout + row * H + 16 * ks + 8 * c);
    }
    const float l = a.lse[row];
    const float lse2 = (l == -INFINITY) ? INFINITY : l * kLog2e;

    const buffer_rsrc krs = make_rsrc(a.k + bk * (size_t)S * H, S * H * 2);
    const buffer_rsrc vrs = make_rsrc(a.v + bk * (size_t)S * H, S * H * 2);
    // key tiles j0 .. j0 + n_t - 1: a left window (causal only, WIN) starts the
    // block at the tile holding its first query's first visible key
    const int WL = a.wl;
    // HM: the wave's head mask and the block's union of tile ranges
    HeadMask hw{kNoWindow, kNoWindow, 0};
    HmRange<BKV> hr{0, 0};
    const int t_w = t - n;  // the wave's first query
    if constexpr (HM) {
        hw = head_mask_of(a.head_mask, kh, a.G, __builtin_amdgcn_readfirstlane(g), T, S, a.causal, a.coff);
        hr = hm_union<BKV>(a, kh, gs * gw, gw, t0, bq);
    }
    const int j0 = HM ? hr.first : (WIN && t0 - WL > 0 ? (t0 - WL) / BKV : 0);
    // causal: the block's diagonal tile qb + coff / BKV comes last
    const int nt_all = HM ? hr.last + 1 : (CAUSAL ? qb + 1 + a.coff / BKV : S / BKV);
    // SEG: the block's list of tiles and the lane's and wave's query ids
    constexpr int KV_CAP = SEG ? kSegKeyCap : 1, NT_CAP = SEG ? kSegKeyCap / BKV : 1;
    __shared__ __attribute__((aligned(16))) int s_kvid[KV_CAP];
    __shared__ int s_tmin[NT_CAP], s_tmax[NT_CAP], s_jlist[NT_CAP], s_nvis;
    int my_qid = 0, w_qmin = 0, w_qmax = 0, n_vis = 0;
    if constexpr (SEG) {
        const int32_t *qs = a.q_seg + (size_t)b * T;
        my_qid = qs[t];
        w_qmin = wave_min_i(my_qid);
        w_qmax = wave_max_i(my_qid);
        n_vis = seg_tile_list<BKV>(qs, a.kv_seg + (size_t)b * S, t0, bq, T, nt_all, s_kvid, s_tmin, s_tmax, s_jlist,
                                   &s_nvis);
        if (n_vis == 0) {
            // no query of the block shares an id with a key it may see
            if (c == 0) {
                a.delta[row] = 0.f;
                a.lse2[row] = lse2;
            }
            return;
        }
    }
    const int n_t = SEG ? n_vis : nt_all - j0;
    auto tile_of = [&](int i) { return SEG ? __builtin_amdgcn_readfirstlane(s_jlist[i]) : j0 + i; };
    // SEG: tile j needs the element mask for this wave's rows
    auto seg_mask = [&](int j) {
        const int kmin = __builtin_amdgcn_readfirstlane(s_tmin[j]), kmax = __builtin_amdgcn_readfirstlane(s_tmax[j]);
        return !(w_qmin == w_qmax && kmin == kmax && kmin == w_qmin);
    };

    // global -> LDS: group A loads K tiles, group B V tiles; wave gwv of a group
    // issues 1 KiB blocks gwv, gwv + NG, ... (padding slots repeat the row's
    // last chunk)
    constexpr int NL = (BLOCKS + NG - 1) / NG;
    int ld_off[NL];
#pragma unroll
    for (int i = 0; i < NL; i++) {
        const int pslot = (gwv + i * NG) * 64 + lane;
        ld_off[i] = ((pslot / RS) * H + min(pslot % RS, CPR - 1) * 8) * 2;
    }
    // tiles j < n_t lie wholly inside K and V (S % BKV == 0), so the tile
    // offset may go in the scalar offset
    auto issue_tile = [&](int j, int slot) {
        const int tile = __builtin_amdgcn_readfirstlane(tile_of(j) * BKV * H * 2);
        __bf16 *dst = grp == 0 ? sk[slot] : sv[slot];
        const buffer_rsrc &rs = grp == 0 ? krs : vrs;
#pragma unroll
        for (int i = 0; i < NL; i++)
            if (gwv + i * NG < BLOCKS) lds_load16_to(rs, (char *)dst + (gwv + i * NG) * 1024, ld_off[i], tile);
    };

    f32x16 sacc[MB], pacc[MB];
    float d_acc = 0.f;
    const int a_lane = n * RS * 8 + c * 8;
    auto m_phase = [&](int slot) {
        const __bf16 *kt = sk[slot];
        const __bf16 *vt = sv[slot];
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int x = 0; x < NX; x++) {
            const int mb = x % MB, ks = x / MB;
            const int off = a_lane + mb * 32 * RS * 8 + ks * 16;
            const bf16x8 kf = *(const bf16x8 *)(kt + off);
            const bf16x8 vf = *(const bf16x8 *)(vt + off);
            sacc[mb] = mfma32x32x16(kf, qf[ks], ks == 0 ? f32x16{} : sacc[mb]);
            pacc[mb] = mfma32x32x16(vf, df[ks], ks == 0 ? f32x16{} : pacc[mb]);
        }
        constexpr int D = kBwdPrefetch < NX ? kBwdPrefetch : NX;
        pp_schedule<NX, 2, 2, D>(std::make_integer_sequence<int, D>(), std::make_integer_sequence<int, NX>());
        __builtin_amdgcn_s_setprio(0);
        wait_lds_loads();
    };
    // V phase: lane (n, c) holds keys s0 + 32 mb + acc_row(r, c) of query t
    auto v_phase = [&](int s0, auto masked) {
        // last and first visible key offsets (causal, window; HM: the head's)
        const int lim = HM ? t + hw.wr - s0 - 4 * c : CAUSAL ? t + a.coff - s0 - 4 * c : INT_MAX;
        const int first = HM ? t - hw.wl - s0 - 4 * c : WIN ? t - WL - s0 - 4 * c : INT_MIN;
#pragma unroll
        for (int mb = 0; mb < MB; mb++)
#pragma unroll
            for (int q4 = 0; q4 < 4; q4++) {
                // SEG: the ids of keys s0 + 32 mb + 8 q4 + 4 c + 0..3
                i32x4 ids{};
                if constexpr (SEG && decltype(masked)::value) ids = *(const i32x4 *)&s_kvid[s0 + 32 * mb + 8 * q4 + 4 * c];
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int r = 4 * q4 + e;
                    float p = exp2_fast(__builtin_fmaf(sacc[mb][r], kLog2e, -lse2));
                    if constexpr (decltype(masked)::value) {
                        const int off = 32 * mb + 8 * q4 + e;
                        bool hide = off > lim || off < first;
                        if constexpr (SEG) hide = hide || ids[e] != my_qid;
                        if constexpr (HM) hide = hide && s0 + off + 4 * c >= hw.pfx;  // prefix keys stay
                        if (hide) p = 0.f;
                    }
                    d_acc = __builtin_fmaf(p, pacc[mb][r], d_acc);
                }
            }
    };
    using yes = std::integral_constant<bool, true>;
    using no = std::integral_constant<bool, false>;

    // prologue: tiles 0 and 1 -> slots 0 and 1
    issue_tile(0, 0);
    if (n_t > 1) issue_tile(1, 1);
    wait_lds_loads();
    barrier_no_drain();
    if (grp == 1) barrier_no_drain();  // group B runs one phase behind
    m_phase(0);
    int slot = 0;  // slot of tile i
    for (int i = 0; i < n_t - 1; i++) {
        const int nslot = slot == NSLOT - 1 ? 0 : slot + 1;
        const int lslot = nslot == NSLOT - 1 ? 0 : nslot + 1;
        barrier_no_drain();
        if (i + 2 < n_t) issue_tile(i + 2, lslot);
        // WIN: the window's left edge, t - WL over the block's BKV queries,
        // cuts at most the block's first two tiles
        bool mk;
        if constexpr (SEG)
            mk = seg_mask(tile_of(i));
        else if constexpr (HM)
            mk = hm_tile_masked<BKV>(hw, j0 + i, t_w);
        else
            mk = WIN && i < 2 && (j0 + i) * BKV < t0 + BKV - 1 - WL;
        if (mk)
            v_phase(tile_of(i) * BKV, yes{});
        else
            v_phase(tile_of(i) * BKV, no{});
        barrier_no_drain();
        m_phase(nslot);
        slot = nslot;
    }
    barrier_no_drain();
    if (HM ? hm_tile_masked<BKV>(hw, j0 + n_t - 1, t_w) : (CAUSAL || SEG))
        v_phase(tile_of(n_t - 1) * BKV, yes{});
    else
        v_phase(tile_of(n_t - 1) * BKV, no{});
    if (grp == 0) barrier_no_drain();  // group A's trailing phase

    d_acc += __shfl_xor(d_acc, 32);
    if (c == 0) {
        a.delta[row] = d_acc;
        a.lse2[row] = lse2;
    }
}


// ---------------------------------------------------------------------------
// dQ for dense shapes (no segments, no window, whole 32-key tiles; causal
// needs T = S) on the forward's ping-pong scheme. 8 waves of 32 query rows
// (the unit's gw heads x bq queries); waves 0-3 (group A) and 4-7 (group B)
// run the same phases, B one phase behind A, with a workgroup barrier between
// phases. A wave alternates
//   M(i): S^T = K Q^T and dP^T = V dO^T of tile i+1, and dQ^T += K^T dS^T of
//         tile i from the bf16 hi part of dS, MFMAs only; then, when V(i)
//         found some |dS| above kDsLoMin, the lo part (K^T read again)
//   V(i): P = exp2(S log2e - lse log2e) and dS = P (dP - D) of tile i
// An M phase reads K and V of tile i+1 and K of tile i, so tiles rotate
// through four LDS slots (slot j % 4 holds K(j), V(j)). During V(i) group A
// loads K(i+2) and group B V(i+2) into slot (i+2) % 4, whose tile (i-2) was
// last read by M(i-2), over for both groups by then; the M phases running
// beside V(i) read slots i % 4 and (i +- 1) % 4. Each wave waits for its own
// loads at the end of its next M phase, one barrier before M(i+1) reads them.
// The K tile takes the dK/dV kernel's Q / dO layout: rows CPR + 4 chunks
// apart and one more chunk after every 4 rows, so that its b128 row reads and
// its transpose reads are both free of bank conflicts. V rows are padded to
// CPR + 1 chunks (row reads only).
//
// SEG (segment ids, S <= 8192): the tiles are those of the block's list
// (seg_tile_list); a tile whose ids and the wave's query ids are not all one
// value takes the element mask.
//
// HM (per-head masks): the block walks the union of its heads' tile ranges
// (hm_union) and each wave masks with its own head's sides and prefix.
template <int H, bool CAUSAL, bool WIN = false, bool SEG = false, bool HM = false>
__global__ __launch_bounds__(512, 2) void attn_bwd_dq_pp_kernel(BwdArgs a, int gw, int bq, int n_gsplit,
                                                                int n_qblocks) {
    static_assert(!(HM && (WIN || SEG)), "per-head masks alone");
    constexpr int BKV = 32;
    constexpr int NG = 4;            // waves per group
    constexpr int KSTEPS = H / 16;   // S and dP MFMAs per tile
    constexpr int HB = H / 32;
    constexpr int PK = BKV / 16;     // 16-key chunks of a tile
    static_assert(PK * HB == KSTEPS, "one dQ step per S / dP step");
    constexpr int CPR = H / 8;
    constexpr int KRS = CPR + 4, KGS = 4 * KRS + 1, VRS = CPR + 1;
    constexpr int KBLK = (BKV / 4 * KGS + 63) / 64, VBLK = (BKV * VRS + 63) / 64;
    constexpr int NL = ((KBLK > VBLK ? KBLK : VBLK) + NG - 1) / NG;
    constexpr int NSLOT = 4;
    __shared__ __attribute__((aligned(1024))) __bf16 sk[NSLOT][KBLK * 512];
    __shared__ __attribute__((aligned(1024))) __bf16 sv[NSLOT][VBLK * 512];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave / NG, gwv = wave % NG;
    const int n = lane & 31, c = lane >> 5;

    // work unit (causal: heaviest query block first) and this lane's row
    const int units = a.B * a.K * n_gsplit;
    int qb = blockIdx.x / units;
    if (CAUSAL) qb = n_qblocks - 1 - qb;
    const int u = blockIdx.x % units;
    const int gs = u % n_gsplit;
    const int kh = (u / n_gsplit) % a.K;
    const int b = u / (n_gsplit * a.K);
    const int t0 = qb * bq;
    const int T = a.T, S = a.S;
    const int rho = wave * 32 + n;  // gw * bq == 256: every row belongs to the unit
    const int g = gs * gw + rho / bq;
    const int t = t0 + rho % bq;    // t < T: T is a whole number of query blocks
    const int t_w = t - n;          // the wave's first query
    const size_t bk = (size_t)b * a.K + kh;
    const size_t row = (bk * a.G + g) * (size_t)T + t;

    bf16x8 qf[KSTEPS], df[KSTEPS];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ks++) {
        qf[ks] = *(const bf16x8 *)(a.q + row * H + 16 * ks + 8 * c);
        df[ks] = *(const bf16x8 *)(a.dout + row * H + 16 * ks + 8 * c);
    }
    const float l = a.lse[row];
    const float lse2 = (l == -INFINITY) ? INFINITY : l * kLog2e;
    const float dlt = a.delta[row];

    const buffer_rsrc krs = make_rsrc(a.k + bk * (size_t)S * H, S * H * 2);
    const buffer_rsrc vrs = make_rsrc(a.v + bk * (size_t)S * H, S * H * 2);
    // key tiles j0 .. j0 + n_t - 1: a left window (causal only, WIN) starts the
    // block at the tile holding its first query's first visible key
    const int WL = a.wl;
    // HM: the wave's head mask and the block's union of tile ranges
    HeadMask hw{kNoWindow, kNoWindow, 0};
    HmRange<BKV> hr{0, 0};
    if constexpr (HM) {
        hw = head_mask_of(a.head_mask, kh, a.G, __builtin_amdgcn_readfirstlane(g), T, S, a.causal, a.coff);
        hr = hm_union<BKV>(a, kh, gs * gw, gw, t0, bq);
    }
    const int j0 = HM ? hr.first : (WIN && t0 - WL > 0 ? (t0 - WL) / BKV : 0);
    // causal: up to the tile of the block's last query's diagonal
    const int nt_all = HM ? hr.last + 1 : (CAUSAL ? (t0 + bq + a.coff) / BKV : S / BKV);
    // SEG: the block's list of tiles and the lane's and wave's query ids
    constexpr int KV_CAP = SEG ? kSegKeyCap : 1, NT_CAP = SEG ? kSegKeyCap / BKV : 1;
    __shared__ __attribute__((aligned(16))) int s_kvid[KV_CAP];
    __shared__ int s_tmin[NT_CAP], s_tmax[NT_CAP], s_jlist[NT_CAP], s_nvis;
    int my_qid = 0, w_qmin = 0, w_qmax = 0, n_vis = 0;
    if constexpr (SEG) {
        const int32_t *qs = a.q_seg + (size_t)b * T;
        my_qid = qs[t];
        w_qmin = wave_min_i(my_qid);
        w_qmax = wave_max_i(my_qid);
        n_vis = seg_tile_list<BKV>(qs, a.kv_seg + (size_t)b * S, t0, bq, T, nt_all, s_kvid, s_tmin, s_tmax, s_jlist,
                                   &s_nvis);
        if (n_vis == 0) {
            // no query of the block shares an id with a key it may see: dQ = 0
            float *dqrow = a.dq + row * H;
#pragma unroll
            for (int hb = 0; hb < HB; hb++)
#pragma unroll
                for (int q4 = 0; q4 < 4; q4++) *(f32x4 *)(dqrow + 32 * hb + 8 * q4 + 4 * c) = f32x4{};
            return;
        }
    }
    const int n_t = SEG ? n_vis : nt_all - j0;
    auto tile_of = [&](int i) { return SEG ? __builtin_amdgcn_readfirstlane(s_jlist[i]) : j0 + i; };

    // global -> LDS: group A loads K tiles, group B V tiles; wave gwv of a group
    // issues 1 KiB blocks gwv, gwv + NG, ... Chunk p of a K tile holds row
    // 4 (p / KGS) + (p % KGS) / KRS; padding chunks repeat an in-range chunk,
    // as do slots past the last row
    const int nblk = grp == 0 ? KBLK : VBLK;
    int ld_off[NL];
#pragma unroll
    for (int i = 0; i < NL; i++) {
        const int pslot = (gwv + i * NG) * 64 + lane;
        if (grp == 0) {
            const int rem = pslot % KGS;
            const int row = min(4 * (pslot / KGS) + min(rem / KRS, 3), BKV - 1);
            ld_off[i] = (row * H + min(rem % KRS, CPR - 1) * 8) * 2;
        } else {
            ld_off[i] = (min(pslot / VRS, BKV - 1) * H + min(pslot % VRS, CPR - 1) * 8) * 2;
        }
    }
    // tiles j < n_t lie wholly inside K and V (S % BKV == 0), so the tile
    // offset may go in the scalar offset
    auto issue_tile = [&](int j, int slot) {
        const int tile = __builtin_amdgcn_readfirstlane(tile_of(j) * BKV * H * 2);
        char *dst = grp == 0 ? (char *)sk[slot] : (char *)sv[slot];
        const buffer_rsrc &rsrc = grp == 0 ? krs : vrs;
#pragma unroll
        for (int i = 0; i < NL; i++)
            if (gwv + i * NG < nblk) lds_load16_to(rsrc, dst + (gwv + i * NG) * 1024, ld_off[i], tile);
    };

    f32x16 sacc, pacc, dq_acc[HB];
#pragma unroll
    for (int hb = 0; hb < HB; hb++) dq_acc[hb] = f32x16{};
    bf16x8 dsh[PK], dsl[PK];
    const int k_lane = ((n >> 2) * KGS + (n & 3) * KRS) * 8 + c * 8, v_lane = n * VRS * 8 + c * 8;
    // transpose read of K^T: lane (gi, hh) of 16-lane group c addresses key
    // 16 kk + 4 c + gi / 4 (+ 8 for the upper half) at h = 32 hb + 16 hh + 4 (gi % 4)
    const int tr_lane = c * KGS * 8 + ((lane & 15) >> 2) * KRS * 8 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

    // M phase: S / dP of the tile in slot `cur` (SD) and dQ of the tile in
    // slot `prev` (DQ) from the hi part of dS, interleaved S, dQ, dP
    auto m_phase = [&](auto sd, auto dq, int cur, int prev) {
        const __bf16 *kc = sk[cur];
        const __bf16 *vc = sv[cur];
        const __bf16 *kp = sk[prev];
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int x = 0; x < KSTEPS; x++) {
            const int kk = x / HB, hb = x % HB;
            bf16x8 kt;
            if constexpr (decltype(dq)::value) {
                const __bf16 *p = kp + tr_lane + kk * 4 * KGS * 8 + hb * 32;
                kt = join_bf16x8(lds_read_tr16(p), lds_read_tr16(p + 2 * KGS * 8));
            }
            if constexpr (decltype(sd)::value) {
                const bf16x8 kf = *(const bf16x8 *)(kc + k_lane + x * 16);
                sacc = mfma32x32x16(kf, qf[x], x == 0 ? f32x16{} : sacc);
            }
            if constexpr (decltype(dq)::value) dq_acc[hb] = mfma32x32x16(kt, dsh[kk], dq_acc[hb]);
            if constexpr (decltype(sd)::value) {
                const bf16x8 vf = *(const bf16x8 *)(vc + v_lane + x * 16);
                pacc = mfma32x32x16(vf, df[x], x == 0 ? f32x16{} : pacc);
            }
        }
        constexpr bool SD = decltype(sd)::value, DQ = decltype(dq)::value;
        constexpr int NM = (SD ? 2 : 0) + (DQ ? 1 : 0);
        constexpr int NR = (SD ? 2 : 0) + (DQ ? 2 : 0);
        constexpr int D = kBwdPrefetch < KSTEPS ? kBwdPrefetch : KSTEPS;
        pp_schedule<KSTEPS, NM, NR, D>(std::make_integer_sequence<int, D>(), std::make_integer_sequence<int, KSTEPS>());
        __builtin_amdgcn_s_setprio(0);
        wait_lds_loads();
    };
    // the lo part of dS into dQ, for a tile whose V phase set need_lo: K^T of
    // the tile read again from slot `prev`, which no wave overwrites before
    // the next barrier
    auto lo_phase = [&](int prev) {
        const __bf16 *kp = sk[prev];
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int x = 0; x < KSTEPS; x++) {
            const int kk = x / HB, hb = x % HB;
            const __bf16 *p = kp + tr_lane + kk * 4 * KGS * 8 + hb * 32;
            const bf16x8 kt = join_bf16x8(lds_read_tr16(p), lds_read_tr16(p + 2 * KGS * 8));
            dq_acc[hb] = mfma32x32x16(kt, dsl[kk], dq_acc[hb]);
        }
        __builtin_amdgcn_s_setprio(0);
    };
    // V phase: lane (n, c) holds keys s0 + acc_row(r, c) of query t; dS as
    // bf16 hi + lo (early causal rows have |dS| of order 10, where one bf16
    // rounding alone costs ~1e-1 in dQ). need_lo (wave-uniform): some |dS| of
    // the wave's tile exceeds kDsLoMin, so its lo part goes into dQ
    bool need_lo = true;
    auto v_phase = [&](int s0) {
        // some key after some query of the wave, or (WIN) before some query's
        // first visible key t - WL; SEG: ids not all one value
        bool masked = HM ? hm_tile_masked<BKV>(hw, s0 / BKV, t_w)
                         : (CAUSAL && s0 + BKV - 1 > t_w + a.coff) || (WIN && s0 < t_w + 31 - WL);
        if constexpr (SEG) {
            const int j = s0 / BKV;
            const int kmin = __builtin_amdgcn_readfirstlane(s_tmin[j]);
            const int kmax = __builtin_amdgcn_readfirstlane(s_tmax[j]);
            masked = masked || !(w_qmin == w_qmax && kmin == kmax && kmin == w_qmin);
        }
        // last and first visible key offsets (causal, window; HM: the head's)
        const int lim = HM ? t + hw.wr - s0 - 4 * c : CAUSAL ? t + a.coff - s0 - 4 * c : INT_MAX;
        const int first = HM ? t - hw.wl - s0 - 4 * c : WIN ? t - WL - s0 - 4 * c : INT_MIN;
        float amax = 0.f;
        // SEG: the ids of keys s0 + 8 q4 + 4 c + 0..3 (read on masked tiles only)
        i32x4 ids[4] = {};
        if constexpr (SEG) {
            if (masked) {
#pragma unroll
                for (int q4 = 0; q4 < 4; q4++) ids[q4] = *(const i32x4 *)&s_kvid[s0 + 8 * q4 + 4 * c];
            }
        }
#pragma unroll
        for (int r = 0; r < 16; r++) {
            float p = exp2_fast(__builtin_fmaf(sacc[r], kLog2e, -lse2));
            const int off = 8 * (r >> 2) + (r & 3);
            bool hide = off > lim || off < first;
            if constexpr (SEG) hide = hide || ids[r >> 2][r & 3] != my_qid;
            if constexpr (HM) hide = hide && s0 + off + 4 * c >= hw.pfx;  // prefix keys stay
            if (masked && hide) p = 0.f;
            const float ds = p * (pacc[r] - dlt);
            amax = fmaxf(amax, fabsf(ds));
            const __bf16 hi = (__bf16)ds;
            dsh[r >> 3][r & 7] = hi;
            dsl[r >> 3][r & 7] = (__bf16)(ds - (float)hi);
        }
        need_lo = __builtin_amdgcn_ballot_w64(!(amax <= kDsLoMin)) != 0;
    };
    using yes = std::integral_constant<bool, true>;
    using no = std::integral_constant<bool, false>;

    // prologue: tiles 0 and 1 -> slots 0 and 1
    issue_tile(0, 0);
    if (n_t > 1) issue_tile(1, 1);
    wait_lds_loads();
    barrier_no_drain();
    if (grp == 1) barrier_no_drain();  // group B runs one phase behind
    m_phase(yes{}, no{}, 0, 0);  // M(-1): S / dP of tile 0
    for (int i = 0; i < n_t - 1; i++) {
        barrier_no_drain();
        if (i + 2 < n_t) issue_tile(i + 2, (i + 2) % NSLOT);
        v_phase(tile_of(i) * BKV);
        barrier_no_drain();
        m_phase(yes{}, yes{}, (i + 1) % NSLOT, i % NSLOT);
        if (need_lo) lo_phase(i % NSLOT);
    }
    barrier_no_drain();
    v_phase(tile_of(n_t - 1) * BKV);
    barrier_no_drain();
    m_phase(no{}, yes{}, 0, (n_t - 1) % NSLOT);
    if (need_lo) lo_phase((n_t - 1) % NSLOT);
    if (grp == 0) barrier_no_drain();  // group A's trailing phase

    // dQ row (fp32): lane (n, c) holds h = 32 hb + acc_row(r, c) of query t
    float *dqrow = a.dq + row * H;
#pragma unroll
    for (int hb = 0; hb < HB; hb++)
#pragma unroll
        for (int q4 = 0; q4 < 4; q4++)
            *(f32x4 *)(dqrow + 32 * hb + 8 * q4 + 4 * c) =
                f32x4{dq_acc[hb][4 * q4], dq_acc[hb][4 * q4 + 1], dq_acc[hb][4 * q4 + 2], dq_acc[hb][4 * q4 + 3]};
}

// ---------------------------------------------------------------------------
template <int H, int NW_DKV, int BKV_DQ, int NW_DQ>
static hipError_t launch_bwd_t(const BwdArgs &a, hipStream_t stream) {
    int gw = 1;
    for (int d = 1; d <= NW_DQ && d <= a.G; d++)
        if (a.G % d == 0) gw = d;
    const int bq = 32 * (NW_DQ / gw);
    const int n_gsplit = a.G / gw;
    const int n_qblocks = (a.T + bq - 1) / bq;
    const dim3 qgrid((unsigned)(a.B * a.K * n_gsplit * n_qblocks));
    // D = rowsum(P * dP), then dQ, then dK / dV (both read D). The D pass has
    // no dQ accumulators, so at H <= 128 it takes key tiles of 64 (half the
    // per-tile barriers and loop overhead of the dQ pass's 32).
    constexpr int BKV_D = H <= 128 ? 64 : BKV_DQ;
    bool delta_done = false;
    const MaskSpec m{a.causal, a.coff, a.wl, a.wr, a.prefix};
    // causal: the diagonal offset a whole number of tiles, T + coff == S
    auto diag_tiles = [&](int bkv) { return !a.causal || (a.coff >= 0 && a.coff % bkv == 0 && a.T + a.coff == a.S); };
    if constexpr (H <= 128 && NW_DQ == 8) {
        // dense shapes: the ping-pong D pass (query blocks of 64 rows x gw heads)
        constexpr int BKV_PP = 64;
        const bool shape = a.q_seg == nullptr && a.head_mask == nullptr && gw * bq == 256 && a.T % bq == 0 &&
                           a.S % BKV_PP == 0 && diag_tiles(BKV_PP) && (!a.causal || bq == BKV_PP);
        const bool dense = shape && !mask_extra(m);
        // a causal left window on an otherwise dense shape
        const bool dense_win = shape && mask_left_window_only(m);
        // segment ids on an otherwise dense shape with at most 8192 keys
        const bool seg_shape = a.q_seg != nullptr && a.head_mask == nullptr && gw * bq == 256 && a.T % bq == 0 &&
                               a.S % BKV_PP == 0 && a.S <= kSegKeyCap && diag_tiles(BKV_PP) &&
                               (!a.causal || bq == BKV_PP) && !mask_extra(m);
        // per-head masks on an otherwise dense shape
        const bool hm_shape = a.q_seg == nullptr && a.head_mask != nullptr && gw * bq == 256 && a.T % bq == 0 &&
                              a.S % BKV_PP == 0 && diag_tiles(BKV_PP) && (!a.causal || bq == BKV_PP) &&
                              !mask_extra(m);
        if (seg_shape) {
            if (a.causal)
                hipLaunchKernelGGL((attn_bwd_delta_pp_kernel<H, BKV_PP, true, false, true>), qgrid, dim3(512), 0,
                                   stream, a, gw, bq, n_gsplit, n_qblocks);
            else
                hipLaunchKernelGGL((attn_bwd_delta_pp_kernel<H, BKV_PP, false, false, true>), qgrid, dim3(512), 0,
                                   stream, a, gw, bq, n_gsplit, n_qblocks);
            delta_done = true;
        } else if (hm_shape) {
            if (a.causal)
                hipLaunchKernelGGL((attn_bwd_delta_pp_kernel<H, BKV_PP, true, false, false, true>), qgrid, dim3(512),
                                   0, stream, a, gw, bq, n_gsplit, n_qblocks);
            else
                hipLaunchKernelGGL((attn_bwd_delta_pp_kernel<H, BKV_PP, false, false, false, true>), qgrid, dim3(512),
                                   0, stream, a, gw, bq, n_gsplit, n_qblocks);
            delta_done = true;
        } else if (dense) {
            if (a.causal)
                hipLaunchKernelGGL((attn_bwd_delta_pp_kernel<H, BKV_PP, true>), qgrid, dim3(512), 0, stream, a, gw,
                                   bq, n_gsplit, n_qblocks);
            else
                hipLaunchKernelGGL((attn_bwd_delta_pp_kernel<H, BKV_PP, false>), qgrid, dim3(512), 0, stream, a, gw,
                                   bq, n_gsplit, n_qblocks);
            delta_done = true;
        } else if (dense_win) {
            hipLaunchKernelGGL((attn_bwd_delta_pp_kernel<H, BKV_PP, true, true>), qgrid, dim3(512), 0, stream, a, gw,
                               bq, n_gsplit, n_qblocks);
            delta_done = true;
        }
    }
    if (!delta_done)
        hipLaunchKernelGGL((attn_bwd_dq_kernel<H, BKV_D, NW_DQ, true>), qgrid, dim3(NW_DQ * 64), 0, stream, a, gw, bq,
                           n_gsplit, n_qblocks);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    bool dq_done = false;
    if constexpr (H <= 128 && NW_DQ == 8) {
        // dense shapes: dQ on the ping-pong kernel (32-key tiles)
        const bool shape = a.q_seg == nullptr && a.head_mask == nullptr && gw * bq == 256 && a.T % bq == 0 &&
                           a.S % 32 == 0 && diag_tiles(32);
        const bool dense = shape && !mask_extra(m);
        // a causal left window on an otherwise dense shape
        const bool dense_win = shape && mask_left_window_only(m);
        // segment ids on an otherwise dense shape with at most 8192 keys
        const bool seg_shape = a.q_seg != nullptr && a.head_mask == nullptr && gw * bq == 256 && a.T % bq == 0 &&
                               a.S % 32 == 0 && a.S <= kSegKeyCap && diag_tiles(32) && !mask_extra(m);
        // per-head masks on an otherwise dense shape
        const bool hm_shape = a.q_seg == nullptr && a.head_mask != nullptr && gw * bq == 256 && a.T % bq == 0 &&
                              a.S % 32 == 0 && diag_tiles(32) && !mask_extra(m);
        if (seg_shape) {
            if (a.causal)
                hipLaunchKernelGGL((attn_bwd_dq_pp_kernel<H, true, false, true>), qgrid, dim3(512), 0, stream, a, gw,
                                   bq, n_gsplit, n_qblocks);
            else
                hipLaunchKernelGGL((attn_bwd_dq_pp_kernel<H, false, false, true>), qgrid, dim3(512), 0, stream, a, gw,
                                   bq, n_gsplit, n_qblocks);
            dq_done = true;
        } else if (hm_shape) {
            if (a.causal)
                hipLaunchKernelGGL((attn_bwd_dq_pp_kernel<H, true, false, false, true>), qgrid, dim3(512), 0, stream,
                                   a, gw, bq, n_gsplit, n_qblocks);
            else
                hipLaunchKernelGGL((attn_bwd_dq_pp_kernel<H, false, false, false, true>), qgrid, dim3(512), 0, stream,
                                   a, gw, bq, n_gsplit, n_qblocks);
            dq_done = true;
        } else if (dense) {
            if (a.causal)
                hipLaunchKernelGGL((attn_bwd_dq_pp_kernel<H, true>), qgrid, dim3(512), 0, stream, a, gw, bq, n_gsplit,
                                   n_qblocks);
            else
                hipLaunchKernelGGL((attn_bwd_dq_pp_kernel<H, false>), qgrid, dim3(512), 0, stream, a, gw, bq, n_gsplit,
                                   n_qblocks);
            dq_done = true;
        } else if (dense_win) {
            hipLaunchKernelGGL((attn_bwd_dq_pp_kernel<H, true, true>), qgrid, dim3(512), 0, stream, a, gw, bq,
                               n_gsplit, n_qblocks);
            dq_done = true;
        }
    }
    if (!dq_done)
        hipLaunchKernelGGL((attn_bwd_dq_kernel<H, BKV_DQ, NW_DQ, false>), qgrid, dim3(NW_DQ * 64), 0, stream, a, gw, bq,
                           n_gsplit, n_qblocks);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int keys_wg = 32 * NW_DKV;
    const int n_kblocks = (a.S + keys_wg - 1) / keys_wg;
    const dim3 kgrid((unsigned)(a.B * a.K * n_kblocks));
    if constexpr (H <= 128 && NW_DKV == 4) {
        // no per-head masks: the wave-pair kernel (8 waves, 128 keys per
        // workgroup), with segment ids up to 8192 queries
        if (a.q_seg == nullptr && a.head_mask == nullptr) {
            if (a.causal)
                hipLaunchKernelGGL((attn_bwd_dkv3_kernel<H, true>), kgrid, dim3(512), 0, stream, a);
            else
                hipLaunchKernelGGL((attn_bwd_dkv3_kernel<H, false>), kgrid, dim3(512), 0, stream, a);
            return hipGetLastError();
        }
        if (a.q_seg != nullptr && a.head_mask == nullptr && a.T <= 8192) {
            if (a.causal)
                hipLaunchKernelGGL((attn_bwd_dkv3_kernel<H, true, true>), kgrid, dim3(512), 0, stream, a);
            else
                hipLaunchKernelGGL((attn_bwd_dkv3_kernel<H, false, true>), kgrid, dim3(512), 0, stream, a);
            return hipGetLastError();
        }
        // per-head masks without segment ids, up to 64 query heads per kv head
        if (a.q_seg == nullptr && a.head_mask != nullptr && a.G <= 64) {
            if (a.causal)
                hipLaunchKernelGGL((attn_bwd_dkv3_kernel<H, true, false, true>), kgrid, dim3(512), 0, stream, a);
            else
                hipLaunchKernelGGL((attn_bwd_dkv3_kernel<H, false, false, true>), kgrid, dim3(512), 0, stream, a);
            return hipGetLastError();
        }
    }
    if constexpr (H > 128) {
        // one pass for dV, one for dK (the two accumulators do not fit one wave together)
        hipLaunchKernelGGL((attn_bwd_dkv_kernel<H, NW_DKV, 1>), kgrid, dim3(NW_DKV * 64), 0, stream, a, n_kblocks);
        hipError_t e2 = hipGetLastError();
        if (e2 != hipSuccess) return e2;
        hipLaunchKernelGGL((attn_bwd_dkv_kernel<H, NW_DKV, 2>), kgrid, dim3(NW_DKV * 64), 0, stream, a, n_kblocks);
    } else {
        hipLaunchKernelGGL((attn_bwd_dkv_kernel<H, NW_DKV, 0>), kgrid, dim3(NW_DKV * 64), 0, stream, a, n_kblocks);
    }
    return hipGetLastError();
}

hipError_t launch_bwd(const BwdArgs &a, int H, hipStream_t stream) {
    switch (H) {
        case 64: return launch_bwd_t<64, 4, 64, 8>(a, stream);
        case 128: return launch_bwd_t<128, 4, 32, 8>(a, stream);
        case 256: return launch_bwd_t<256, 4, 32, 4>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gqa
