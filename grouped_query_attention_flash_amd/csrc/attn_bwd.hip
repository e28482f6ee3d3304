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
// dQ product as a bf16 hi + lo pair. Gradients are written in fp32. The G-sum of dK/dV stays inside one workgroup: no atomics, and the
// result is deterministic.
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

// pipelined dK/dV kernel for shapes without segment ids at H <= 128
#ifndef GQA_BWD_DKV2
#define GQA_BWD_DKV2 1
#endif
// its operand reads are issued this many MFMAs ahead of their use
#ifndef GQA_BWD_DELTA_PP
#define GQA_BWD_DELTA_PP 1
#endif
// dense shapes at H <= 128 run dQ on the ping-pong kernel
#ifndef GQA_BWD_DQ_PP
#define GQA_BWD_DQ_PP 1
#endif
// its M phase issues the LDS operand reads of a step this many steps ahead
// (0: no pinned schedule)
#ifndef GQA_BWD_DQ_PREF
#define GQA_BWD_DQ_PREF 2
#endif
// the same for the ping-pong D pass
#ifndef GQA_BWD_D_PREF
#define GQA_BWD_D_PREF 2
#endif
#ifndef GQA_BWD_D_BKV
#define GQA_BWD_D_BKV 64
#endif
#ifndef GQA_BWD_DKV_PREF
#define GQA_BWD_DKV_PREF 6
#endif
// its bf16 weight conversions pinned into their slots
#ifndef GQA_BWD_CVTPIN
#define GQA_BWD_CVTPIN 0
#endif
// its lse / D reads at the end of the iteration before (1) or at the top (0)
#ifndef GQA_BWD_LDPRE
#define GQA_BWD_LDPRE 1
#endif

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
template <int H, int NW>
__global__ __launch_bounds__(NW * 64) void attn_bwd_dkv_kernel(BwdArgs a, int n_kblocks) {
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

    // K^T and V^T operands (B operands): lane (n, c), k-step ks holds row s, h = 16ks + 8c .. +7
    bf16x8 kf[KSTEPS], vf[KSTEPS];
    {
        const __bf16 *krow = a.k + (bk * S + s) * H;
        const __bf16 *vrow = a.v + (bk * S + s) * H;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ks++) {
            kf[ks] = k_valid ? *(const bf16x8 *)(krow + 16 * ks + 8 * c) : bf16x8{};
            vf[ks] = k_valid ? *(const bf16x8 *)(vrow + 16 * ks + 8 * c) : bf16x8{};
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
    // band sides L, R, or every query for a block that starts in the prefix
    const int WL = a.wl, WR = a.wr, PFX = a.prefix;
    const int n_qt_all = (T + BQ - 1) / BQ;
    const bool blk_pfx = s0_wg < PFX;
    const int qt_begin = blk_pfx ? 0 : min(n_qt_all, max(0, s0_wg - WR) / BQ);
    const int n_qt = blk_pfx ? n_qt_all
                             : max(qt_begin, min(n_qt_all, (s0_wg + 32 * NW - 1 + WL) / BQ + 1));  // end of the tile range
    const int n_steps = G * (n_qt - qt_begin);  // (g, query tile) pairs, g outer

    auto q_ids = [&](int qt, int &qmin, int &qmax) {
        const int t = qt * BQ + lane;
        const bool ok = lane < BQ && t < T;
        const int id = ok ? qsb[t] : 0;
        qmin = wave_min_i(ok ? id : INT_MAX);
        qmax = wave_max_i(ok ? id : INT_MIN);
    };
    auto next_step = [&](int st) {
        if (!segs) return st;
        for (; st < n_steps; st++) {
            int qmin, qmax;
            q_ids(qt_begin + st % (n_qt - qt_begin), qmin, qmax);
            if (!(qmax < wg_kmin || qmin > wg_kmax)) break;
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
                    pacc = mfma32x32x16(*(const bf16x8 *)(drow + off), vf[ks], pacc);
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
                    pacc[r] = p * (pacc[r] - d4[e]);
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
                    const bf16x8 dot = join_bf16x8(lds_read_tr16(sdo + o0), lds_read_tr16(sdo + o1));
                    dv_acc[hb] = mfma32x32x16(dot, pf, dv_acc[hb]);
                    const bf16x8 qt = join_bf16x8(lds_read_tr16(sq + o0), lds_read_tr16(sq + o1));
                    dk_acc[hb] = mfma32x32x16(qt, sf, dk_acc[hb]);
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
                *(f32x4 *)(dkrow + h) = f32x4{dk_acc[hb][4 * q4], dk_acc[hb][4 * q4 + 1], dk_acc[hb][4 * q4 + 2],
                                              dk_acc[hb][4 * q4 + 3]};
                *(f32x4 *)(dvrow + h) = f32x4{dv_acc[hb][4 * q4], dv_acc[hb][4 * q4 + 1], dv_acc[hb][4 * q4 + 2],
                                              dv_acc[hb][4 * q4 + 3]};
            }
    }
    (void)n_kblocks;
}

// ---------------------------------------------------------------------------
// dK, dV for shapes without segment ids at H <= 128: the same products as the
// kernel above, software-pipelined three steps deep. Q, dO, lse and D of each
// 32-query step go straight from memory into a four-stage LDS ring (no
// register staging); iteration i runs the S and dP MFMAs of step i+2 and the
// dV and dK MFMAs of step i, and computes the weights of step i+1 (whose S and
// dP came from the previous iteration) between them, so the VALU work never
// waits on the MFMAs of its own iteration. One wave per SIMD (up to 512
// registers): the overlap is inside the wave.
//
// The loads write 1 KiB per wave instruction lane-linearly into padded-row
// tiles, each lane fetching the global chunk that belongs in its slot.
template <int H, bool CAUSAL>
__global__ __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, 1))) void attn_bwd_dkv2_kernel(BwdArgs a, int n_kblocks) {
    constexpr int NW = 4, BQ = 32;
    constexpr int CPR = H / 8;
    constexpr int KSTEPS = H / 16;
    constexpr int HB = H / 32;
    // Q / dO tiles in LDS: 32 rows of RS = CPR + 3 16-byte chunks (padded rows:
    // the b128 row reads are conflict-free and the transpose reads 2-way), so
    // that every operand address is a per-lane base plus an immediate
    constexpr int RS = CPR + 3;
    constexpr int TBLK = (BQ * RS + 63) / 64;     // 1 KiB wave loads per tile
    constexpr int TILE = TBLK * 512;              // bf16 elements per tile buffer
    constexpr int TBW = (TBLK + NW - 1) / NW;     // per wave and tensor
    constexpr int NLD = 2 * TBW + 1;              // loads per wave and step (Q, dO blocks; lse or D)
    constexpr int NSTAGE = 5;
    __shared__ __attribute__((aligned(1024))) __bf16 sq[NSTAGE][TILE];
    __shared__ __attribute__((aligned(1024))) __bf16 sdo[NSTAGE][TILE];
    __shared__ __attribute__((aligned(1024))) float sld[NSTAGE][2][256];  // lse, D (32 used)
    // destination of the loads a wave issues only to keep its count per step
    // the same as the other waves' (out of range: they read nothing)
    __shared__ __attribute__((aligned(1024))) char sdummy[1024];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31, c = lane >> 5;
    const int T = a.T, S = a.S, G = a.G;

    const int units = a.B * a.K;
    const int kb_idx = blockIdx.x / units;  // heaviest (causal) key block first
    const int u = blockIdx.x % units;
    const int kh = u % a.K, b = u / a.K;
    const int s0_wg = kb_idx * 32 * NW;
    const int s_w = s0_wg + 32 * wave;
    const int s = s_w + n;
    const bool k_valid = s < S;
    const size_t bk = (size_t)b * a.K + kh;

    bf16x8 kf[KSTEPS], vf[KSTEPS];
    {
        const __bf16 *krow = a.k + (bk * S + s) * H;
        const __bf16 *vrow = a.v + (bk * S + s) * H;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ks++) {
            kf[ks] = k_valid ? *(const bf16x8 *)(krow + 16 * ks + 8 * c) : bf16x8{};
            vf[ks] = k_valid ? *(const bf16x8 *)(vrow + 16 * ks + 8 * c) : bf16x8{};
        }
    }

    // steps: (g, query tile) pairs, g outer; causal: tiles holding some t >= s0_wg
    // query tiles that can see the block's keys: t in [s - R, s + L] for the
    // band sides L, R, or all of them for a block that starts in the prefix;
    // qt_end is exclusive
    const int WL = a.wl, WR = a.wr;
    const int n_qt = (T + BQ - 1) / BQ;
    const bool blk_pfx = s0_wg < a.prefix;
    const int qt_begin = blk_pfx ? 0 : min(n_qt, max(0, s0_wg - WR) / BQ);
    const int qt_end = blk_pfx ? n_qt : max(qt_begin, min(n_qt, (s0_wg + 32 * NW - 1 + WL) / BQ + 1));
    const int nq = qt_end - qt_begin;
    const int n_steps = G * nq;

    // loads of one step: Q and dO tiles (wave w: blocks w, w + NW, ...), lse
    // (wave 0), D (wave 1). Every wave issues NLD loads per step, without
    // branches: a block past the tile, the lse / D load of waves 2 and 3, and
    // every load of a step past the last one get an out-of-range offset and
    // the dummy destination.
    const i32x4 qrs = make_rsrc_words(a.q + bk * G * (size_t)T * H, G * T * H * 2);
    const i32x4 drs = make_rsrc_words(a.dout + bk * G * (size_t)T * H, G * T * H * 2);
    const i32x4 ldrs = wave == 0 ? make_rsrc_words(a.lse + bk * G * (size_t)T, G * T * 4)
                                 : make_rsrc_words(a.delta + bk * G * (size_t)T, G * T * 4);
    constexpr unsigned kOutOfRange = 0x80000000u;
    // slot p of a tile holds chunk min(p % RS, CPR - 1) of row p / RS (the
    // padding slots repeat the row's last chunk; rows past 31 are not read)
    int t_off[TBW];
#pragma unroll
    for (int i = 0; i < TBW; i++) {
        const int p = (wave + i * NW) * 64 + lane;
        t_off[i] = ((p / RS) * H + min(p % RS, CPR - 1) * 8) * 2;
    }
    const unsigned q_dst0 = lds_addr(sq[0]) + wave * 1024, d_dst0 = lds_addr(sdo[0]) + wave * 1024;
    const unsigned ld_dst0 = lds_addr(sld[0][wave & 1]), dummy = lds_addr(sdummy);
    // load j (< NLD) of a step whose query rows start at row0 (g T + t0), or
    // of no step (row0 < 0), into a stage
    auto issue_load = [&](int j, int row0, int stage) {
        if (j < 2 * TBW) {
            const int i = j >> 1;
            const bool ok = row0 >= 0 && wave + i * NW < TBLK;
            const unsigned voff = ok ? (unsigned)(row0 * H * 2 + t_off[i]) : kOutOfRange;
            const unsigned dst = ok ? ((j & 1) ? d_dst0 : q_dst0) + stage * (TILE * 2) + i * NW * 1024 : dummy;
            lds_dma16((j & 1) ? drs : qrs, __builtin_amdgcn_readfirstlane(dst), voff);
        } else {
            // 32 floats of lse / D: lanes 0-7 fetch them, the other lanes repeat
            // in-range addresses into slots that are not read
            const bool ok = row0 >= 0 && wave < 2;
            const unsigned voff = ok ? (unsigned)(row0 * 4 + (lane & 7) * 16) : kOutOfRange;
            const unsigned dst = ok ? ld_dst0 + stage * (2 * 256 * 4) : dummy;
            lds_dma16(ldrs, __builtin_amdgcn_readfirstlane(dst), voff);
        }
    };
    // steps walk (g, query tile) with g outer; a cursor gives a step's first
    // query row (g T + t0), or -1 past the last step
    struct Cursor {
        int g, qt;
    };
    auto advance = [&](Cursor &cu) {
        if (++cu.qt == qt_end) {
            cu.qt = qt_begin;
            ++cu.g;
        }
    };
    auto row_of = [&](const Cursor &cu) { return cu.g < G ? cu.g * T + cu.qt * BQ : -1; };
    auto issue_step = [&](int row0, int stage) {
#pragma unroll
        for (int j = 0; j < NLD; j++) issue_load(j, row0, stage);
    };

    f32x16 dv_acc[HB], dk_acc[HB];
#pragma unroll
    for (int hb = 0; hb < HB; hb++) {
        dv_acc[hb] = f32x16{};
        dk_acc[hb] = f32x16{};
    }

    // S = Q K^T and dP = dO V^T of a step (32 queries x the wave's 32 keys)
    const int row_lane = n * RS * 8 + c * 8;  // row n, chunk c
    auto sdp = [&](int stage, f32x16 &sacc, f32x16 &pacc) {
        const __bf16 *qrow = sq[stage] + row_lane;
        const __bf16 *drow = sdo[stage] + row_lane;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ks++) {
            sacc = mfma32x32x16(*(const bf16x8 *)(qrow + 16 * ks), kf[ks], ks == 0 ? f32x16{} : sacc);
            pacc = mfma32x32x16(*(const bf16x8 *)(drow + 16 * ks), vf[ks], ks == 0 ? f32x16{} : pacc);
        }
    };
    // P = exp2(S log2e - lse log2e) and dS = P (dP - D), as bf16 MFMA operands
    // (2 x 8 queries each). Invisible (query, key) pairs get P = 0. A pair is
    // visible iff u = t - s + R lies in [0, min(L + R + 1, T - s + R)), which
    // covers the window, causal masking (R = 0) and t < T with one unsigned
    // compare per element. The bound is clamped at 0: a key that no query can
    // see (past S, or past T - 1 + R) gets bound 0. A prefix key is visible to
    // every query: its lane takes unbounded sides (LL = RR = kNoWindow), so
    // only t < T remains.
    const bool k_pfx = s < a.prefix;
    const int LL = k_pfx ? kNoWindow : WL, RR = k_pfx ? kNoWindow : WR;
    const unsigned vis_bound = k_valid ? (unsigned)max(0, min(LL + RR + 1, T - s + RR)) : 0u;
    // lse and D of the lane's 16 query rows of a step
    auto read_ld = [&](int stage, f32x4 (&l4s)[4], f32x4 (&d4s)[4]) {
#pragma unroll
        for (int q4 = 0; q4 < 4; q4++) {
            l4s[q4] = *(const f32x4 *)(&sld[stage][0][8 * q4 + 4 * c]);
            d4s[q4] = *(const f32x4 *)(&sld[stage][1][8 * q4 + 4 * c]);
        }
    };
    auto weights = [&](int t0, const f32x4 (&l4s)[4], const f32x4 (&d4s)[4], const f32x16 &sacc, const f32x16 &pacc,
                       bf16x8 (&pf)[2], bf16x8 (&sf)[2]) {
        const int tb = t0 + 4 * c - s + RR;
#pragma unroll
        for (int q4 = 0; q4 < 4; q4++) {
            const f32x4 l4 = l4s[q4];
            const f32x4 d4 = d4s[q4];
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int r = 4 * q4 + e;
                float p = exp2_fast(__builtin_fmaf(sacc[r], kLog2e, -l4[e] * kLog2e));
                p = (unsigned)(tb + 8 * q4 + e) < vis_bound ? p : 0.f;
                pf[r >> 3][r & 7] = (__bf16)p;
                sf[r >> 3][r & 7] = (__bf16)(p * (pacc[r] - d4[e]));
            }
        }
    };
    // dV^T += dO^T P and dK^T += Q^T dS for a step (k = the step's 32 queries):
    // A operands by transpose reads. Lane (gi, hh) of 16-lane group c addresses
    // query row 16 kk + 4 c + gi / 4 (+ 8 for the upper half) at
    // h = 32 hb + 16 hh + 4 (gi % 4)
    const int gi = lane & 15, hh = (lane >> 4) & 1;
    const int tr_lane = (4 * c + (gi >> 2)) * RS * 8 + 16 * hh + 4 * (gi & 3);
    if (n_steps > 0) {
        // prologue: steps 0 .. 3 into stages 0 .. 3; P and dS of step 0, S and
        // dP of step 1
        Cursor c_ld{0, qt_begin};  // the next step to load
#pragma unroll
        for (int st = 0; st < 4; st++) {
            issue_step(row_of(c_ld), st);
            advance(c_ld);
        }
        wait_lds_loads();
        __syncthreads();
        f32x16 sa, pa;          // S, dP of step i+1 at the top of iteration i
        bf16x8 pfa[2], sfa[2];  // P, dS of step i
        {
            f32x16 s0, p0;
            sdp(0, s0, p0);
            f32x4 l4s[4], d4s[4];
            read_ld(0, l4s, d4s);
            weights(qt_begin * BQ, l4s, d4s, s0, p0, pfa, sfa);
            sdp(1, sa, pa);
        }
        Cursor c_w{0, qt_begin};  // step i+1 in iteration i (its weights)
        advance(c_w);
        // Iteration i: dV / dK of step i (stage i % 5), the weights of step i+1
        // (S and dP from the previous iteration, lse and D from stage
        // (i+1) % 5) and S / dP of step i+2 (stage (i+2) % 5). Step i+4 is
        // loaded into stage (i+4) % 5, which held step i-1, and must land by the
        // end of iteration i+1; steps past the last load nothing. The products
        // of steps past the last are never used.
        //
        // Explicit schedule in NSLOT fenced slots: slot m issues MFMA m and the
        // operand reads of MFMA m + PREF; slots 0 .. NQ - 1 are the S / dP
        // MFMAs, the rest the dV / dK MFMAs; every WSTRIDE-th slot also computes
        // one weight (P and dS) of step i+1, so the VALU work runs beside the
        // MFMAs, and every LSTRIDE-th slot issues one of the NLD loads of step
        // i+4. The lse and D of an iteration are read at the end of the one
        // before (their stage is complete by then).
        constexpr int NQ = 2 * KSTEPS, NSLOT = NQ + 4 * HB, PREF = GQA_BWD_DKV_PREF;
        constexpr int WSTRIDE = NSLOT / 16;  // slots per weight
        static_assert(WSTRIDE * 16 == NSLOT, "16 weights per lane and step");
        constexpr int LSTRIDE = NSLOT / NLD;
        static_assert(LSTRIDE >= 1, "a slot per load");
        int st0 = 0, st1 = 1, st2 = 2, st4 = 4;  // stages of steps i, i+1, i+2, i+4
        f32x4 l4s[4], d4s[4];
#if GQA_BWD_LDPRE
        read_ld(st1, l4s, d4s);
#endif
        for (int i = 0; i < n_steps; i++) {
            barrier_no_drain();
#if !GQA_BWD_LDPRE
            read_ld(st1, l4s, d4s);
#endif
            const int row_ld = row_of(c_ld);
            advance(c_ld);
            const int tb = c_w.qt * BQ + 4 * c - s + RR;
            advance(c_w);
            auto read_op = [&](int m) -> bf16x8 {
                if (m < NQ) {
                    const __bf16 *base = (m & 1) ? sdo[st2] : sq[st2];
                    return *(const bf16x8 *)(base + row_lane + 16 * (m >> 1));
                }
                const int j = m - NQ, kk = j / (2 * HB), hb = (j >> 1) % HB;
                const __bf16 *base = ((j & 1) ? sq[st0] : sdo[st0]) + tr_lane + 16 * kk * RS * 8 + 32 * hb;
                return join_bf16x8(lds_read_tr16(base), lds_read_tr16(base + 8 * RS * 8));
            };
            bf16x8 op[NSLOT];
#pragma unroll
            for (int m = 0; m < PREF; m++) op[m] = read_op(m);
            sched_fence();
            f32x16 sb, pb;
            bf16x8 pfb[2], sfb[2];
            float p_even = 0.f, ds_even = 0.f;
#pragma unroll
            for (int m = 0; m < NSLOT; m++) {
                if (m + PREF < NSLOT) op[m + PREF] = read_op(m + PREF);
                if (m < NQ) {
                    const int ks = m >> 1;
                    if (m & 1)
                        pb = mfma32x32x16(op[m], vf[ks], ks == 0 ? f32x16{} : pb);
                    else
                        sb = mfma32x32x16(op[m], kf[ks], ks == 0 ? f32x16{} : sb);
                } else {
                    const int j = m - NQ, kk = j / (2 * HB), hb = (j >> 1) % HB;
                    if (j & 1)
                        dk_acc[hb] = mfma32x32x16(op[m], sfa[kk], dk_acc[hb]);
                    else
                        dv_acc[hb] = mfma32x32x16(op[m], pfa[kk], dv_acc[hb]);
                }
                if (m % WSTRIDE == WSTRIDE - 1) {
                    // weight r of step i+1: row 8 (r / 4) + 4 c + r % 4 of its tile
                    const int r = m / WSTRIDE, q4 = r >> 2, e = r & 3;
                    float p = exp2_fast(__builtin_fmaf(sa[r], kLog2e, -l4s[q4][e] * kLog2e));
                    p = (unsigned)(tb + 8 * q4 + e) < vis_bound ? p : 0.f;
                    const float ds = p * (pa[r] - d4s[q4][e]);
                    if (r & 1) {
                        pfb[r >> 3][(r & 7) - 1] = (__bf16)p_even;
                        pfb[r >> 3][r & 7] = (__bf16)p;
                        sfb[r >> 3][(r & 7) - 1] = (__bf16)ds_even;
                        sfb[r >> 3][r & 7] = (__bf16)ds;
#if GQA_BWD_CVTPIN
                        // convert in this slot (the compiler would leave all
                        // conversions to the end of the iteration)
                        if ((r & 7) == 7 || GQA_BWD_CVTPIN > 1) {
                            pin_value(pfb[r >> 3]);
                            pin_value(sfb[r >> 3]);
                        }
#endif
                    } else {
                        p_even = p;
                        ds_even = ds;
                    }
                }
                if (m % LSTRIDE == LSTRIDE / 2 && m / LSTRIDE < NLD) issue_load(m / LSTRIDE, row_ld, st4);
                sched_fence();
            }
            pfa[0] = pfb[0];
            pfa[1] = pfb[1];
            sfa[0] = sfb[0];
            sfa[1] = sfb[1];
            sa = sb;
            pa = pb;
            // the loads of step i+3 (issued in the previous iteration) land
            // before the next barrier; this iteration's NLD stay in flight
            wait_lds_loads_but<NLD>();
            st0 = st1;
            st1 = st2;
            st2 = st2 == NSTAGE - 1 ? 0 : st2 + 1;
            st4 = st4 == NSTAGE - 1 ? 0 : st4 + 1;
#if GQA_BWD_LDPRE
            // the next iteration's lse / D (step i+2: landed before this
            // iteration's barrier)
            read_ld(st1, l4s, d4s);
#endif
        }
        // the last iteration's loads (of no step: out of range) complete
        // before the workgroup's LDS is released
        wait_lds_loads();
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
                *(f32x4 *)(dkrow + h) = f32x4{dk_acc[hb][4 * q4], dk_acc[hb][4 * q4 + 1], dk_acc[hb][4 * q4 + 2],
                                              dk_acc[hb][4 * q4 + 3]};
                *(f32x4 *)(dvrow + h) = f32x4{dv_acc[hb][4 * q4], dv_acc[hb][4 * q4 + 1], dv_acc[hb][4 * q4 + 2],
                                              dv_acc[hb][4 * q4 + 3]};
            }
    }
    (void)n_kblocks;
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

    // key tiles: the band of the block's first and last query, and the
    // prefix keys s < PFX
    const int WL = a.wl, WR = a.wr, PFX = a.prefix;
    const int n_tiles = (S + BKV - 1) / BKV;
    const int t_last = min(t0 + bq, T) - 1;
    const int s_last = max(min(t_last + WR, S - 1), PFX - 1);
    const int j_end = s_last < 0 ? 0 : min(n_tiles, s_last / BKV + 1);
    const int j_begin = (PFX > 0 || t0 - WL <= 0) ? 0 : (t0 - WL) / BKV;

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
        if (!segs && PFX == 0) return j;
        for (; j < j_end; j++) {
            const int s0 = j * BKV;
            if (!(s0 < PFX || (s0 + BKV - 1 >= t0 - WL && s0 <= t_last + WR))) continue;
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
        if (q_valid && c == 0) a.delta[row] = d_acc;
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
template <int H, int BKV, bool CAUSAL, bool WIN = false>
__global__ __launch_bounds__(512, 2) void attn_bwd_delta_pp_kernel(BwdArgs a, int gw, int bq, int n_gsplit,
                                                                   int n_qblocks) {
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
    const int j0 = WIN && t0 - WL > 0 ? (t0 - WL) / BKV : 0;
    // causal: the block's diagonal tile qb + coff / BKV comes last
    const int n_t = (CAUSAL ? qb + 1 + a.coff / BKV : S / BKV) - j0;

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
        const int tile = __builtin_amdgcn_readfirstlane((j0 + j) * BKV * H * 2);
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
#if GQA_BWD_D_PREF > 0
        constexpr int D = GQA_BWD_D_PREF < NX ? GQA_BWD_D_PREF : NX;
        pp_schedule<NX, 2, 2, D>(std::make_integer_sequence<int, D>(), std::make_integer_sequence<int, NX>());
#endif
        __builtin_amdgcn_s_setprio(0);
        wait_lds_loads();
    };
    // V phase: lane (n, c) holds keys s0 + 32 mb + acc_row(r, c) of query t
    auto v_phase = [&](int s0, auto masked) {
        const int lim = t + a.coff - s0 - 4 * c;                // last visible key offset (causal)
        const int first = WIN ? t - WL - s0 - 4 * c : INT_MIN;  // first visible key offset (window)
#pragma unroll
        for (int mb = 0; mb < MB; mb++)
#pragma unroll
            for (int r = 0; r < 16; r++) {
                float p = exp2_fast(__builtin_fmaf(sacc[mb][r], kLog2e, -lse2));
                if constexpr (decltype(masked)::value) {
                    const int off = 32 * mb + 8 * (r >> 2) + (r & 3);
                    if (off > lim || off < first) p = 0.f;
                }
                d_acc = __builtin_fmaf(p, pacc[mb][r], d_acc);
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
        if (WIN && i < 2 && (j0 + i) * BKV < t0 + BKV - 1 - WL)
            v_phase((j0 + i) * BKV, yes{});
        else
            v_phase((j0 + i) * BKV, no{});
        barrier_no_drain();
        m_phase(nslot);
        slot = nslot;
    }
    barrier_no_drain();
    if (CAUSAL)
        v_phase((j0 + n_t - 1) * BKV, yes{});
    else
        v_phase((j0 + n_t - 1) * BKV, no{});
    if (grp == 0) barrier_no_drain();  // group A's trailing phase

    d_acc += __shfl_xor(d_acc, 32);
    if (c == 0) a.delta[row] = d_acc;
}


// ---------------------------------------------------------------------------
// dQ for dense shapes (no segments, no window, whole 32-key tiles; causal
// needs T = S) on the forward's ping-pong scheme. 8 waves of 32 query rows
// (the unit's gw heads x bq queries); waves 0-3 (group A) and 4-7 (group B)
// run the same phases, B one phase behind A, with a workgroup barrier between
// phases. A wave alternates
//   M(i): S^T = K Q^T and dP^T = V dO^T of tile i+1, and dQ^T += K^T dS^T of
//         tile i (dS as bf16 hi + lo parts, one MFMA each), MFMAs only
//   V(i): P = exp2(S log2e - lse log2e) and dS = P (dP - D) of tile i
// An M phase reads K and V of tile i+1 and K of tile i, so tiles rotate
// through four LDS slots (slot j % 4 holds K(j), V(j)). During V(i) group A
// loads K(i+2) and group B V(i+2) into slot (i+2) % 4, whose tile (i-2) was
// last read by M(i-2), over for both groups by then; the M phases running
// beside V(i) read slots i % 4 and (i +- 1) % 4. Each wave waits for its own
// loads at the end of its next M phase, one barrier before M(i+1) reads them.
// K rows are padded to CPR + 3 chunks (its b128 row reads conflict-free and
// its transpose reads 2-way), V rows to CPR + 1.
template <int H, bool CAUSAL, bool WIN = false>
__global__ __launch_bounds__(512, 2) void attn_bwd_dq_pp_kernel(BwdArgs a, int gw, int bq, int n_gsplit,
                                                                int n_qblocks) {
    constexpr int BKV = 32;
    constexpr int NG = 4;            // waves per group
    constexpr int KSTEPS = H / 16;   // S and dP MFMAs per tile
    constexpr int HB = H / 32;
    constexpr int PK = BKV / 16;     // 16-key chunks of a tile
    static_assert(PK * HB == KSTEPS, "one dQ step per S / dP step");
    constexpr int CPR = H / 8;
    constexpr int KRS = CPR + 3, VRS = CPR + 1;
    constexpr int KBLK = (BKV * KRS + 63) / 64, VBLK = (BKV * VRS + 63) / 64;
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
    const int j0 = WIN && t0 - WL > 0 ? (t0 - WL) / BKV : 0;
    // causal: up to the tile of the block's last query's diagonal
    const int n_t = (CAUSAL ? (t0 + bq + a.coff) / BKV : S / BKV) - j0;

    // global -> LDS: group A loads K tiles, group B V tiles; wave gwv of a group
    // issues 1 KiB blocks gwv, gwv + NG, ... (padding slots repeat the row's
    // last chunk; slots past the last padded row re-read row BKV - 1)
    const int rs = grp == 0 ? KRS : VRS;
    const int nblk = grp == 0 ? KBLK : VBLK;
    int ld_off[NL];
#pragma unroll
    for (int i = 0; i < NL; i++) {
        const int pslot = (gwv + i * NG) * 64 + lane;
        ld_off[i] = (min(pslot / rs, BKV - 1) * H + min(pslot % rs, CPR - 1) * 8) * 2;
    }
    // tiles j < n_t lie wholly inside K and V (S % BKV == 0), so the tile
    // offset may go in the scalar offset
    auto issue_tile = [&](int j, int slot) {
        const int tile = __builtin_amdgcn_readfirstlane((j0 + j) * BKV * H * 2);
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
    const int k_lane = n * KRS * 8 + c * 8, v_lane = n * VRS * 8 + c * 8;
    // transpose read of K^T: lane (gi, hh) of 16-lane group c addresses key
    // 16 kk + 4 c + gi / 4 (+ 8 for the upper half) at h = 32 hb + 16 hh + 4 (gi % 4)
    const int tr_lane = (4 * c + ((lane & 15) >> 2)) * KRS * 8 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

    // M phase: S / dP of the tile in slot `cur` (SD) and dQ of the tile in
    // slot `prev` (DQ), interleaved S, dQ hi, dP, dQ lo
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
                const __bf16 *p = kp + tr_lane + kk * 16 * KRS * 8 + hb * 32;
                kt = join_bf16x8(lds_read_tr16(p), lds_read_tr16(p + 8 * KRS * 8));
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
            if constexpr (decltype(dq)::value) dq_acc[hb] = mfma32x32x16(kt, dsl[kk], dq_acc[hb]);
        }
#if GQA_BWD_DQ_PREF > 0
        constexpr bool SD = decltype(sd)::value, DQ = decltype(dq)::value;
        constexpr int NM = (SD ? 2 : 0) + (DQ ? 2 : 0);
        constexpr int D = GQA_BWD_DQ_PREF < KSTEPS ? GQA_BWD_DQ_PREF : KSTEPS;
        pp_schedule<KSTEPS, NM, NM, D>(std::make_integer_sequence<int, D>(), std::make_integer_sequence<int, KSTEPS>());
#endif
        __builtin_amdgcn_s_setprio(0);
        wait_lds_loads();
    };
    // V phase: lane (n, c) holds keys s0 + acc_row(r, c) of query t; dS as
    // bf16 hi + lo (early causal rows have |dS| of order 10, where one bf16
    // rounding alone costs ~1e-1 in dQ)
    auto v_phase = [&](int s0) {
        // some key after some query of the wave, or (WIN) before some query's
        // first visible key t - WL
        const bool masked = (CAUSAL && s0 + BKV - 1 > t_w + a.coff) || (WIN && s0 < t_w + 31 - WL);
        const int lim = t + a.coff - s0 - 4 * c;                // last visible key offset (causal)
        const int first = WIN ? t - WL - s0 - 4 * c : INT_MIN;  // first visible key offset (window)
#pragma unroll
        for (int r = 0; r < 16; r++) {
            float p = exp2_fast(__builtin_fmaf(sacc[r], kLog2e, -lse2));
            const int off = 8 * (r >> 2) + (r & 3);
            if (masked && (off > lim || off < first)) p = 0.f;
            const float ds = p * (pacc[r] - dlt);
            const __bf16 hi = (__bf16)ds;
            dsh[r >> 3][r & 7] = hi;
            dsl[r >> 3][r & 7] = (__bf16)(ds - (float)hi);
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
    m_phase(yes{}, no{}, 0, 0);        // M(-1): S / dP of tile 0
    for (int i = 0; i < n_t - 1; i++) {
        barrier_no_drain();
        if (i + 2 < n_t) issue_tile(i + 2, (i + 2) % NSLOT);
        v_phase((j0 + i) * BKV);
        barrier_no_drain();
        m_phase(yes{}, yes{}, (i + 1) % NSLOT, i % NSLOT);
    }
    barrier_no_drain();
    v_phase((j0 + n_t - 1) * BKV);
    barrier_no_drain();
    m_phase(no{}, yes{}, 0, (n_t - 1) % NSLOT);
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
    constexpr int BKV_D = H <= 128 && GQA_BWD_D_BKV > BKV_DQ ? GQA_BWD_D_BKV : BKV_DQ;
    bool delta_done = false;
    const MaskSpec m{a.causal, a.coff, a.wl, a.wr, a.prefix};
    // causal: the diagonal offset a whole number of tiles, T + coff == S
    auto diag_tiles = [&](int bkv) { return !a.causal || (a.coff >= 0 && a.coff % bkv == 0 && a.T + a.coff == a.S); };
    if constexpr (GQA_BWD_DELTA_PP && H <= 128 && NW_DQ == 8) {
        // dense shapes: the ping-pong D pass (query blocks of 64 rows x gw heads)
        constexpr int BKV_PP = 64;
        const bool shape = a.q_seg == nullptr && gw * bq == 256 && a.T % bq == 0 && a.S % BKV_PP == 0 &&
                           diag_tiles(BKV_PP) && (!a.causal || bq == BKV_PP);
        const bool dense = shape && !mask_extra(m);
        // a causal left window on an otherwise dense shape
        const bool dense_win = shape && mask_left_window_only(m);
        if (dense) {
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
    if constexpr (GQA_BWD_DQ_PP && H <= 128 && NW_DQ == 8) {
        // dense shapes: dQ on the ping-pong kernel (32-key tiles)
        const bool shape = a.q_seg == nullptr && gw * bq == 256 && a.T % bq == 0 && a.S % 32 == 0 && diag_tiles(32);
        const bool dense = shape && !mask_extra(m);
        // a causal left window on an otherwise dense shape
        const bool dense_win = shape && mask_left_window_only(m);
        if (dense) {
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
    if constexpr (GQA_BWD_DKV2 && H <= 128 && NW_DKV == 4) {
        if (a.q_seg == nullptr) {
            if (a.causal)
                hipLaunchKernelGGL((attn_bwd_dkv2_kernel<H, true>), kgrid, dim3(256), 0, stream, a, n_kblocks);
            else
                hipLaunchKernelGGL((attn_bwd_dkv2_kernel<H, false>), kgrid, dim3(256), 0, stream, a, n_kblocks);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((attn_bwd_dkv_kernel<H, NW_DKV>), kgrid, dim3(NW_DKV * 64), 0, stream, a, n_kblocks);
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
