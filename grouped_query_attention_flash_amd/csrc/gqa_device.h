// Device-side helpers shared by the forward and backward kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kLog2e = 1.4426950408889634f;  // log2(e)
constexpr float kLn2 = 0.6931471805599453f;    // ln(2)
// The online softmax moves its reference max only when a row max grows by more
// than this many powers of two, so unnormalised weights stay below 2^8.
constexpr float kRescaleLog2 = 8.0f;
constexpr float kRescaleBound = 256.0f;  // 2^kRescaleLog2

// Lazy mask bounds, resolved on the host (see MaskSpec in gqa_launch.h): key s
// is visible to query t when s < prefix or t - wl <= s <= t + wr. An
// unbounded side is kNoWindow, which exceeds any sequence length the API
// accepts (T, S < 2^23), so t - wl, t + wr and wl + wr + 1 cannot overflow;
// wr may be negative (a causal diagonal below the first query).
constexpr int kNoWindow = 1 << 29;

// The mask sides of query head (kh, g) from a per-head table int32 [K][G][3]
// (window left, window right, prefix), normalised as the host normalises a
// call's single mask: a negative side, or one that bounds nothing for these
// sizes, is kNoWindow; a causal diagonal s <= t + coff caps the right side;
// the prefix is clamped to [0, S]. Every table value is thus accepted.
struct HeadMask {
    int wl, wr, pfx;
};
__device__ __forceinline__ HeadMask head_mask_of(const int32_t *tab, int kh, int G, int g, int T, int S, int causal,
                                                 int coff) {
    const int32_t *e = tab + ((size_t)kh * G + g) * 3;
    const int wl = e[0], wr = e[1], pf = e[2];
    HeadMask h;
    h.wl = (wl < 0 || wl >= T - 1) ? kNoWindow : wl;
    h.wr = (wr < 0 || wr >= S - 1) ? kNoWindow : wr;
    if (causal) h.wr = h.wr < coff ? h.wr : coff;
    h.pfx = pf < 0 ? 0 : (pf < S ? pf : S);
    return h;
}
// Does key tile j (BKV keys) hold a pair that head mask hw hides from a
// wave's query rows t_w .. t_w + 31?
template <int BKV>
__device__ __forceinline__ bool hm_tile_masked(const HeadMask &hw, int j, int t_w) {
    const int s0 = j * BKV;
    const bool all_pfx = s0 + BKV - 1 < hw.pfx;
    const bool all_band = s0 >= t_w + 31 - hw.wl && s0 + BKV - 1 <= t_w + hw.wr;
    return !(all_pfx || all_band);
}

// D = A * B + C on a 32x32 fp32 tile, A 32x16 and B 16x32 in bf16.
// Operand layout (64-wide wave): lane l holds A[l%32][8*(l/32) .. +7] and
// B[8*(l/32) .. +7][l%32]; result register r of lane l is
// D[8*(r/4) + 4*(l/32) + r%4][l%32].
__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row of the 32x32 accumulator tile held by register r of a lane in half c (= lane / 32).
__device__ __forceinline__ constexpr int acc_row(int r, int c) { return 8 * (r >> 2) + 4 * c + (r & 3); }

// LDS layouts of K and V tiles (BKV key rows of H bf16): rows are padded so
// that the MFMA operand reads are bank-conflict free on 64 banks x 4 bytes.
//   K: row stride CPR + 1 chunks of 16 bytes. The A-operand read of 16 lanes
//      (16 consecutive rows, one chunk) hits 16 distinct 16-byte bank groups.
//   V: row stride CPR + 4 chunks. A transpose read of 32 lanes covers 4 rows x
//      64 bytes; rows 4 chunks apart fill the 64 banks exactly once.
// Sizes are rounded up to whole 1 KiB wave loads.
template <int H, int BKV>
struct TileLayout {
    static constexpr int CPR = H / 8;
    static constexpr int KRS = CPR + 1;
    static constexpr int VRS = CPR + 4;
    static constexpr int K_BLOCKS = (BKV * KRS + 63) / 64;
    static constexpr int V_BLOCKS = (BKV * VRS + 63) / 64;
    static constexpr int K_ELEMS = K_BLOCKS * 512;
    static constexpr int V_ELEMS = V_BLOCKS * 512;
};

// XOR swizzle of 16-byte chunks inside one LDS row of CPR chunks. Rows
// r..r+15 (aligned) map one logical chunk to 16 distinct chunk slots, and
// 4 consecutive rows x 4 consecutive chunks (the transpose-read footprint)
// land in distinct 64-byte bank groups.
template <int CPR>
__device__ __forceinline__ int swz(int r) {
    if constexpr (CPR >= 16)
        return ((r & 3) << 2) | ((r >> 2) & 3);
    else
        return ((r & 3) << 1) | ((r >> 2) & 1);
}

// Transposing LDS read (ds_read_b64_tr_b16). Within each 16-lane group,
// lane j receives element (j % 4) of the 4-element chunks addressed by the
// group's lanes j/4, 4 + j/4, 8 + j/4 and 12 + j/4, in that order.
__device__ __forceinline__ s16x4 lds_read_tr16(const __bf16 *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p));
}

// Two 4 x 16-bit transpose-read results as one 8-element bf16 MFMA operand
// (whole-vector bit casts; lo fills elements 0..3, hi 4..7).
__device__ __forceinline__ bf16x8 join_bf16x8(const s16x4 &lo, const s16x4 &hi) {
    typedef int i32x2 __attribute__((ext_vector_type(2)));
    const i32x2 a = __builtin_bit_cast(i32x2, lo);
    const i32x2 b = __builtin_bit_cast(i32x2, hi);
    const i32x4 w = {a[0], a[1], b[0], b[1]};
    return __builtin_bit_cast(bf16x8, w);
}

// Buffer resource over [base, base + bytes): loads past the end return zeros.
typedef __amdgpu_buffer_rsrc_t buffer_rsrc;
// The fields are forced wave-uniform so that the descriptor lives in SGPRs.
__device__ __forceinline__ buffer_rsrc make_rsrc(const void *base, int bytes) {
    const uint64_t p = (uint64_t)(size_t)base;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
    void *ub = (void *)(size_t)(((uint64_t)hi << 32) | lo);
    // 0x00020000: the raw 32-bit data format of gfx9-family buffer descriptors
    return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// 32-bit LDS byte address of a __shared__ object.
__device__ __forceinline__ unsigned lds_addr(const void *p) {
    return (unsigned)(size_t)(const __attribute__((address_space(3))) void *)p;
}

// 16 bytes per lane from a buffer straight into LDS (no registers). The wave's
// 64 lanes write 1 KiB at the LDS destination (a pointer into a __shared__
// array plus a wave-uniform offset, so that the compiler knows which array the
// load writes): lane l at dst + 16 l. voffset is the lane's whole byte offset
// in the buffer: the hardware's range check (a lane at or past the end reads
// zeros) covers the per-lane offset only, not a scalar offset, so none is used.
__device__ __forceinline__ void lds_load16_to(const buffer_rsrc &rs, void *dst, int voffset) {
    typedef __attribute__((address_space(3))) void lds_void;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)dst, 16, voffset, 0, 0, 0);
}
// The same with a wave-uniform scalar offset added to the address: only for
// loads known to stay inside the buffer (the range check ignores soffset).
__device__ __forceinline__ void lds_load16_to(const buffer_rsrc &rs, void *dst, int voffset, int soffset) {
    typedef __attribute__((address_space(3))) void lds_void;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)dst, 16, voffset, soffset, 0, 0);
}

// Buffer descriptor as four wave-uniform words (for inline assembly): base,
// stride 0, num_records = bytes, raw 32-bit data format. Loads past the end
// return zeros.
__device__ __forceinline__ i32x4 make_rsrc_words(const void *base, int bytes) {
    const uint64_t p = (uint64_t)(size_t)base;
    return i32x4{(int)__builtin_amdgcn_readfirstlane((uint32_t)p), (int)__builtin_amdgcn_readfirstlane((uint32_t)(p >> 32)),
                 __builtin_amdgcn_readfirstlane(bytes), 0x00020000};
}

// 16 bytes per lane from a buffer into LDS (lane l writes LDS byte address
// dst + 16 l; dst wave-uniform), issued from inline assembly. voffset is the
// lane's whole byte offset (range-checked as above; 0x80000000 or more reads
// zeros without touching memory). The compiler does not track this load: it
// inserts no wait for it anywhere, so an LDS read of another stage of the same
// array is not held back until the load lands. The caller waits itself
// (wait_lds_loads / wait_lds_loads_but) and passes a barrier before any wave
// reads the destination. M0 carries the destination (one wait state before
// the load reads it) and is restored.
__device__ __forceinline__ void lds_dma16(const i32x4 &rs, unsigned dst, unsigned voffset) {
    int saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(dst), "v"(voffset), "s"(rs));
}

// The same with a wave-uniform byte offset in the scalar offset (not covered
// by the range check: only for loads known to stay inside the buffer).
__device__ __forceinline__ void lds_dma16_so(const i32x4 &rs, unsigned dst, unsigned voffset, int soffset) {
    int saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %2, %3, %4 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(dst), "v"(voffset), "s"(rs), "s"(soffset));
}

// Wait until this wave's LDS-direct loads have landed (vmcnt = 0 only).
__device__ __forceinline__ void wait_lds_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// Wait until at most N of this wave's vector-memory loads are outstanding (they
// complete in issue order), i.e. all but the N most recent have landed.
template <int N>
__device__ __forceinline__ void wait_lds_loads_but() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Workgroup barrier without the release/acquire fence of __syncthreads(),
// which would make every wave drain all of its outstanding global-to-LDS
// loads first. Callers wait themselves (wait_lds_loads_but / wait_lds_loads)
// for the loads that other waves read after the barrier. The wave's own LDS
// reads complete first (lgkmcnt 0), so no wave overwrites a buffer after the
// barrier that another wave is still reading. The memory clobber keeps the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void barrier_no_drain() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Make a value exist in registers at this point of the program: the compiler
// may not sink its computation past here (an empty volatile asm that reads
// and rewrites it).
template <typename V>
__device__ __forceinline__ void pin_value(V &x) {
    asm volatile("" : "+v"(x));
}

// Keep the compiler's scheduler from moving instructions across this point
// (bounds how far ahead it hoists LDS operand reads, and so register pressure).
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// max that propagates NaN (IEEE 754-2019 maximum): gfx950 has a three-input
// form of it, and unlike fmaxf it needs no canonicalisation of its inputs.
__device__ __forceinline__ float max_nan(float a, float b) { return __builtin_elementwise_maximum(a, b); }

__device__ __forceinline__ int wave_min_i(int x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = min(x, __shfl_xor(x, o));
    return x;
}
__device__ __forceinline__ int wave_max_i(int x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = max(x, __shfl_xor(x, o));
    return x;
}

}  // namespace gqa
