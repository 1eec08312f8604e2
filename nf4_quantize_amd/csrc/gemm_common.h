// gemm_common.h - device helpers shared by the large-M fused NF4 linear
// kernels (linear_fwd.hip, linear_dgrad.hip); internal.
#pragma once

#include "linear_common.h"

namespace nf4 {
namespace gemm {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __amdgpu_buffer_rsrc_t Rsrc;

constexpr int kRsrcFlags = 0x00020000;  // raw buffer, 32-bit data format
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ Rsrc rsrc(const void *base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)(uint32_t)bytes,
                                             kRsrcFlags);
}

// acc += a . b^T on one 16x16x32 tile. Written as an instruction so that the
// accumulators are pinned to AGPRs; the MFMA's own hazards are respected by
// the schedule (no two dependent MFMAs are adjacent, operands are written
// long before use) and by explicit s_nop before the accumulators are read.
// The statement is volatile so that it stays ordered with the wait below.
__device__ __forceinline__ void mfma(f32x4_t &c, const u32x4 &a, const u32x4 &b) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}

// Wait states after the last MFMA that writes an accumulator before any other
// instruction reads it (more than the longest MFMA latency on gfx950).
__device__ __forceinline__ void mfma_drain() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile(
        "s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\t"
        "s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7");
    __builtin_amdgcn_sched_barrier(0);
}

// s_waitcnt immediate that waits until at most n vector-memory loads are
// outstanding (gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt and
// lgkmcnt left at their no-wait maximum).
constexpr int vmcnt_at_most(int n) { return (n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }
// The same with every LDS operation of the wave complete (lgkmcnt 0).
constexpr int vmcnt_at_most_lds_done(int n) { return (n & 15) | ((n >> 4) << 14) | (0x7 << 4); }

// Wait states between VALU writes of MFMA operands and the first MFMA.
__device__ __forceinline__ void valu_to_mfma() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7");
    __builtin_amdgcn_sched_barrier(0);
}

// gfx950's transposing LDS read of 16-bit data (ds_read_b64_tr_b16): every
// lane gives the address of an 8-byte piece (4 elements); within each group
// of 16 lanes, lane i receives element i % 4 of the pieces of lanes i / 4,
// i / 4 + 4, i / 4 + 8 and i / 4 + 12, in that order. With lane j pointing at
// row tau + j / 4, columns 4 (j % 4) .. +3 of a row-major tile, lane i thus
// receives rows tau .. tau + 3 of column i: half of an MFMA operand whose
// contraction runs down the tile's rows.
__device__ __forceinline__ u32x2 lds_read_tr16(const char *p) {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
    const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(p));
    return __builtin_bit_cast(u32x2, v);
}

// Two fp32 values as an fp16 pair (low half first).
__device__ __forceinline__ uint32_t f16_pair(float lo, float hi) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
}

// An fp16 pair of levels scaled by sc and rounded to a bf16 pair. Each half
// is widened exactly and multiplied in fp32 (one rounding) by v_fma_mix_f32,
// which reads the fp16 half directly: 3 VALU instructions for 2 weights.
__device__ __forceinline__ uint32_t scale_pair(uint32_t hh, float sc) {
    float lo, hi;
    asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel_hi:[1,0,0]" : "=v"(lo) : "v"(hh), "v"(sc));
    asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(hi) : "v"(hh), "v"(sc));
    return pack_bf16x2(lo, hi);
}

// Workgroup -> (m tile, n tile). Consecutive workgroups go round robin to the
// 8 XCDs; when the tile count is a multiple of 8 each XCD is given a
// contiguous run of the order below. The order walks bands of 8 column tiles,
// rows fastest within a band, so the ~32 workgroups an XCD runs at once
// cover about 4 row tiles x 8 column tiles and share X rows and W rows in
// that XCD's L2.
__device__ __forceinline__ void tile_of(int64_t wg, int64_t tm, int64_t tn, int64_t &mt, int64_t &nt) {
    const int64_t total = tm * tn;
    const int64_t L = (total % 8 == 0) ? (wg % 8) * (total / 8) + wg / 8 : wg;
    constexpr int64_t kGN = 8;
    const int64_t band = L / (kGN * tm), within = L % (kGN * tm);
    const int64_t nb = min(kGN, tn - band * kGN);
    mt = within / nb;
    nt = band * kGN + within % nb;
}

// A value that is the same in every lane, moved to scalar registers.
__device__ __forceinline__ int64_t uniform(int64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// LDS layout of a tile of 128-byte rows (64 bf16 of K) fed by direct-to-LDS
// loads and read as MFMA fragments. Row r sits in 128-byte segment
// tile_seg(r): rows 0-7 of each 16-row block at its even segments, rows 8-15
// at the odd ones; its 16-byte chunk c at position c ^ (r & 7).
//  - A fragment read (lanes 16k .. 16k+15 read one chunk of 16 consecutive
//    rows) then puts lanes 0-7 of each group on one half of the 64 LDS banks
//    and lanes 8-15 on the other, each on 8 distinct 16-byte positions: the
//    ds_read_b128 rate of a contiguous read, measured on gfx950. A chunk
//    swizzle by row with both halves inside each 8-lane octet runs at 0.7 of
//    it (bank conflicts).
//  - A direct-to-LDS load writes 16 bytes per lane, lane-linearly: lanes 8j
//    .. 8j+7 fill one segment, so they read one row's 128 bytes.
__host__ __device__ constexpr int tile_seg(int r) { return (r & ~15) | ((r & 7) << 1) | ((r >> 3) & 1); }
// the row held by segment s (the inverse of tile_seg)
__host__ __device__ constexpr int seg_row(int s) { return (s & ~15) | ((s >> 1) & 7) | ((s & 1) << 3); }
static_assert(seg_row(tile_seg(13)) == 13 && tile_seg(seg_row(7)) == 7, "tile_seg and seg_row are inverse");

}  // namespace gemm
}  // namespace nf4
