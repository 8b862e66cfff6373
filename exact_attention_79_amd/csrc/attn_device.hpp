// attn_device.hpp -- gfx950 device helpers shared by the attention kernels.
//
// MFMA lane layouts used throughout (v_mfma_f32_32x32x16_bf16, wave64):
//   A (32 x 16, row m, col k):  lane l holds A[l % 32][8 * (l / 32) + v], v = 0..7
//   B (16 x 32, row k, col n):  lane l holds B[8 * (l / 32) + v][l % 32], v = 0..7
//   C (32 x 32):                lane l, register r holds
//                               C[8 * (r / 4) + 4 * (l / 32) + (r % 4)][l % 32]
// The C layout gives every lane one column n.  When C is fed back as the B
// operand of the next product, register r of K-step t (r = 8t .. 8t+7) stands
// for row 8 * (r / 4) + 4 * (l / 32) + r % 4 of C, i.e. the contraction index
// is permuted: slot v of lane-half h in K-step t is row
//   16 t + 8 (v / 4) + 4 h + (v % 4).
// The A operand of that product is read with the same permutation, so the
// sum is unchanged and no data moves between lanes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define LDS_AS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Finite stand-in for "no key seen yet" in the running max, so that
// (S - m) never evaluates -inf - (-inf).
constexpr float kMaxInit = -1.0e30f;

// Buffer resource over [base, base + bytes): loads beyond the end return 0.
// Word 3 = 0x00020000 selects 32-bit raw data for gfx9-family buffer ops.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base,
                                                           uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r,
                                            uint32_t byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                       r, (int)byte_off, 0, 0));
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Transposing LDS read: within each 16-lane group, lane i receives element
// (i % 4) of the 8-byte words addressed by lanes 4k + i/4, k = 0..3.  With
// lane j of the group addressing row (r0 + j / 4), columns c0 + 4 (j % 4) ..
// +3 of a row-major bf16 matrix, lane i receives column c0 + i of rows
// r0 .. r0 + 3.
__device__ __forceinline__ bf16x4 lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(p));
}

__device__ __forceinline__ bf16x8 cat4(bf16x4 a, bf16x4 b) {
  return (bf16x8){a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Combine a value with the one held by lane l ^ 32 (the other half of the
// wave).  The lower-half value is always the left operand, so both halves
// compute the identical rounded result.
__device__ __forceinline__ float other_half(float x) {
  return __shfl_xor(x, 32, 64);
}
__device__ __forceinline__ float halves_max(float x) {
  return fmaxf(x, other_half(x));
}
__device__ __forceinline__ float halves_sum(float x) {
  const float y = other_half(x);
  return (threadIdx.x & 32) ? y + x : x + y;
}

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}

// Key j visible to query i (see include/attn.h).
__device__ __forceinline__ bool visible(int i, int j, int N, int causal,
                                        int window) {
  bool ok = j < N;
  if (causal) ok = ok && (j <= i);
  if (window > 0) ok = ok && (i - j < window) && (j - i < window);
  return ok;
}

// Workgroups are dispatched round-robin over the 8 XCDs.  Renumber them so
// that each XCD receives one contiguous range of logical ids (whole heads,
// sharing K/V in that XCD's L2).
__device__ __forceinline__ int xcd_remap(int wg, int total) {
  constexpr int kXcd = 8;
  int q = total / kXcd, r = total % kXcd;
  int xcd = wg % kXcd, local = wg / kXcd;
  return (xcd < r) ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
}

// The key/value head that query head bh (= b * H + h) reads when H query
// heads share Hkv key/value heads: consecutive query heads form a group.
__device__ __forceinline__ int kv_head(int bh, int H, int Hkv) {
  return (bh / H) * Hkv + (bh % H) / (H / Hkv);
}

// Which (batch*head, tile rank) workgroup wg of a grid of BH * n_tiles
// works on.  Whole heads stay on one XCD.  With rank_major (uneven work:
// rank 0 is the heaviest tile of a head) each XCD walks its heads rank by
// rank, so the longest workgroups of all its heads are dispatched before
// any short one; otherwise it walks them head by head.  Rank-major needs
// BH to be a multiple of 8; other grids fall back to head-major order.
struct TileId {
  int bh, rank;
};
__device__ __forceinline__ TileId tile_order(int wg, int BH, int n_tiles, bool rank_major) {
  constexpr int kXcd = 8;
  if (rank_major && BH % kXcd == 0) {
    const int hpx = BH / kXcd, xcd = wg % kXcd, j = wg / kXcd;
    return {xcd * hpx + j % hpx, j / hpx};
  }
  const int logical = xcd_remap(wg, BH * n_tiles);
  return {logical / n_tiles, logical % n_tiles};
}

// ---- LDS tiles of bf16 rows (d elements each), swizzled in 16-byte chunks ----
//
// Two read patterns hit every tile:
//  * row reads: 16 consecutive lanes read the same 16-byte chunk of 16
//    consecutive rows (MFMA A operand, d contiguous);
//  * transposing reads (lds_read_tr16): 32 lanes read 4 consecutive rows
//    (starting at a multiple of 4) x 4 adjacent 16-byte chunks.
// Chunk c of row r is stored at chunk c ^ swz(r).  The swizzle puts the 16
// rows of a row read on 16 different 16-byte bank slots of a 256-byte span,
// and the 4 rows of a transposing read on 4 different groups of 4 slots.
template <int D>
__device__ __forceinline__ int swz(int r);
template <>
__device__ __forceinline__ int swz<128>(int r) {  // 16 chunks per row
  return ((r & 3) << 2) | ((r >> 2) & 3);
}
template <>
__device__ __forceinline__ int swz<64>(int r) {   // 8 chunks; 2 rows per span
  return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// Element offset of (row r, 16-byte chunk ch) inside a swizzled tile.
template <int D>
__device__ __forceinline__ int tile_off(int r, int ch) {
  return r * D + ((ch ^ swz<D>(r)) << 3);
}

// 8 consecutive bf16 of row r starting at column 8*ch.
template <int D>
__device__ __forceinline__ bf16x8 tile_row8(const __bf16* t, int r, int ch) {
  return *(const bf16x8*)&t[tile_off<D>(r, ch)];
}

// Transposing read at (row, col); col is a multiple of 4.
template <int D>
__device__ __forceinline__ bf16x4 tile_tr4(const __bf16* t, int row, int col) {
  return lds_read_tr16(&t[tile_off<D>(row, col >> 3) + (col & 7)]);
}

// Lane coordinates of a transposing read that produces the A operand
// (rows = contraction index in the C-layout permutation, cols = M index):
// for K-step kk and M-tile mt the lane reads rows 16kk + tr_row (+8) at
// column 32mt + tr_col.
struct TrCoord {
  int row, col;
  __device__ __forceinline__ TrCoord(int lane) {
    const int j = lane & 15, g = lane >> 4;
    col = 16 * (g & 1) + 4 * (j & 3);
    row = 4 * (g >> 1) + (j >> 2);
  }
};

template <int D>
__device__ __forceinline__ bf16x8 tile_a_tr(const __bf16* t, const TrCoord& c,
                                            int kk, int mt) {
  const int r = 16 * kk + c.row, col = 32 * mt + c.col;
  return cat4(tile_tr4<D>(t, r, col), tile_tr4<D>(t, r + 8, col));
}

// Global -> LDS copy of a ROWS x D bf16 tile without passing through VGPRs
// (buffer_load_dwordx4 ... lds): each wave instruction writes 64 consecutive
// 16-byte LDS chunks (lane L -> chunk base + L), so each lane fetches the
// global chunk that the swizzle places there.  Rows past the end of the
// buffer resource land as zeros.  Completion is tracked by vmcnt.
template <int D, int ROWS, int NW>
__device__ __forceinline__ void tile_load_lds(__amdgpu_buffer_rsrc_t rs, int row0,
                                              __bf16* t, int w, int lane) {
  constexpr int CH = D / 8;
  constexpr int ROUNDS = ROWS * CH / (64 * NW);
  static_assert((ROWS * CH) % (64 * NW) == 0, "tile must split evenly over waves");
#pragma unroll
  for (int i = 0; i < ROUNDS; ++i) {
    const int base = (i * NW + w) * 64;  // first physical chunk of this instruction
    const int pc = base + lane, row = pc / CH, ch = (pc % CH) ^ swz<D>(row);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (LDS_AS void*)(t + base * 8), 16,
        (int)((uint32_t)((row0 + row) * D + ch * 8) * 2u), 0, 0, 0);
  }
}

// Global -> LDS copy of ROWS consecutive fp32 values (ROWS <= 64) by one
// wave: lane L fetches element row0 + L into LDS word L.
template <int ROWS>
__device__ __forceinline__ void vec_load_lds(__amdgpu_buffer_rsrc_t rs, int row0,
                                             float* t, int lane) {
  static_assert(ROWS == 64, "one dword per lane of one wave");
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void*)t, 4,
                                           (int)((uint32_t)(row0 + lane) * 4u), 0, 0,
                                           0);
}

// s_waitcnt immediate that waits until at most `n` vector-memory operations
// of this wave are outstanding (LDS and export counters not waited on).
__host__ __device__ constexpr int waitcnt_vm(int n) {
  return (n & 0xF) | (0x7 << 4) | (0xF << 8) | ((n >> 4) << 14);
}

}  // namespace attn
