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

#include "attn_kernels.hpp"

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
// wave) without going through LDS: v_permlane32_swap on two copies of x
// leaves one copy holding the lower half's values in every lane and the
// other the upper half's, and both halves then compute the identical
// rounded result (max and sum are taken of the same two operands).
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                                  __builtin_bit_cast(unsigned, x), false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                                  __builtin_bit_cast(unsigned, x), false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
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
// rank 0 is the heaviest tile of a head) each XCD walks its heads in groups
// of `group` heads, and each group rank by rank, so within a group the
// longest workgroups are dispatched before any short one while only the
// group's heads stream through the XCD's L2 at a time; otherwise it walks
// them head by head.  Rank-major needs BH to be a multiple of 8 (a group
// size that does not divide the XCD's heads means one group of all of
// them); other grids fall back to head-major order.
struct TileId {
  int bh, rank;
};
// Heads per group of the causal walk (0 = all heads of the XCD).  At d = 128
// a head's streamed tensors (K and V, or Q and dO: 4 N d bytes) are 1 MB at
// N = 2048, so the XCD's eight heads at B4 H16 overflow its 4 MB L2: with
// groups of four, a causal B4 H16 N4096 forward fetches 326 MB per launch
// instead of 885 (201 MB compulsory), the dK/dV pass 610 instead of 1089,
// in equal or slightly less time.  Smaller groups fetch less still but
// balance worse and run slower; at d = 64 the heads are half the size and
// grouping only costs balance (3 % slower), so all heads form one group.
template <int D>
constexpr int causal_group() { return D == 128 ? 4 : 0; }
__device__ __forceinline__ TileId tile_order(int wg, int BH, int n_tiles, bool rank_major,
                                             int group) {
  constexpr int kXcd = 8;
  if (rank_major && BH % kXcd == 0) {
    const int hpx = BH / kXcd, xcd = wg % kXcd, j = wg / kXcd;
    const int g = (group > 0 && hpx % group == 0) ? group : hpx;
    const int per = g * n_tiles, grp = j / per, k = j % per;
    return {xcd * hpx + grp * g + k % g, k / g};
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

// Global -> LDS copy of rows row0 .. row0+ROWS-1 of a bf16 [rows][D] head
// (head_bytes long) without passing through VGPRs (buffer_load_dwordx4 ...
// lds): each wave instruction writes 64 consecutive 16-byte LDS chunks (lane
// L -> chunk base + L), so each lane fetches the global chunk that the
// swizzle places there.  The buffer resource starts at row row0 and is built
// with scalar instructions, so each lane's offset is the same for every tile
// and no vector instruction is spent on addresses.  Rows past the end of the
// head land as zeros.  Completion is tracked by vmcnt.
template <int D, int ROWS, int NW>
__device__ __forceinline__ void tile_load_lds(const __bf16* head, uint32_t head_bytes,
                                              int row0, __bf16* t, int w, int lane) {
  constexpr int CH = D / 8;
  constexpr int ROUNDS = ROWS * CH / (64 * NW);
  static_assert((ROWS * CH) % (64 * NW) == 0, "tile must split evenly over waves");
  const uint32_t rows = head_bytes / (D * 2), r0 = (uint32_t)row0;
  const auto rs = make_rsrc(head + (size_t)r0 * D, r0 < rows ? head_bytes - r0 * (D * 2) : 0u);
#pragma unroll
  for (int i = 0; i < ROUNDS; ++i) {
    const int base = (i * NW + w) * 64;  // first physical chunk of this instruction
    const int pc = base + lane, row = pc / CH, ch = (pc % CH) ^ swz<D>(row);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (LDS_AS void*)(t + base * 8), 16, (int)((uint32_t)(row * D + ch * 8) * 2u), 0,
        0, 0);
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

// ---- e4m3 inputs widened to bf16 ----

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Eight e4m3 codes (the bytes of x0, then those of x1) widened to bf16, which
// holds every e4m3 value exactly.  Q and K go through this same routine, so
// the order it gives the eight values in is the same on both sides of a dot
// product.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t x0, uint32_t x1) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)x0, 1.f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)x0, 1.f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)x1, 1.f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)x1, 1.f, true);
  return (bf16x8){a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// The same widening to fp16 (which also holds every e4m3 value exactly).
__device__ __forceinline__ f16x8 e4m3x8_to_f16(uint32_t x0, uint32_t x1) {
  const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)x0, 1.f, false);
  const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)x0, 1.f, true);
  const f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)x1, 1.f, false);
  const f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)x1, 1.f, true);
  return (f16x8){a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Global -> LDS copy of rows row0 .. row0+ROWS-1 of an e4m3 [rows][D] head
// by NW waves, unswizzled: LDS chunk c of the tile holds the tile's 16-byte
// chunk c (row c / (D/16)), so each wave instruction moves 1 KB of
// consecutive bytes.  Rows past the head's end read as zero.
template <int D, int ROWS, int NW>
__device__ __forceinline__ void tile_stage_lds8(const uint8_t* head, uint32_t head_bytes,
                                                int row0, uint8_t* t, int w, int lane) {
  constexpr int ROUNDS = ROWS * D / 16 / (64 * NW);
  static_assert(ROUNDS >= 1 && (ROWS * D / 16) % (64 * NW) == 0, "tile split");
  const uint32_t rows = head_bytes / D, r0 = (uint32_t)row0;
  const auto rs = make_rsrc(head + (size_t)r0 * D, r0 < rows ? head_bytes - r0 * D : 0u);
#pragma unroll
  for (int i = 0; i < ROUNDS; ++i) {
    const int base = (i * NW + w) * 64;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void*)(t + base * 16), 16,
                                             (int)((uint32_t)(base + lane) * 16u), 0, 0, 0);
  }
}

// s_waitcnt immediate that waits until at most `n` vector-memory operations
// of this wave are outstanding (LDS and export counters not waited on).
__host__ __device__ constexpr int waitcnt_vm(int n) {
  return (n & 0xF) | (0x7 << 4) | (0xF << 8) | ((n >> 4) << 14);
}

// ---- dropout on P: keep bytes from a counter-based generator ----
//
// The pages name dropout on the probabilities without fixing a random-number
// contract; the one implemented here: element (query i, key j) of query head
// bh is kept iff its byte is >= the threshold t = round(256 p), kept values
// are scaled by 256 / (256 - t), and the byte comes from Philox-4x32-10
// (Salmon et al., SC 2011) with counter (j/4, i/4, bh, offset) and key
// (seed low, seed high): word i%4 of the output belongs to query i, byte j%4
// of that word (least significant first) to key j.  One generator call thus
// covers a 4 x 4 sub-block of the score matrix, which either MFMA C layout
// (query per lane or key per lane) reaches with one call per lane per 32 x 32
// block plus a transpose within each group of four lanes.
struct Dropout {
  uint32_t thresh;   // t; 0 = no dropout
  uint32_t offset;   // counter word 3
  uint32_t key0, key1;
  float inv_keep;    // 256 / (256 - t)
};

inline Dropout make_dropout(const DropoutArgs& a) {
  Dropout d;
  d.thresh = a.thresh;
  d.offset = a.offset;
  d.key0 = (uint32_t)a.seed;
  d.key1 = (uint32_t)(a.seed >> 32);
  d.inv_keep = a.thresh ? 256.f / (float)(256u - a.thresh) : 1.f;
  return d;
}

__device__ __forceinline__ u32x4 philox4x32_10(u32x4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
    c = (u32x4){(uint32_t)(p1 >> 32) ^ c[1] ^ k0, (uint32_t)p1,
                (uint32_t)(p0 >> 32) ^ c[3] ^ k1, (uint32_t)p0};
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

// Lane i of each group of four reads lane i ^ 1 (quad_perm 1,0,3,2) or
// lane i ^ 2 (quad_perm 2,3,0,1).
__device__ __forceinline__ uint32_t quad_xor1(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t quad_xor2(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false);
}

// Word w of lane s (s = lane % 4) becomes word s of lane w, within each group
// of four lanes: two exchange steps, one per bit of (s, w), in each of which
// the lanes whose bit differs from the word's swap words with the partner.
__device__ __forceinline__ u32x4 quad_transpose(u32x4 a, int s) {
  const bool b0 = s & 1, b1 = s & 2;
  const uint32_t u1 = quad_xor1(b0 ? a[0] : a[1]);
  const uint32_t u3 = quad_xor1(b0 ? a[2] : a[3]);
  a[0] = b0 ? u1 : a[0];
  a[1] = b0 ? a[1] : u1;
  a[2] = b0 ? u3 : a[2];
  a[3] = b0 ? a[3] : u3;
  const uint32_t v0 = quad_xor2(b1 ? a[0] : a[2]);
  const uint32_t v1 = quad_xor2(b1 ? a[1] : a[3]);
  a[0] = b1 ? v0 : a[0];
  a[1] = b1 ? v1 : a[1];
  a[2] = b1 ? a[2] : v0;
  a[3] = b1 ? a[3] : v1;
  return a;
}

// Byte b of word r becomes byte r of word b.
__device__ __forceinline__ u32x4 byte_transpose(u32x4 w) {
  u32x4 o;
#pragma unroll
  for (int b = 0; b < 4; ++b)
    o[b] = ((w[0] >> (8 * b)) & 0xFFu) | (((w[1] >> (8 * b)) & 0xFFu) << 8) |
           (((w[2] >> (8 * b)) & 0xFFu) << 16) | (((w[3] >> (8 * b)) & 0xFFu) << 24);
  return o;
}

// Keep bytes of the 32 x 32 score block of query head bh whose queries start
// at qb and keys at kb (both multiples of 32), arranged like this lane's C
// registers: register r's byte is byte r % 4 of word r / 4.  KEY_PER_LANE
// false: the block is S^T (keys on M, one query per lane); true: S (queries
// on M, one key per lane).
template <bool KEY_PER_LANE>
__device__ __forceinline__ u32x4 dropout_bytes(const Dropout& dr, int bh, int qb, int kb,
                                               int lane) {
  const int n = lane & 31, h = lane >> 5, s = n & 3;
  // This lane draws the sub-block of its quad's 4 rows (n & ~3 on the lane
  // side) and of the rows 8s + 4h .. +3 on the M side.
  const uint32_t I = KEY_PER_LANE ? (uint32_t)(qb / 4 + 2 * s + h) : (uint32_t)(qb / 4 + (n >> 2));
  const uint32_t J = KEY_PER_LANE ? (uint32_t)(kb / 4 + (n >> 2)) : (uint32_t)(kb / 4 + 2 * s + h);
  u32x4 w = philox4x32_10((u32x4){J, I, (uint32_t)bh, dr.offset}, dr.key0, dr.key1);
  // Word r is query row r of the sub-block and byte b its key b; a key-per-
  // lane layout wants one word per key instead.
  if (KEY_PER_LANE) w = byte_transpose(w);
  return quad_transpose(w, s);
}

__device__ __forceinline__ bool dropout_keep(const u32x4& m, int r, uint32_t thresh) {
  return ((m[r >> 2] >> (8 * (r & 3))) & 0xFFu) >= thresh;
}

}  // namespace attn
