// h2_layout.hpp -- LDS tile layouts of the chunked HGRN2 kernel and the per-access address forms
// it uses.
//
// Three layouts, all XOR swizzles that keep every access of the kernel free of LDS bank conflicts
// on gfx950, whose LDS serves 256 bytes (64 banks of 4 bytes) per cycle: a wave's 8-byte access is
// served in two phases of 32 lanes, a 16-byte access in four phases of 16 lanes, and a phase is
// conflict-free when its lanes touch distinct bank words.
//   qk: [64 rows][128 cols] bf16; 16-byte segment s of row r stored at m(s) ^ f(r), with the 4-bit
//       f(r) = (r2) | (r0 r1) << 1 | r3 << 3 (r_k: bit k of the row) and the linear map m sending
//       segment bits 0..3 to 9, 4, 2, 8; 16 bytes of padding follow every 16 rows, so that rows 16
//       apart (the two token tiles one wave reads in a single two-address instruction) fall on
//       different banks.  m is chosen by measurement: for 16-byte reads of 16 rows by four lane
//       groups, the conflict counters are zero when the lane-group bit that differs between lanes
//       16 apart moves the segment by 9 (rows 12 apart for the same segment), and four cycles per
//       instruction when it moves it by 1 (rows 4 apart), as the plain s ^ f(r) layout does; and
//       9 keeps the transposing K reads, whose lane bits map to 2, 4, 8 and 9, one-to-one;
//   vw: [64 rows][64 cols] bf16; 4-element chunk c of row r stored at c ^ g(r),
//       g(r) = r1 << 2 | (r2 ^ r3) << 3;
//   gv: [64 rows][64 cols] bf16 (staged gate inputs); chunk c of row r stored at c ^ 9 r1.
// qk_off / vw_off / gv_off give the element offset of (row, col) directly.  The kernel addresses
// its operands through the factored forms below: each splits the swizzle into a per-lane term
// computed once per chunk and a term fixed by the (unrolled) loop indices or the wave, so an access
// costs one or two integer operations.  Each factored form equals the direct form for all of its
// arguments (checked exhaustively on the host).
#pragma once

namespace ssd {
namespace h2 {

constexpr int kQkCols = 128;
constexpr int kQkGroupPad = 8;                      // elements (16 bytes) after every 16 rows
constexpr int kQkGroup = 16 * kQkCols + kQkGroupPad;  // elements per 16-row group
constexpr int kQkTile = 4 * kQkGroup;                 // elements per 64-row tile
constexpr int kVwCols = 64;

__host__ __device__ __forceinline__ int qk_f(int row) { return ((row >> 2) & 1) | ((row & 3) << 1) | (row & 8); }
// Linear map of the 4-bit segment index before the row XOR: bits 0, 1, 2, 3 -> 9, 4, 2, 8.
__host__ __device__ __forceinline__ int qk_m(int s) {
  return ((s & 1) ? 9 : 0) ^ ((s & 2) ? 4 : 0) ^ ((s & 4) ? 2 : 0) ^ ((s & 8) ? 8 : 0);
}
__host__ __device__ __forceinline__ int vw_g(int row) {
  return (((row >> 1) & 1) << 2) | ((((row >> 2) ^ (row >> 3)) & 1) << 3);
}
__host__ __device__ __forceinline__ int qk_off(int row, int col) {
  return row * kQkCols + (row >> 4) * kQkGroupPad + ((qk_m(col >> 3) ^ qk_f(row)) << 3) + (col & 7);
}
__host__ __device__ __forceinline__ int vw_off(int row, int col) {
  return row * kVwCols + (((col >> 2) ^ vw_g(row)) << 2) + (col & 3);
}
__host__ __device__ __forceinline__ int gv_off(int row, int col) {
  return row * kVwCols + (((col >> 2) ^ (9 * ((row >> 1) & 1))) << 2) + (col & 3);
}

// Lane decomposition of an MFMA wave: l16 = lane % 16, lg = lane / 16; for 4 x 16 transposing reads
// the lanes of a group split further into b = l16 / 4 (row of the 4-row block), c = l16 % 4 (chunk).

// (A) row 16a + l16, 8-element segment at column 32 ks + 8 lg (MFMA A / B operand rows).
__host__ __device__ __forceinline__ int qk_seg_lane(int l16, int lg) { return qk_m(lg) ^ qk_f(l16); }
__host__ __device__ __forceinline__ int qk_seg_off(int l16, int xa, int a, int ks) {
  return l16 * kQkCols + kQkGroup * a + ((xa ^ qk_m(4 * ks)) << 3);
}

// (B) row 16a + l16, 4 elements at column 32 ks + 16 h + 4 lg.
__host__ __device__ __forceinline__ int qk_quad_lane(int l16, int lg) { return qk_m(lg >> 1) ^ qk_f(l16); }
__host__ __device__ __forceinline__ int qk_quad_off(int l16, int lg, int xb, int a, int ks, int h) {
  return l16 * kQkCols + kQkGroup * a + ((xb ^ qk_m(4 * ks) ^ qk_m(2 * h)) << 3) + 4 * (lg & 1);
}

// (C) transposing read of K: row 32 ks + 8 lg + b + 4 h, 4 elements at column 16 jt + 4 c.
__host__ __device__ __forceinline__ int qk_tr_lane(int l16, int lg) {
  return qk_m((l16 & 3) >> 1) ^ ((l16 >> 2) << 1) ^ (8 * (lg & 1));
}
__host__ __device__ __forceinline__ int qk_tr_off(int l16, int lg, int xd, int ks, int h, int jt) {
  const int b = l16 >> 2, c = l16 & 3;
  return (8 * lg + b) * kQkCols + (lg >> 1) * kQkGroupPad + (32 * ks + 4 * h) * kQkCols + 2 * ks * kQkGroupPad +
         ((xd ^ qk_m(2 * jt) ^ h) << 3) + 4 * (c & 1);
}

// (D) transposing read of the W tile for the output product: row 32 ks + 16 h + 4 lg + b,
//     4 elements at column 16 rt + 4 c (rt: the wave's row tile).
__host__ __device__ __forceinline__ int vw_out_lane(int l16, int lg, int rt) {
  const int b = l16 >> 2, c = l16 & 3;
  const int g = ((b >> 1) << 2) | (((lg & 1) ^ (lg >> 1)) << 3);
  return (4 * lg + b) * kVwCols + ((((4 * rt) ^ c) ^ g) << 2);
}
__host__ __device__ __forceinline__ int vw_out_off(int lane_term, int ks, int h) {
  return lane_term + (32 * ks + 16 * h) * kVwCols;
}

// (E) transposing read of the W tile for the state update: row 32 ks + 8 lg + b + 4 h,
//     4 elements at column 16 rt + 4 c.
__host__ __device__ __forceinline__ int vw_state_lane(int l16, int lg, int rt, int h) {
  const int b = l16 >> 2, c = l16 & 3;
  const int g = ((b >> 1) << 2) | ((h ^ (lg & 1)) << 3);
  return (8 * lg + b + 4 * h) * kVwCols + ((((4 * rt) ^ c) ^ g) << 2);
}
__host__ __device__ __forceinline__ int vw_state_off(int lane_term_h, int ks) { return lane_term_h + 32 * ks * kVwCols; }

// (F) transposing read of the staged gate tiles (gv layout): row 8 gp + b + 4 h, 4 elements at
//     column 16 lg + 4 c.
__host__ __device__ __forceinline__ int gv_gate_off(int l16, int lg, int gp, int h) {
  const int b = l16 >> 2, c = l16 & 3;
  return (8 * gp + 4 * h + b) * kVwCols + ((((4 * lg) ^ c) ^ (9 * (b >> 1))) << 2);
}

// (G) gate-step write of W at row 8 gp + u, column gi (vw layout).
__host__ __device__ __forceinline__ int vw_gate_lane(int gi, int gp) { return (gi >> 2) ^ (8 * (gp & 1)); }
__host__ __device__ __forceinline__ int vw_gate_wr(int gi, int xg, int gp, int u) {
  return (8 * gp + u) * kVwCols + ((xg ^ (4 * ((u >> 1) & 1)) ^ (8 * ((u >> 2) & 1))) << 2) + (gi & 3);
}

}  // namespace h2
}  // namespace ssd
