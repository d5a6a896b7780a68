// tile_map.h - the scheduler's index arithmetic: which tile (and which piece of it) a
// logical tile index names, for every layout of the grouped GEMM. Pure integer
// functions on host and device, so the kernel's decoding and a host-side exhaustive
// check (tests/tile_map_check.cpp) run the same code.
//
// A call's tiles are numbered 0 .. total-1 and processed in rounds of one per
// workgroup: workgroup b takes logical tiles first_tile_of(b), + grid, + 2 grid, ...
#pragma once

#include <hip/hip_runtime.h>

namespace mgg {

// Logical index of workgroup b's first tile. Workgroups are dispatched to the XCDs
// round-robin (block b runs on XCD b % xcds); each XCD gets a contiguous range of
// grid / xcds logical tiles per round, so neighbouring tiles (same expert, same weight
// panel) share that XCD's L2. A permutation of 0 .. grid-1.
__host__ __device__ inline long first_tile_of(int b, int grid, int xcds) {
  if (grid % xcds != 0) return b;
  const int per = grid / xcds;
  return (long)(b % xcds) * per + b / xcds;
}

// The last round of an M-grouped call, split along N. When there are at least two
// rounds and the last would leave at least half of the workgroups idle, each of its
// tiles becomes 2 or 4 pieces of whole wave columns (bn / pieces >= wtn), one per
// workgroup. Logical indices below `base` are whole tiles; from `base` on, index
// base + k names piece k % pieces of tile base + k / pieces.
struct SplitRound {
  int base;    // first logical index of the split round (== total when not split)
  int pieces;  // pieces per tile of that round (1: no split)
  int total;   // logical indices in all
};

__host__ __device__ inline SplitRound split_last_round(int tiles, int grid, int bn, int wtn) {
  SplitRound r = {tiles, 1, tiles};
  if (tiles <= grid) return r;
  const int base = (tiles - 1) / grid * grid;  // first tile of the last round
  const int last = tiles - base;
  int pieces = 1;
  if (4 * last <= grid && bn / 4 >= wtn) pieces = 4;
  else if (2 * last <= grid && bn / 2 >= wtn) pieces = 2;
  if (pieces > 1) {
    r.base = base;
    r.pieces = pieces;
    r.total = base + last * pieces;
  }
  return r;
}

// The tile a logical index names, and which piece of it.
struct Piece {
  long tile;
  int piece;
  int pieces;
};

__host__ __device__ inline Piece piece_of(long L, int split_base, int split_pieces) {
  Piece q = {L, 0, 1};
  if (L >= split_base) {
    q.pieces = split_pieces;
    q.tile = split_base + (L - split_base) / split_pieces;
    q.piece = (int)((L - split_base) % split_pieces);
  }
  return q;
}

// Weight rows (output columns) [n0, n_end) of piece `piece` of `pieces` of n-tile nt
// (bn columns per n-tile) with N columns in all. A piece of a ragged last n-tile may
// start at or past N: it is then empty (n_end == n0).
__host__ __device__ inline void piece_columns(int nt, int bn, int piece, int pieces, int N,
                                              int* n0, int* n_end) {
  const int width = bn / pieces;
  const int a = nt * bn + piece * width;
  const int b = a + width < N ? a + width : N;
  *n0 = a;
  *n_end = b > a ? b : a;
}

// Masked and prefix-sum layouts: the expert of tile t, i.e. the largest g in [0, G)
// with prefix[g] <= t, where prefix[g] counts the tiles of experts 0 .. g-1 (experts
// with no tiles share their successor's prefix and are never returned for a t below
// the total).
__host__ __device__ inline int expert_of_tile(long t, const int* prefix, int G) {
  int lo = 0, hi = G - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (prefix[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Tile `local` of an expert with mt_g m-tiles: m-tile fastest, so the m-tiles that
// share a weight panel are neighbours.
__host__ __device__ inline void expert_tile(int local, int mt_g, int* mt, int* nt) {
  *nt = local / mt_g;
  *mt = local % mt_g;
}

// Contiguous layout: tile t names n-tile t % ntn of sub-tile `sub` of the valid row block
// with list index `block` (sub_per_block sub-tiles of BM rows per 128-row block).
__host__ __device__ inline void contiguous_tile(long t, int ntn, int sub_per_block, int* block,
                                                int* sub, int* nt) {
  *nt = (int)(t % ntn);
  const long rest = t / ntn;
  *sub = (int)(rest % sub_per_block);
  *block = (int)(rest / sub_per_block);
}

// K-grouped layout: output tile `local` of an expert's mtn x ntn tiles. Tiles go in
// groups of group_m m-tiles, m-tile fastest inside a group; with a 256-workgroup grid
// each XCD runs 32 consecutive tiles at once, which then cover 8 m-tiles x 4 n-tiles of
// the output and read a quarter of the expert's N-side operand per round.
__host__ __device__ inline void kgrouped_tile(int local, int mtn, int ntn, int group_m, int* mt,
                                              int* nt) {
  const int gm = local / (group_m * ntn);  // group of group_m m-tiles
  const int m_first = gm * group_m;
  const int gsz = group_m < mtn - m_first ? group_m : mtn - m_first;  // m-tiles in it
  const int in_g = local - gm * group_m * ntn;
  *mt = m_first + in_g % gsz;
  *nt = in_g / gsz;
}

}  // namespace mgg
