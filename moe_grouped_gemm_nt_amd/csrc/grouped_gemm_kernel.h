// grouped_gemm_kernel.h - the persistent grouped NT GEMM kernel template (the design is
// described in gemm_engine.h). Included by exactly one translation unit, which
// instantiates it for every (tile, variant, dtype, scale format, weight-scale
// granularity, accumulation) combination the host dispatcher can pick.
//
// Pipeline. A workgroup walks a flat sequence of work items (tile, 128-byte K slice)
// with four copy waves, four or eight MFMA waves and, with an accumulation input, four
// epilogue waves:
//   - copy waves run the issue cursor: they start the direct global -> LDS copies of
//     item i + S - 1 into ring stage (i + S - 1) % S. Each copy wave issues the same
//     number of copy instructions for every item (out-of-range lanes and idle items
//     copy zeros), so before the barrier of item i it waits (vmcnt counts in issue
//     order) for exactly its copies of item i;
//   - MFMA waves run the compute cursor: the MFMAs of item i from stage i % S and, on a
//     tile's last slice, the epilogue. They never issue copies, so they never stall
//     waiting to enter the memory pipeline;
//   - with an accumulation input (K-grouped D = C + A B^T), epilogue waves: the MFMA
//     waves write each finished tile into one of two LDS exchange buffers instead of
//     storing it; the epilogue waves keep the C tiles of the next kCPrefetch tiles in
//     flight in their registers, and after the barrier that publishes a tile they add
//     it to its C tile and store D.
// One barrier per item makes the copies of item i visible and guarantees that the stage
// about to be refilled is no longer being read. Every group walks the same tile
// sequence and executes the same number of barriers (one per item, plus a final one
// that publishes the last exchange tile), so nothing else needs synchronising.
#pragma once

#include <type_traits>

#include "act_math.h"
#include "gemm_engine.h"
#include "tile_map.h"

namespace mgg {

// Everything a workgroup needs to run one output tile. All fields are uniform.
struct TileCtx {
  int valid;     // 0 once the workgroup has no more tiles
  int g;         // expert
  int m0, n0;    // first activation row / weight row of the tile
  int n_end;     // end of the tile's weight rows (output columns): min(N, n0 + BN)
  int nk;        // 128-byte K slices to run (at least 1)
  int k_bytes;   // bytes of K in an activation row (0: nothing to load; FP4 weights: half)
  int a_lim;     // activation rows < a_lim are loaded (others read as zero)
  int row_end;   // masked: valid rows end; contiguous/K-grouped: M
  const uint8_t* a_base;  // the tile's first activation row (row m0)
  uint32_t a_bytes;       // bytes of the tile's rows that exist in the operand
  const uint8_t* b_base;  // weight rows from b_row0 on (this n-tile's, or the expert's)
  uint32_t b_bytes;
  int b_row0;             // weight row at b_base
  int lda, ldb;  // row strides in bytes
  long sfa_off;  // element offset of scale group 0, row 0
  int sfa_ld;    // elements between consecutive scale groups
  long sfb_off;
  int sfb_ld;
  uint8_t* d_base;  // the tile's first output row (row m0)
  uint32_t d_bytes; // bytes of the tile's output rows that exist
};

template <class T, int VAR>
struct Sched {
  int* s_a;    // masked, psum: tile prefix [G]; K-grouped: p_e [G + 1], with
               // kKUnusable set on experts outside the routing contract
  int* s_b;    // masked, psum: row counts [G]; contiguous: packed (block << 12 | expert)
               // of each valid block
  int* s_c;    // psum: first row of each expert's segment [G]
  int total;   // number of tiles (a split last round counts each piece)
  int ntn;     // n tiles per expert
  int mtn;     // K-grouped: m tiles per expert
  int split_base;  // M-grouped: first tile of a last round that is split along N
  int split_p;     // pieces per tile of that round (1: no split)
};

// LDS layout of one pipeline stage. Every region is a whole number of copy
// instructions (1 KB for 16-byte copies, 256 B for 4-byte copies).
template <class T, int VAR, int DT, int SF, int GRAN, bool ACC>
struct Layout {
  static constexpr bool FP8 = DT != kBF16;  // scaled FP8 activations (FP8 or FP4 weights)
  static constexpr bool FP4W = DT == kFP4W;
  static constexpr int cdiv(int a, int b) { return (a + b - 1) / b; }
  // Weight bytes per row per 128-K slice (FP4: two elements per byte).
  static constexpr int B_ROW = FP4W ? kSliceBytes / 2 : kSliceBytes;
  // Scale runs: float32 -> one lane per scale; UE8M0 -> one lane per aligned dword of
  // the byte run (the run may start anywhere inside a dword).
  static constexpr int SA_LANES = FP8 ? (SF == kSfF32 ? T::BM : T::BM / 4 + 2) : 0;
  static constexpr int SBN_BLOCK = T::BN >= 128 ? T::BN / 128 : 1;
  // FP4 weights: one dword per weight row per slice (its four 32-K block scales).
  static constexpr int SB_LANES =
      FP4W ? T::BN
           : FP8 ? (GRAN == kSfbChannel ? (SF == kSfF32 ? T::BN : T::BN / 4 + 2) : SBN_BLOCK)
                 : 0;
  static constexpr int SA_INSTR = cdiv(SA_LANES, 64);
  static constexpr int SB_INSTR = cdiv(SB_LANES, 64);
  static constexpr int RI_INSTR = VAR == kContig ? cdiv(T::BM, 64) : 0;
  // Copy slots per wave. Operand rows: slot u of wave w copies rows 8(4u + w) ..
  // 8(4u + w) + 7 of the [A; B] tile, so A and B slots are fixed per u (BM % 32 == 0);
  // FP4 weight rows are 64 bytes, so a weight slot covers 16 of them.
  // Scale and row-index copies are few: they are dealt to the four waves ("small"
  // slots: small copy e goes to wave e % 4, so a wave issues U_SM or U_SM - 1 of them).
  static constexpr int U_A = T::BM / 32, U_B = T::BN * B_ROW / 4096, U_AB = U_A + U_B;
  static constexpr int SMALL = SA_INSTR + SB_INSTR + RI_INSTR;
  static constexpr int U_SM = cdiv(SMALL, 4);
  static constexpr int PER_WAVE = U_AB + U_SM;  // most copy instructions per wave per item
  // copy instructions per item of copy wave cw: its operand slots and the small copies
  // dealt to it (e = 4 us + cw < SMALL)
  static constexpr int per_wave(int cw) {
    int n = U_AB;
    for (int us = 0; us < U_SM; ++us) n += 4 * us + cw < SMALL ? 1 : 0;
    return n;
  }

  static constexpr int A_OFF = 0;
  static constexpr int B_OFF = T::BM * kSliceBytes;
  static constexpr int SA_OFF = B_OFF + T::BN * B_ROW;
  static constexpr int SB_OFF = SA_OFF + SA_INSTR * 256;
  static constexpr int RI_OFF = SB_OFF + SB_INSTR * 256;
  static constexpr int STAGE = RI_OFF + RI_INSTR * 256;
  static constexpr int PIPE = T::S * STAGE;

  // Accumulation: threads per workgroup (MFMA waves + epilogue waves) and the two fp32
  // tile exchange buffers after the ring. A row of R_ROW_CHUNKS 16-byte chunks; chunk c
  // of row r sits at position c ^ (r % R_ROW_CHUNKS), which keeps both the MFMA-layout
  // writes and the row-order reads free of bank conflicts.
  static constexpr int EPI0 = T::NMW;                   // first epilogue wave
  static constexpr int COPY0 = T::NMW + (ACC ? 4 : 0);  // first of the four copy waves
  static constexpr int NT = (COPY0 + 4) * 64;
  static_assert(!ACC || T::NMW == 4, "accumulating tiles use four MFMA waves");
  static constexpr int R_ROW_CHUNKS = T::BN / 4;
  static constexpr int R_HALF = ACC ? T::BM * T::BN * 4 : 0;
  static constexpr int R_OFF = PIPE;
  static constexpr int SCHED_OFF = PIPE + 2 * R_HALF;  // scheduler tables follow

  static_assert(FP8 || (T::WTM % 32 == 0 && T::WTN % 32 == 0), "BF16 needs 32x32 subtiles");
  static_assert(!FP4W || (SF == kSfUE8M0 && GRAN == kSfbBlock32 && VAR != kKGrouped &&
                          T::BN % 64 == 0),
                "FP4 weights: UE8M0 scales applied by the MFMA, M-grouped, whole 16-row copies");
  static_assert(FP4W == (GRAN == kSfbBlock32), "32-K weight scales go with FP4 weights");
  static_assert(PER_WAVE * (T::S - 1) <= 63, "vmcnt range of a copy wave");
  static_assert(!ACC || ((R_ROW_CHUNKS & (R_ROW_CHUNKS - 1)) == 0 && R_ROW_CHUNKS <= 64 &&
                         (T::BM * T::BN / 4) % 256 == 0),
                "accumulation exchange: power-of-two row chunks, whole chunks per lane");
  static_assert(!(ACC && VAR != kKGrouped), "accumulation is K-grouped only");
};

// The tiles of an M-grouped call go in rounds of one per workgroup; a mostly idle last
// round is split along N (split_last_round in tile_map.h): every output is computed
// exactly as in the whole tile, and a memory-bound last round gets two or four times as
// many CUs fetching its weights.
template <class T, int VAR>
__device__ __forceinline__ void split_rounds(Sched<T, VAR>& S) {
  const SplitRound r = split_last_round(S.total, gridDim.x, T::BN, T::WTN);
  S.split_base = r.base;
  S.split_p = r.pieces;
  S.total = r.total;
}

template <class T, int VAR, int NT>
__device__ __forceinline__ void sched_init(Sched<T, VAR>& S, const Params& p, int* s_tmp,
                                           int* s_flag) {
  const int tid = threadIdx.x;
  S.ntn = (p.N + T::BN - 1) / T::BN;
  if constexpr (VAR == kMasked) {
    for (int g = tid; g < p.G; g += NT) {
      int c = p.meta[g];
      c = c < 0 ? 0 : (c > p.rows ? p.rows : c);
      S.s_b[g] = c;
      S.s_a[g] = ((c + T::BM - 1) / T::BM) * S.ntn;
    }
    __syncthreads();
    S.total = block_exclusive_scan<NT>(S.s_a, p.G, s_tmp);
    split_rounds(S);
  } else if constexpr (VAR == kPsum) {
    // Expert g owns rows [start_g, end_g): end_g = clamp(psum[g], 0, M) raised to the
    // running maximum of the earlier ends, start_g = end_{g-1} (0 for g = 0), so the
    // segments never overlap whatever the routing holds.
    for (int g = tid; g < p.G; g += NT) {
      int e = p.meta[g];
      S.s_c[g] = e < 0 ? 0 : (e > p.rows ? p.rows : e);
    }
    __syncthreads();
    block_inclusive_max<NT>(S.s_c, p.G, s_tmp);  // s_c[g] = end_g
    int st0[8], cnt[8];  // this thread's experts (G <= 8 * NT)
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int g = tid + q * NT;
      st0[q] = cnt[q] = 0;
      if (g < p.G) {
        st0[q] = g > 0 ? S.s_c[g - 1] : 0;
        cnt[q] = S.s_c[g] - st0[q];
      }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int g = tid + q * NT;
      if (g < p.G) {
        S.s_c[g] = st0[q];
        S.s_b[g] = cnt[q];
        S.s_a[g] = ((cnt[q] + T::BM - 1) / T::BM) * S.ntn;
      }
    }
    __syncthreads();
    S.total = block_exclusive_scan<NT>(S.s_a, p.G, s_tmp);
    split_rounds(S);
  } else if constexpr (VAR == kContig) {
    // s_flag (transient, inside the pipeline stages) holds the block flags and then
    // their prefix; s_ent (transient, after it) the block's packed entry. Valid blocks are
    // packed into s_b in block order as (sub-tiles << 24 | block << 12 | expert), where
    // "sub-tiles" counts the leading BM-row sub-tiles whose first row still belongs to
    // the expert (valid rows come first in a block). Every routing value is read once,
    // here: the tile decode reads only these tables, so every wave of the workgroup
    // walks the same tile sequence whatever the routing buffer holds.
    constexpr int SUB = kContigBlock / T::BM;
    const int nb = (p.rows + kContigBlock - 1) / kContigBlock;
    int* s_ent = s_flag + nb;
    for (int b = tid; b < nb; b += NT) {
      const long r0 = (long)b * kContigBlock;
      const int e = p.meta[r0];
      const bool ok = e >= 0 && e < p.G;
      int nsub = ok ? 1 : 0;
      for (int k = 1; k < SUB && nsub == k; ++k) {
        const long r = r0 + k * T::BM;
        if (r < p.rows && p.meta[r] == e) ++nsub;
      }
      s_flag[b] = ok ? 1 : 0;
      s_ent[b] = (nsub << 24) | (b << 12) | (ok ? e : 0);
    }
    __syncthreads();
    const int nvalid = block_exclusive_scan<NT>(s_flag, nb, s_tmp);
    for (int b = tid; b < nb; b += NT)
      if (s_ent[b] >> 24) S.s_b[s_flag[b]] = s_ent[b];
    __syncthreads();
    S.total = nvalid * SUB * S.ntn;
    S.split_base = S.total;
    S.split_p = 1;
    // 128-row tiles only: every logical tile is then a real one (no padding sub-tiles)
    if constexpr (SUB == 1 && !T::SWI) split_rounds(S);
  } else {
    // p_e = sum_{j<e} max(k_j, 0) saturated at K + 1: an expert is usable only if its
    // tokens end at or before K, so the saturation changes no decision, and no routing
    // value can overflow the prefix or move an operand base outside its tensor. A usable
    // expert's count is p_{e+1} - p_e (p_G closes the table).
    // The counts, clamped to [-1, K + 1] (which keeps every decision), wait in s_flag
    // (transient) so the routing buffer is read once.
    S.mtn = (p.rows + T::BM - 1) / T::BM;
    const int cap = p.K + 1;  // K <= 2^28
    for (int g = tid; g < p.G; g += NT) {
      const long k = p.meta_psum ? (long)p.meta[g] - (g > 0 ? (long)p.meta[g - 1] : 0L)
                                 : (long)p.meta[g];
      const int kc = k < 0 ? -1 : (k > cap ? cap : (int)k);
      s_flag[g] = kc;
      S.s_a[g] = kc < 0 ? 0 : kc;
    }
    __syncthreads();
    const int pg = block_exclusive_scan_sat<NT>(S.s_a, p.G, s_tmp, cap);
    if (tid == 0) S.s_a[p.G] = pg;
    for (int g = tid; g < p.G; g += NT) {
      const int k = s_flag[g];
      const int pe = S.s_a[g];
      const bool usable = k >= 0 && (k % p.k_granule) == 0 && (pe % p.k_granule) == 0 &&
                          pe + k <= p.K;
      if (!usable) S.s_a[g] = pe | kKUnusable;
    }
    __syncthreads();
    S.total = p.G * S.mtn * S.ntn;
    S.split_base = S.total;
    S.split_p = 1;
  }
}

// Logical index of the workgroup's first tile; its later tiles follow in steps of the
// grid size (the XCD-aware order of first_tile_of in tile_map.h).
__device__ __forceinline__ long first_tile() {
  return first_tile_of(blockIdx.x, gridDim.x, kXcds);
}

// Decodes logical tile L; tiles with nothing to do are skipped by advancing L in steps
// of the grid size, and L is left at the tile returned.
constexpr int kKGroupM = 8;  // K-grouped tile order: m-tiles per group (see decode_tile)

// The tile context is the same for every lane of a wave, but the scheduler tables it is
// decoded from are read from LDS into vector registers. Each value read from a table goes
// through wave_uniform (one readfirstlane), so that everything derived from it is computed
// in scalar registers and the decoded context does not hold ~25 vector registers through
// the slice loop.
__device__ __forceinline__ int wave_uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ uint32_t wave_uniform(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}
__device__ __forceinline__ long wave_uniform(long v) {
  const uint64_t u = (uint64_t)v;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(u >> 32));
  return (long)(((uint64_t)hi << 32) | lo);
}
template <class P>
__device__ __forceinline__ P* wave_uniform(P* v) {
  return reinterpret_cast<P*>(wave_uniform(reinterpret_cast<long>(v)));
}
// Every field of a decoded context (most are already scalar; this pins the rest).
__device__ __forceinline__ void make_uniform(TileCtx& t) {
  t.valid = wave_uniform(t.valid);
  t.g = wave_uniform(t.g);
  t.m0 = wave_uniform(t.m0);
  t.n0 = wave_uniform(t.n0);
  t.n_end = wave_uniform(t.n_end);
  t.nk = wave_uniform(t.nk);
  t.k_bytes = wave_uniform(t.k_bytes);
  t.a_lim = wave_uniform(t.a_lim);
  t.row_end = wave_uniform(t.row_end);
  t.a_base = wave_uniform(t.a_base);
  t.a_bytes = wave_uniform(t.a_bytes);
  t.b_base = wave_uniform(t.b_base);
  t.b_bytes = wave_uniform(t.b_bytes);
  t.b_row0 = wave_uniform(t.b_row0);
  t.lda = wave_uniform(t.lda);
  t.ldb = wave_uniform(t.ldb);
  t.sfa_off = wave_uniform(t.sfa_off);
  t.sfa_ld = wave_uniform(t.sfa_ld);
  t.sfb_off = wave_uniform(t.sfb_off);
  t.sfb_ld = wave_uniform(t.sfb_ld);
  t.d_base = wave_uniform(t.d_base);
  t.d_bytes = wave_uniform(t.d_bytes);
}

template <class T, int VAR, int DT, int GRAN, bool PIN>
__device__ __forceinline__ TileCtx decode_fields(const Sched<T, VAR>& S, const Params& p, long& L) {
  auto pin = [](int v) { return PIN ? wave_uniform(v) : v; };
  TileCtx t = {};  // valid == 0, null bases: an idle cursor copies nothing
  constexpr int esz = DT == kBF16 ? 2 : 1;  // activation bytes per element
  if constexpr (VAR == kMasked || VAR == kPsum) {
    if (L < S.total) {
      const Piece q = piece_of(L, S.split_base, S.split_p);
      const int g = pin(expert_of_tile(q.tile, S.s_a, p.G));
      const int c = pin(S.s_b[g]);
      const int mt_g = (c + T::BM - 1) / T::BM;
      int mt, nt;
      expert_tile((int)(q.tile - pin(S.s_a[g])), mt_g, &mt, &nt);
      const int Kb = p.K * esz;
      const int KB = p.K / 128;
      t.valid = 1;
      t.g = g;
      t.m0 = mt * T::BM;
      // an empty piece (n_end == n0) has a weight resource of size 0 and stores nothing
      piece_columns(nt, T::BN, q.piece, q.pieces, p.N, &t.n0, &t.n_end);
      t.k_bytes = Kb;
      t.nk = (Kb + kSliceBytes - 1) / kSliceBytes;
      t.a_lim = c;
      t.row_end = c;
      // masked: expert g's block of cap rows; psum: its segment of the [M] rows. Buffer
      // resources start at the tile's first row (and first weight row), so 32-bit offsets
      // never span more than one tile whatever the operand sizes, and end at its last
      // valid row: the padding rows of a masked block read as zeros without being fetched.
      const long r0 = VAR == kPsum ? (long)pin(S.s_c[g]) : (long)g * p.rows;
      const long rt = min((long)T::BM, (long)c - t.m0);  // valid rows of the tile
      const int Kbw = DT == kFP4W ? Kb / 2 : Kb;  // weight bytes per row
      t.a_base = p.A + (r0 + t.m0) * Kb;
      t.a_bytes = (uint32_t)(rt * Kb);
      t.b_row0 = T::SWI ? 0 : t.n0;
      t.b_base = p.B + ((long)g * p.N + t.b_row0) * Kbw;
      t.b_bytes = (uint32_t)((T::SWI ? (long)p.N : (long)(t.n_end - t.n0)) * Kbw);
      t.lda = Kb;
      t.ldb = Kbw;
      t.sfa_off = VAR == kPsum ? r0 : (long)g * KB * p.rows;
      t.sfa_ld = p.rows;
      if constexpr (GRAN == kSfbBlock) {
        t.sfb_off = (long)g * ((p.N + 127) / 128) * KB;
        t.sfb_ld = KB;  // distance between consecutive 128-row blocks
      } else {
        t.sfb_off = (long)g * KB * p.N;
        t.sfb_ld = p.N;
      }
      t.d_base = reinterpret_cast<uint8_t*>(p.D) + (r0 + t.m0) * p.N * 2;
      t.d_bytes = (uint32_t)(rt * p.N * 2);
    }
  } else if constexpr (VAR == kContig) {
    constexpr int SUB = kContigBlock / T::BM;
    while (L < S.total) {
      const Piece q = piece_of(L, S.split_base, S.split_p);
      int block, sub, nt;
      contiguous_tile(q.tile, S.ntn, SUB, &block, &sub, &nt);
      const int packed = pin(S.s_b[block]);
      const int blk = (packed >> 12) & 0xfff, e = packed & 0xfff, nsub = packed >> 24;
      const int m0 = blk * kContigBlock + sub * T::BM;
      // A sub-tile that starts on padding is padding throughout (valid rows come first
      // in a block); skip it without loading anything.
      if (sub >= nsub || m0 >= p.rows) { L += gridDim.x; continue; }
      const int Kb = p.K * esz;
      const int KB = p.K / 128;
      t.valid = 1;
      t.g = e;
      t.m0 = m0;
      if constexpr (T::SWI) {
        t.n0 = nt * T::BN;
        t.n_end = p.N;
      } else {
        piece_columns(nt, T::BN, q.piece, q.pieces, p.N, &t.n0, &t.n_end);
      }
      t.k_bytes = Kb;
      t.nk = (Kb + kSliceBytes - 1) / kSliceBytes;
      t.a_lim = p.rows;
      t.row_end = p.rows;
      const long rt = min((long)T::BM, (long)(p.rows - m0));  // rows of the tile that exist
      const int Kbw = DT == kFP4W ? Kb / 2 : Kb;  // weight bytes per row
      t.a_base = p.A + (long)m0 * Kb;
      t.a_bytes = (uint32_t)(rt * Kb);
      t.b_row0 = T::SWI ? 0 : t.n0;
      t.b_base = p.B + ((long)e * p.N + t.b_row0) * Kbw;
      t.b_bytes = (uint32_t)((T::SWI ? (long)p.N : (long)(t.n_end - t.n0)) * Kbw);
      t.lda = Kb;
      t.ldb = Kbw;
      t.sfa_off = 0;
      t.sfa_ld = p.rows;
      if constexpr (GRAN == kSfbBlock) {
        t.sfb_off = (long)e * ((p.N + 127) / 128) * KB;
        t.sfb_ld = KB;
      } else {
        t.sfb_off = (long)e * KB * p.N;
        t.sfb_ld = p.N;
      }
      // bf16 [rows][N]; the fused SwiGLU tile writes E4M3 codes [rows][N/2]
      const long ldd = T::SWI ? p.N / 2 : (long)p.N * 2;
      t.d_base = reinterpret_cast<uint8_t*>(p.D) + (long)m0 * ldd;
      t.d_bytes = (uint32_t)(rt * ldd);
      break;
    }
  } else {
    while (L < S.total) {
      const int per = S.mtn * S.ntn;
      const int e = (int)(L / per);
      const int local = (int)(L % per);
      const int se = __builtin_amdgcn_readfirstlane(S.s_a[e]);
      const int k = (__builtin_amdgcn_readfirstlane(S.s_a[e + 1]) & ~kKUnusable) - se;
      if ((se & kKUnusable) || (k == 0 && p.accumulate)) { L += gridDim.x; continue; }
      // groups of kKGroupM m-tiles (kgrouped_tile in tile_map.h): with n-tile fastest,
      // every XCD read the expert's whole N-side operand in each round (8x its bytes)
      int mt, nt;
      kgrouped_tile(local, S.mtn, S.ntn, kKGroupM, &mt, &nt);
      const long pe = se;
      t.valid = 1;
      t.g = e;
      t.m0 = mt * T::BM;
      t.n0 = nt * T::BN;
      t.n_end = min(p.N, t.n0 + T::BN);
      t.k_bytes = k * esz;
      t.nk = t.k_bytes > 0 ? (t.k_bytes + kSliceBytes - 1) / kSliceBytes : 1;
      t.a_lim = p.rows;
      t.row_end = p.rows;
      const long rt = min((long)T::BM, (long)(p.rows - t.m0));
      const long ct = min((long)T::BN, (long)(p.N - t.n0));
      // expert e's blocks [M][k_e] and [N][k_e], entered at the tile's first row
      t.a_base = p.A + ((long)p.rows * pe + (long)t.m0 * k) * esz;
      t.a_bytes = (uint32_t)(rt * k * esz);
      t.b_row0 = t.n0;
      t.b_base = p.B + ((long)p.N * pe + (long)t.n0 * k) * esz;
      t.b_bytes = (uint32_t)(ct * k * esz);
      t.lda = t.ldb = k * esz;
      t.sfa_off = (pe / 128) * p.rows;
      t.sfa_ld = p.rows;
      t.sfb_off = (pe / 128) * p.N;
      t.sfb_ld = p.N;
      t.d_base = reinterpret_cast<uint8_t*>(p.D) + ((long)e * p.rows + t.m0) * p.N * 4;
      t.d_bytes = (uint32_t)(rt * p.N * 4);
      break;
    }
  }
  return t;
}

// PIN: whether the context is moved to scalar registers. It relieves the vector registers
// of every tile that runs close to its register limit; the contiguous layout with UE8M0
// scales, which has room and decodes a new tile every few slices, runs faster without.
template <class T, int VAR, int DT, int GRAN, bool PIN = true>
__device__ __forceinline__ TileCtx decode_tile(const Sched<T, VAR>& S, const Params& p, long& L) {
  TileCtx t = decode_fields<T, VAR, DT, GRAN, PIN>(S, p, L);
  if constexpr (PIN) make_uniform(t);
  return t;
}

// ----------------------------------------------------------------------------- epilogue
// waves of an accumulating K-grouped call

// Runs on the four epilogue waves (ew = 0..3) from the first tile t0 (logical index L0)
// onwards. Lane chunk u of a tile is the 16-byte piece q = 256 u + 64 ew + lane in row
// order (row q / R_ROW_CHUNKS, column chunk q % R_ROW_CHUNKS), so every load and store
// instruction covers whole 256-byte row segments. The C tile of the k-th tile from now
// sits in ring slot k % kCPrefetch; the MFMA waves publish tile x in exchange buffer
// x % 2 with the barrier that follows its last slice.
template <class T, int VAR, int DT, int GRAN, class Lay>
__device__ __forceinline__ void accumulate_waves(const Sched<T, VAR>& Sd, const Params& p,
                                                 const uint8_t* smem, TileCtx t0, long L0,
                                                 int ew, int lane) {
  constexpr int ROWC = Lay::R_ROW_CHUNKS;
  constexpr int PER = T::BM * T::BN / 4 / 256;  // chunks per lane per tile
  constexpr int P = kCPrefetch;
  static_assert(P % 2 == 0, "exchange buffer parity follows the ring slot");
  const int grid = gridDim.x;
  int rr[PER], cc[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int q = 256 * u + 64 * ew + lane;
    rr[u] = q / ROWC;
    cc[u] = q % ROWC;
  }
  auto offset = [&](const TileCtx& t, int u) -> uint32_t {
    const int m = t.m0 + rr[u], n = t.n0 + 4 * cc[u];
    return (t.valid && m < p.rows && n < p.N) ? (uint32_t)(((long)rr[u] * p.N + n) * 4) : kOOB;
  };
  v4i ring[P][PER];
  TileCtx tp = t0;  // prefetch cursor, P tiles ahead of te
  long Lp = L0;
  auto prefetch = [&](v4i* slot) {
    const v4i rs = make_rsrc(tp.d_base, tp.d_bytes);
#pragma unroll
    for (int u = 0; u < PER; ++u) slot[u] = load_b128<kCacheStream>(rs, offset(tp, u));
    if (tp.valid) {
      Lp += grid;
      tp = decode_tile<T, VAR, DT, GRAN>(Sd, p, Lp);
    }
  };
  // Between the first P prefetches go PER dropped stores each (zero-size resource), so
  // the first pass around the loop sees the same count of younger memory operations as
  // every later one (a slot's loads are followed by P - 1 tiles' stores and loads).
#pragma unroll
  for (int q = 0; q < P; ++q) {
    prefetch(ring[q]);
    if (q < P - 1) {
      const v4i none = make_rsrc(nullptr, 0);
#pragma unroll
      for (int u = 0; u < PER; ++u) store_b128(none, kOOB + 16 * u, (v4i){0, 0, 0, 0});
    }
  }

  TileCtx te = t0;
  long Le = L0;
  int nb = te.nk + 1;  // barriers until the first tile is published
  while (true) {
#pragma unroll
    for (int q = 0; q < P; ++q) {
      for (int b = 0; b < nb; ++b) lds_barrier();
      const uint8_t* R = smem + Lay::R_OFF + (q & 1) * Lay::R_HALF;
      const v4i rs = make_rsrc(te.d_base, te.d_bytes);
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int pc = cc[u] ^ (rr[u] % ROWC);
        const v4f r = *reinterpret_cast<const v4f*>(R + rr[u] * T::BN * 4 + pc * 16);
        const v4i c = ring[q][u];
        const v4f d = r + (v4f){__int_as_float(c.x), __int_as_float(c.y),
                                __int_as_float(c.z), __int_as_float(c.w)};
        store_b128<kCacheStream>(rs, offset(te, u),
                                 (v4i){__float_as_int(d[0]), __float_as_int(d[1]),
                                       __float_as_int(d[2]), __float_as_int(d[3])});
      }
      prefetch(ring[q]);
      Le += grid;
      te = decode_tile<T, VAR, DT, GRAN>(Sd, p, Le);
      nb = te.nk;  // 0 once the sequence has ended: the remaining slots only idle
    }
    // The only exit is here, after all P slots, so every path around the loop passes
    // every slot and the compiler's wait for a slot's C tile stays P - 1 tiles deep.
    if (!te.valid) return;
  }
}

// ----------------------------------------------------------------------------- kernel

template <class T, int VAR, int DT, int SF, int GRAN, bool ACC>
__global__ __launch_bounds__((Layout<T, VAR, DT, SF, GRAN, ACC>::NT)) void grouped_gemm_kernel(
    Params p) {
  using Lay = Layout<T, VAR, DT, SF, GRAN, ACC>;
  constexpr bool FP8 = Lay::FP8;
  constexpr int NI = T::NI, MJ = T::MJ, S = T::S;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cwave = (wave - Lay::COPY0) & 3;  // slot index of a copy wave
  const int lr = lane & 15, lg = lane >> 4;
  // MFMA waves are numbered down the tile's columns, so the waves of one wave column (all
  // the work of a 64-column piece of a split last round) sit on different SIMDs
  const int wave_m = wave % T::WM, wave_n = wave / T::WM;
  const int wm0 = wave_m * T::WTM, wn0 = wave_n * T::WTN;

  // ---- scheduler (its scan scratch lies in the pipeline stages, unused until the
  // first copy is issued)
  Sched<T, VAR> Sd;
  {
    int* base = reinterpret_cast<int*>(smem + Lay::SCHED_OFF);
    const int n = (VAR == kContig) ? (p.rows + kContigBlock - 1) / kContigBlock : p.G;
    Sd.s_a = base;
    Sd.s_b = base + (VAR == kContig ? 0 : n);  // unused by K-grouped calls
    Sd.s_c = base + 2 * n;
    int* s_tmp = reinterpret_cast<int*>(smem);
    int* s_flag = s_tmp + kThreads;
    sched_init<T, VAR, Lay::NT>(Sd, p, s_tmp, s_flag);
  }
  const uint32_t lds0 = lds_addr(smem);
  const int grid = gridDim.x;

  v4i rs_sfa = FP8 ? make_rsrc(p.SFA, p.sfa_bytes) : v4i{0, 0, 0, 0};
  v4i rs_sfb = FP8 ? make_rsrc(p.SFB, p.sfb_bytes) : v4i{0, 0, 0, 0};
  v4i rs_meta = make_rsrc(p.meta, p.meta_bytes);
  pin_sgpr(rs_sfa);
  pin_sgpr(rs_sfb);
  pin_sgpr(rs_meta);

  // ---- the issue cursor's per-tile copy state: resource descriptors and per-lane
  // byte offsets of every operand-row copy slot (kOOB for rows outside the tile's
  // valid range); a slice only adds its K offset.
  // Global weight row of tile-local weight row w, and whether it exists. The fused
  // SwiGLU tile's rows 0..127 are the gate rows of its 128 output columns and rows
  // 128..255 the matching up rows, N / 2 further on.
  auto weight_row = [&](const TileCtx& t, int w, int& n) -> bool {
    if constexpr (T::SWI) {
      const int oc = t.n0 / 2 + (w & 127);
      n = (w < 128 ? 0 : p.N / 2) + oc;
      return oc < p.N / 2;
    } else {
      n = t.n0 + w;
      return n < p.N;
    }
  };
  struct Issue {
    TileCtx t;
    v4i rs_a, rs_b;
    uint32_t vab[Lay::U_AB];
  };
  // Logical 16-byte chunk this lane copies: the LDS row of every copy is 8q + lane / 8
  // (so its low 3 bits are lane / 8) and the chunk is XOR-swizzled with them.
  const int c16 = ((lane & 7) ^ (lane >> 3)) << 4;
  auto prepare = [&](Issue& I) {
    const TileCtx& t = I.t;
    I.rs_a = make_rsrc(t.a_base, t.a_bytes);
    I.rs_b = make_rsrc(t.b_base, t.b_bytes);
    pin_sgpr(I.rs_a);
    pin_sgpr(I.rs_b);
#pragma unroll
    for (int u = 0; u < Lay::U_AB; ++u) {
      const int R = 8 * (4 * u + cwave) + (lane >> 3);
      if (u < Lay::U_A) {
        const int m = t.m0 + R;
        I.vab[u] = (t.valid && m < t.a_lim) ? (uint32_t)(R * t.lda + c16) : kOOB;
      } else if constexpr (Lay::FP4W) {
        // 16 weight rows of 64 bytes per copy; chunk c of LDS row Rb sits at position
        // c ^ ((Rb / 2) % 4), so 8 consecutive rows read at one logical chunk hit 8
        // different 16-byte bank groups.
        const int Rb = 16 * (4 * (u - Lay::U_A) + cwave) + (lane >> 2);
        const int lc = (lane & 3) ^ ((Rb >> 1) & 3);
        int n;
        const bool ok = weight_row(t, weight_row_of_lds<T, false>(Rb), n);
        I.vab[u] = (t.valid && ok) ? (uint32_t)((n - t.b_row0) * t.ldb + 16 * lc) : kOOB;
      } else {
        int n;
        const bool ok = weight_row(t, weight_row_of_lds<T, !FP8>(R - T::BM), n);
        I.vab[u] = (t.valid && ok) ? (uint32_t)((n - t.b_row0) * t.ldb + c16) : kOOB;
      }
    }
  };

  // ---- copies of one item (tile I.t, slice s) into stage `stg` by copy wave `cw` (a
  // compile-time constant); an idle cursor copies zeros so a wave's instruction count per
  // item never changes.
  auto issue = [&](const Issue& I, int s, int stg, auto cw) {
    constexpr int CW = decltype(cw)::value;
    const TileCtx& t = I.t;
    const uint32_t st = lds0 + stg * Lay::STAGE;
    const int kb0 = s * kSliceBytes;
    const bool full = kb0 + kSliceBytes <= t.k_bytes;  // no K tail inside this slice
    const bool k_any = t.k_bytes > 0;
    dma_fence();
    // Rows that end inside the slice (a BF16 K tail) need a per-lane test; every other
    // slice copies with the slice's K offset in the instruction's scalar offset, so a
    // lane's offset (kOOB for rows outside the tile) is the same for every slice of the
    // tile. FP8 activations come in whole 128-K groups, so FP8 slices are never cut (an
    // FP8 tile with no K, an empty K-grouped expert, has resources of size 0 and its
    // copies read zeros); FP4 weight rows advance 64 bytes per slice.
    auto operands = [&](auto tail) {
#pragma unroll
      for (int u = 0; u < Lay::U_AB; ++u) {
        const uint32_t lds_u = st + Lay::A_OFF + 1024 * (4 * u + CW);
        const v4i rs = u < Lay::U_A ? I.rs_a : I.rs_b;
        // Weight rows read once stream past the caches (tiles built for it, chosen on
        // the host).
        constexpr bool nt_w = T::STREAMW;
        if constexpr (decltype(tail)::value) {
          uint32_t voff = I.vab[u] + kb0;
          if (kb0 + c16 + 16 > t.k_bytes) voff = kOOB;
          if (u >= Lay::U_A && nt_w) dma_x4_nt(lds_u, rs, voff);
          else dma_x4(lds_u, rs, voff);
        } else {
          const uint32_t so = Lay::FP4W && u >= Lay::U_A ? (uint32_t)(s * Lay::B_ROW)
                                                          : (uint32_t)kb0;
          if (u >= Lay::U_A && nt_w) dma_x4_nt_so(lds_u, rs, I.vab[u], so);
          else dma_x4_so(lds_u, rs, I.vab[u], so);
        }
      }
    };
    if constexpr (Lay::FP8) {
      operands(std::false_type{});
    } else {
      if (full) operands(std::false_type{});
      else operands(std::true_type{});
    }
    static_for<0, Lay::U_SM>([&](auto us_c) {
      constexpr int e = 4 * decltype(us_c)::value + CW;  // small copy dealt to this wave
      if constexpr (e < Lay::SA_INSTR) {
        const int l = 64 * e + lane;
        const long o = t.sfa_off + (long)s * t.sfa_ld + t.m0;
        uint32_t voff = kOOB;
        if constexpr (SF == kSfF32) {
          if (t.valid && k_any && l < T::BM) voff = (uint32_t)((o + l) * 4);
        } else {
          if (t.valid && k_any && l < Lay::SA_LANES) voff = (uint32_t)((o & ~3L) + 4 * l);
        }
        dma_x1(st + Lay::SA_OFF + 256 * e, rs_sfa, voff);
      } else if constexpr (e < Lay::SA_INSTR + Lay::SB_INSTR) {
        const int j = e - Lay::SA_INSTR;
        const int l = 64 * j + lane;
        uint32_t voff = kOOB;
        if constexpr (GRAN == kSfbBlock32 || (GRAN == kSfbChannel && SF == kSfF32)) {
          // one dword per weight row: four 32-K block scales, or one float32 scale
          const long o = t.sfb_off + (long)s * t.sfb_ld;
          int n;
          const bool ok = l < T::BN && weight_row(t, l, n);
          if (t.valid && k_any && ok) voff = (uint32_t)((o + n) * 4);
        } else if constexpr (GRAN == kSfbChannel) {
          const long o = t.sfb_off + (long)s * t.sfb_ld + t.n0;
          static_assert(!T::SWI, "byte-run channel scales are not gathered");
          if (t.valid && k_any && l < Lay::SB_LANES) voff = (uint32_t)((o & ~3L) + 4 * l);
        } else {
          // 128x128 blocks; the fused tile's two are its gate block and its up block
          const int nb = T::SWI ? (l == 0 ? t.n0 / 256 : p.N / 256 + t.n0 / 256) : t.n0 / 128 + l;
          const long o = t.sfb_off + (long)nb * t.sfb_ld + s;
          if (t.valid && k_any && l < Lay::SBN_BLOCK && nb * 128 < p.N)
            voff = SF == kSfF32 ? (uint32_t)(o * 4) : (uint32_t)(o & ~3L);
        }
        dma_x1(st + Lay::SB_OFF + 256 * j, rs_sfb, voff);
      } else if constexpr (e < Lay::SMALL) {
        const int j = e - Lay::SA_INSTR - Lay::SB_INSTR;
        const int l = 64 * j + lane;
        const int m = t.m0 + l;
        dma_x1(st + Lay::RI_OFF + 256 * j, rs_meta,
               (t.valid && l < T::BM && m < p.rows) ? (uint32_t)(m * 4) : kOOB);
      }
    });
  };

  // ---- per-lane constant LDS offsets of the MFMA fragments (XOR swizzle folded in)
  const int x_lo = ((lg) ^ (lr & 7)) << 4;
  const int x_hi = ((lg + 4) ^ (lr & 7)) << 4;
  const int x_w4 = (lg ^ ((lr >> 1) & 3)) << 4;  // FP4 weight rows (16 | R - lr)

  constexpr int NI2 = T::NI2, MJ2 = T::MJ2;
  v4f acc[FP8 ? NI : 1][FP8 ? MJ : 1];     // FP8: 16x16 subtiles
  v16f acc2[FP8 ? 1 : NI2][FP8 ? 1 : MJ2];  // BF16: 32x32 subtiles

  // MFMA work of one slice held in stage `stg`.
  auto compute = [&](const TileCtx& t, int s, int stg) {
    const uint8_t* st = smem + stg * Lay::STAGE;
    if constexpr (FP8 && SF == kSfUE8M0) {
      constexpr int kFmtW = Lay::FP4W ? 4 : 0;  // weight operand format: E2M1 or E4M3
      // Power-of-two scales: the MFMA applies them itself (its E8M0 operand scales, one
      // per lane for the 32 K elements that lane supplies: activation and FP8 weight
      // scales are the same across the slice, FP4 weight scales change every 32 K) and
      // accumulates into the tile accumulator, so no promotion instructions are needed:
      // the weight scale goes with the first operand (weight rows), the activation
      // scale with the second (activation rows).
      // Scale bytes first (see the float32-scale path below for the order of the rest).
      int sab[MJ];
      const long oa = t.sfa_off + (long)s * t.sfa_ld + t.m0;
#pragma unroll
      for (int j = 0; j < MJ; ++j) sab[j] = st[Lay::SA_OFF + (int)(oa & 3) + wm0 + 16 * j + lr];
      int sbw = 0, sbw2 = 0;  // block scale of the wave's rows (fused tile: gate, up)
      if constexpr (GRAN == kSfbBlock) {
        if constexpr (T::SWI) {
          const long og = t.sfb_off + (long)(t.n0 / 256) * t.sfb_ld + s;
          const long ou = t.sfb_off + (long)(p.N / 256 + t.n0 / 256) * t.sfb_ld + s;
          sbw = st[Lay::SB_OFF + (int)(og & 3)];
          sbw2 = st[Lay::SB_OFF + 4 + (int)(ou & 3)];
        } else {
          const int lb = ((t.n0 & 127) + wn0) >> 7;
          const long ob = t.sfb_off + (long)(t.n0 / 128 + lb) * t.sfb_ld + s;
          sbw = st[Lay::SB_OFF + 4 * lb + (int)(ob & 3)];
        }
      }
      // Activation fragment j: 16 rows x 128 K of the wave's rows.
      auto load_a = [&](int j, v8i& b) {
        const uint8_t* rp = st + Lay::A_OFF + (wm0 + 16 * j + lr) * kSliceBytes;
        const v4i lo = *reinterpret_cast<const v4i*>(rp + x_lo);
        const v4i hi = *reinterpret_cast<const v4i*>(rp + x_hi);
        b = (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      };
      // Weight fragment i and the scale of the weight row this lane supplies.
      auto load_w = [&](int i, v8i& afr, int& sb) {
        const int R = wn0 + 16 * i + lr;
        if constexpr (Lay::FP4W) {
          // 32 FP4 elements (K 32 lg .. 32 lg + 31) in the first four registers, and the
          // scale of exactly that 32-K block of the weight row
          const v4i q = *reinterpret_cast<const v4i*>(st + Lay::B_OFF + R * Lay::B_ROW + x_w4);
          afr = (v8i){q.x, q.y, q.z, q.w, 0, 0, 0, 0};
          sb = st[Lay::SB_OFF + 4 * weight_row_of_lds<T, false>(R) + lg];
        } else {
          const uint8_t* rp = st + Lay::B_OFF + R * kSliceBytes;
          const v4i lo = *reinterpret_cast<const v4i*>(rp + x_lo);
          const v4i hi = *reinterpret_cast<const v4i*>(rp + x_hi);
          afr = (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
          // fused tile: LDS rows 16 i + lr hold weight rows 64 (lr / 4) + 4 i + lr % 4, so
          // lanes lr >= 8 supply up rows
          sb = (T::SWI && lr >= 8) ? sbw2 : sbw;
          if constexpr (GRAN == kSfbChannel) {
            const long ob = t.sfb_off + (long)s * t.sfb_ld + t.n0;
            sb = st[Lay::SB_OFF + (int)(ob & 3) + weight_row_of_lds<T, false>(R)];
          }
        }
      };
      v8i bfr[MJ];
      v8i wf[3];
      int sw[3];
      auto mfma = [&](int i, int j) {
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            wf[i % 3], bfr[j], acc[i][j], kFmtW, 0, 0, sw[i % 3], 0, sab[j]);
      };
      constexpr int NA = MJ > 2 ? MJ - 2 : 0;  // activation reads behind the first group
      constexpr int NW = NI - 1 < 2 ? NI - 1 : 2;  // weight reads behind it
      auto later_read = [&](int q) {
        if (q < NA) load_a(q + 2, bfr[q + 2]);
        else if (q - NA < NW) load_w(q - NA + 1, wf[q - NA + 1], sw[q - NA + 1]);
      };
      load_w(0, wf[0], sw[0]);
      load_a(0, bfr[0]);
      if (MJ > 1) load_a(1, bfr[1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < MJ; ++j) {
        mfma(0, j);
        later_read(j);
        if (j == MJ - 1) {
#pragma unroll
          for (int q = MJ; q < NA + NW; ++q) later_read(q);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int i = 1; i < NI; ++i) {
#pragma unroll
        for (int j = 0; j < MJ; ++j) {
          mfma(i, j);
          if (j == 0 && i + 2 < NI) load_w(i + 2, wf[(i + 2) % 3], sw[(i + 2) % 3]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    } else if constexpr (FP8) {
      // Scales first: they are small reads, and the waits for them then never wait on
      // the fragment reads issued behind them.
      float sa[MJ];
      const long oa = t.sfa_off + (long)s * t.sfa_ld + t.m0;
#pragma unroll
      for (int j = 0; j < MJ; ++j) {
        const int row = wm0 + 16 * j + lr;
        if constexpr (SF == kSfF32)
          sa[j] = reinterpret_cast<const float*>(st + Lay::SA_OFF)[row];
        else
          sa[j] = ue8m0_to_float(st[Lay::SA_OFF + (int)(oa & 3) + row]);
      }
      float sbw = 0.f, sbw2 = 0.f;  // block scale of the wave's rows (fused tile: gate, up)
      if constexpr (GRAN == kSfbBlock) {
        const int lb = ((t.n0 & 127) + wn0) >> 7;
        if constexpr (SF == kSfF32) {
          sbw = reinterpret_cast<const float*>(st + Lay::SB_OFF)[T::SWI ? 0 : lb];
          if constexpr (T::SWI) sbw2 = reinterpret_cast<const float*>(st + Lay::SB_OFF)[1];
        } else {
          static_assert(!T::SWI || SF == kSfF32, "unreachable: UE8M0 takes the MFMA-scaled path");
          const long ob = t.sfb_off + (long)(t.n0 / 128 + lb) * t.sfb_ld + s;
          sbw = ue8m0_to_float(st[Lay::SB_OFF + 4 * lb + (int)(ob & 3)]);
        }
      }
      // Activation fragment j: 16 rows x 128 K of the wave's rows.
      auto load_a = [&](int j, v8i& b) {
        const uint8_t* rp = st + Lay::A_OFF + (wm0 + 16 * j + lr) * kSliceBytes;
        const v4i lo = *reinterpret_cast<const v4i*>(rp + x_lo);
        const v4i hi = *reinterpret_cast<const v4i*>(rp + x_hi);
        b = (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      };
      // Weight fragment i (and its per-channel scales) from LDS.
      auto load_w = [&](int i, v8i& afr, v4f& sbv) {
        const uint8_t* rp = st + Lay::B_OFF + (wn0 + 16 * i + lr) * kSliceBytes;
        const v4i lo = *reinterpret_cast<const v4i*>(rp + x_lo);
        const v4i hi = *reinterpret_cast<const v4i*>(rp + x_hi);
        afr = (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        {
          // fused tile: this lane's output columns 64 lg + 4 i + r are up columns for lg >= 2
          const float b = (T::SWI && lg >= 2) ? sbw2 : sbw;
          sbv = (v4f){b, b, b, b};
        }
        if constexpr (GRAN == kSfbChannel) {
          const int col = wn0 + lg * 4 * NI + 4 * i;
          if constexpr (SF == kSfF32) {
            sbv = *reinterpret_cast<const v4f*>(st + Lay::SB_OFF + 4 * col);
          } else {
            const long ob = t.sfb_off + (long)s * t.sfb_ld + t.n0;
            const uint8_t* bp = st + Lay::SB_OFF + (int)(ob & 3) + col;
            sbv = (v4f){ue8m0_to_float(bp[0]), ue8m0_to_float(bp[1]), ue8m0_to_float(bp[2]),
                        ue8m0_to_float(bp[3])};
          }
        }
      };
      // Software pipeline, with its order fixed by scheduling fences (left alone, the
      // scheduler waits for every read of the slice before the first MFMA and gathers
      // most promotion FMAs behind the last one, where they cannot overlap MFMA work):
      //  - the first MFMA waits only for weight fragment 0 and activation fragment 0;
      //    each MFMA of weight fragment 0 is followed by one read of a later fragment;
      //  - each MFMA of weight fragment i >= 1 is followed by the promotion of one
      //    partial sum of fragment i - 1 into the float32 accumulator, so the FMAs run
      //    while the MFMA pipe is busy; fragment i + 2 is read behind the last of them.
      // Partial sums alternate between two register sets (format 0 = FP8 E4M3 for both
      // operands; scale exponent 127 = 2^0).
      const v4f zero = {0.f, 0.f, 0.f, 0.f};
      v4f part[2][MJ];
      v8i bfr[MJ];
      v8i wf[3];
      v4f sv[3];
      auto promote = [&](int i, int j) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          acc[i][j][r] = __builtin_fmaf(part[i & 1][j][r], sa[j] * sv[i % 3][r], acc[i][j][r]);
      };
      constexpr int NA = MJ > 2 ? MJ - 2 : 0;  // activation reads behind the first group
      constexpr int NW = NI - 1 < 2 ? NI - 1 : 2;  // weight reads behind it
      auto later_read = [&](int q) {
        if (q < NA) load_a(q + 2, bfr[q + 2]);
        else if (q - NA < NW) load_w(q - NA + 1, wf[q - NA + 1], sv[q - NA + 1]);
      };
      load_w(0, wf[0], sv[0]);
      load_a(0, bfr[0]);
      if (MJ > 1) load_a(1, bfr[1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < MJ; ++j) {
        part[0][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf[0], bfr[j], zero, 0, 0,
                                                                      0, 127, 0, 127);
        later_read(j);
        if (j == MJ - 1) {
#pragma unroll
          for (int q = MJ; q < NA + NW; ++q) later_read(q);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int i = 1; i < NI; ++i) {
#pragma unroll
        for (int j = 0; j < MJ; ++j) {
          part[i & 1][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              wf[i % 3], bfr[j], zero, 0, 0, 0, 127, 0, 127);
          promote(i - 1, j);
          // fragment i + 2 reuses the registers of fragment i - 1, whose scales the
          // promotions above still read
          if (j == MJ - 1 && i + 2 < NI) load_w(i + 2, wf[(i + 2) % 3], sv[(i + 2) % 3]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
#pragma unroll
      for (int j = 0; j < MJ; ++j) promote(NI - 1, j);
    } else {
      // 32x32x16 MFMAs: MFMA h of the slice takes K elements 16h .. 16h + 15; lane group
      // g = lane / 32 supplies elements 16h + 8g .. 16h + 8g + 7, the 16-byte chunk
      // 2h + g of its row.
      // The fragments of step h + 1 are read from LDS while the MFMAs of step h run.
      const int l32 = lane & 31, g2 = lane >> 5;
      v8bf bf[2][MJ2], wf[2][NI2];
      auto load_h = [&](int h, v8bf* b, v8bf* w) {
        const int xo = ((2 * h + g2) ^ (l32 & 7)) << 4;
#pragma unroll
        for (int j = 0; j < MJ2; ++j)
          b[j] = *reinterpret_cast<const v8bf*>(st + Lay::A_OFF + (wm0 + 32 * j + l32) * kSliceBytes + xo);
#pragma unroll
        for (int i = 0; i < NI2; ++i)
          w[i] = *reinterpret_cast<const v8bf*>(st + Lay::B_OFF + (wn0 + 32 * i + l32) * kSliceBytes + xo);
      };
      load_h(0, bf[0], wf[0]);
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        if (h + 1 < 4) load_h(h + 1, bf[(h + 1) & 1], wf[(h + 1) & 1]);
#pragma unroll
        for (int i = 0; i < NI2; ++i)
#pragma unroll
          for (int j = 0; j < MJ2; ++j)
            acc2[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[h & 1][i], bf[h & 1][j],
                                                                 acc2[i][j], 0, 0, 0);
      }
      // Instruction order for the scheduler: the first step's reads, then each MFMA
      // followed by one read of the next step's fragments.
      {
        constexpr int kReads = MJ2 + NI2;
        __builtin_amdgcn_sched_group_barrier(0x100, kReads, 0);  // LDS reads
#pragma unroll
        for (int h = 0; h < 4; ++h)
#pragma unroll
          for (int q = 0; q < NI2 * MJ2; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            if (h + 1 < 4 && q < kReads) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
      }
    }
  };

  // Row-masked stores of the finished tile: lanes outside the valid rows / columns use
  // an out-of-range offset. With an
  // accumulation input the tile goes to the exchange buffer at byte offset `rx` instead.
  auto epilogue = [&](const TileCtx& t, int stg, int rx) {
    const uint8_t* st = smem + stg * Lay::STAGE;
    uint8_t* R = smem + Lay::R_OFF + rx;
    const v4i rs_d = make_rsrc(t.d_base, t.d_bytes);
    if constexpr (T::SWI) {
      // Fused SwiGLU + FP8 1x128 quantization of the tile's 128 output columns. Each
      // accumulator is first rounded to bf16 (the value a separate GEMM would store), so
      // the codes equal those of the separate SwiGLU kernel run on that output. Lane group
      // g (lane / 16) holds tile columns 64 g .. 64 g + 63 of its row: gate columns for
      // g < 2, the matching up columns for g >= 2 (lane + 32). The two lanes of a pair
      // swap halves so that each ends with 32 gate and 32 up values of the same output
      // columns: lane g < 2 computes outputs 64 g .. 64 g + 31, lane g + 2 outputs
      // 64 g + 32 .. 64 g + 63. The row's maximum meets over the four lanes.
      static_assert(MJ == 1 && NI == 16 && VAR == kContig, "fused tile: one 16-row band per wave");
      const int rl = wm0 + lr;
      const int m = t.m0 + rl;
      const int I = p.N / 2, oc0 = t.n0 / 2;
      bool row_ok = m < t.row_end && oc0 < I;
      row_ok = row_ok && reinterpret_cast<const int*>(st + Lay::RI_OFF)[rl] == t.g;
      const bool lo = lg < 2;
      float x[8][4];
      float amax = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float h0 = __uint_as_float(f32_to_bf16_rne(acc[i][0][r]) << 16);
          const float h1 = __uint_as_float(f32_to_bf16_rne(acc[i + 8][0][r]) << 16);
          const float other = __shfl_xor(lo ? h1 : h0, 32);  // the partner's half
          const float gate = lo ? h0 : other, up = lo ? other : h1;
          x[i][r] = silu_fixed(gate) * up;
          amax = fmaxf(amax, fabsf(x[i][r]));
        }
      amax = fmaxf(amax, __shfl_xor(amax, 16));
      amax = fmaxf(amax, __shfl_xor(amax, 32));
      uint32_t bits;
      const float inv = p.sfq_ue8m0 ? group_scale_1x128<true>(amax, p.sf_zero, bits)
                                    : group_scale_1x128<false>(amax, p.sf_zero, bits);
      const int col = oc0 + 64 * (lg & 1) + (lo ? 0 : 32);  // first output column of lane
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        v4i w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float* v = x[4 * q + e];
          w[e] = (int)to_e4m3x4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
        }
        const uint32_t voff = row_ok ? (uint32_t)((long)rl * I + col + 16 * q) : kOOB;
        store_b128(rs_d, voff, w);
      }
      const v4i rs_q = make_rsrc(p.SFQ, p.sfq_bytes);
      const long qi = (long)(oc0 / 128) * p.rows + m;
      const bool wq = row_ok && lg == 0;
      if (p.sfq_ue8m0)
        store_b8(rs_q, wq ? (uint32_t)qi : kOOB, bits);
      else
        store_b32(rs_q, wq ? (uint32_t)(qi * 4) : kOOB, bits);
      return;
    }
    if constexpr (FP8) {
      const int nl0 = wn0 + lg * 4 * NI;  // tile-local first column of this lane
      const int n_start = t.n0 + nl0;
#pragma unroll
      for (int j = 0; j < MJ; ++j) {
        const int rl = wm0 + 16 * j + lr;
        const int m = t.m0 + rl;
        bool row_ok = m < t.row_end;
        if constexpr (VAR == kContig)
          row_ok = row_ok && reinterpret_cast<const int*>(st + Lay::RI_OFF)[rl] == t.g;
        if constexpr (VAR == kKGrouped) {
#pragma unroll
          for (int i = 0; i < NI; ++i) {
            const v4f v = acc[i][j];
            if constexpr (ACC) {
              const int pc = ((nl0 + 4 * i) / 4) ^ (rl % Lay::R_ROW_CHUNKS);
              *reinterpret_cast<v4f*>(R + rl * T::BN * 4 + pc * 16) = v;
              continue;
            }
            const bool ok = row_ok && n_start + 4 * i + 4 <= p.N;
            const uint32_t voff = ok ? (uint32_t)(((long)rl * p.N + n_start + 4 * i) * 4) : kOOB;
            store_b128(rs_d, voff, (v4i){__float_as_int(v[0]), __float_as_int(v[1]),
                                         __float_as_int(v[2]), __float_as_int(v[3])});
          }
        } else {
#pragma unroll
          for (int h = 0; h < NI / 2; ++h) {
            const v4f x = acc[2 * h][j], y = acc[2 * h + 1][j];
            const v4i w = {(int)pack_bf16x2(x[0], x[1]), (int)pack_bf16x2(x[2], x[3]),
                           (int)pack_bf16x2(y[0], y[1]), (int)pack_bf16x2(y[2], y[3])};
            const bool ok = row_ok && n_start + 8 * h + 8 <= t.n_end;
            const uint32_t voff = ok ? (uint32_t)(((long)rl * p.N + n_start + 8 * h) * 2) : kOOB;
            store_b128(rs_d, voff, w);
          }
        }
      }
    } else {
      // 32x32 outputs: the lane holds column m = 32 j + lane % 32 and 16 contiguous
      // weight columns 32 i + 16 (lane / 32) + r of each subtile (weight_row_of_lds).
      const int l32 = lane & 31, g2 = lane >> 5;
#pragma unroll
      for (int j = 0; j < MJ2; ++j) {
        const int rl = wm0 + 32 * j + l32;
        const int m = t.m0 + rl;
        bool row_ok = m < t.row_end;
        if constexpr (VAR == kContig)
          row_ok = row_ok && reinterpret_cast<const int*>(st + Lay::RI_OFF)[rl] == t.g;
#pragma unroll
        for (int i = 0; i < NI2; ++i) {
          const int nl0 = wn0 + 32 * i + 16 * g2;
          const int n_start = t.n0 + nl0;
          const v16f v = acc2[i][j];
          if constexpr (VAR == kKGrouped) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const v4f x = {v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
              if constexpr (ACC) {
                const int pc = (nl0 / 4 + q) ^ (rl % Lay::R_ROW_CHUNKS);
                *reinterpret_cast<v4f*>(R + rl * T::BN * 4 + pc * 16) = x;
                continue;
              }
              const bool ok = row_ok && n_start + 4 * q + 4 <= p.N;
              const uint32_t voff = ok ? (uint32_t)(((long)rl * p.N + n_start + 4 * q) * 4) : kOOB;
              store_b128(rs_d, voff, (v4i){__float_as_int(x[0]), __float_as_int(x[1]),
                                           __float_as_int(x[2]), __float_as_int(x[3])});
            }
          } else {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const v4i w = {(int)pack_bf16x2(v[8 * h + 0], v[8 * h + 1]),
                             (int)pack_bf16x2(v[8 * h + 2], v[8 * h + 3]),
                             (int)pack_bf16x2(v[8 * h + 4], v[8 * h + 5]),
                             (int)pack_bf16x2(v[8 * h + 6], v[8 * h + 7])};
              const bool ok = row_ok && n_start + 8 * h + 8 <= t.n_end;
              const uint32_t voff = ok ? (uint32_t)(((long)rl * p.N + n_start + 8 * h) * 2) : kOOB;
              store_b128(rs_d, voff, w);
            }
          }
        }
      }
    }
  };

  // ---- the pipeline
  long Li = first_tile();
  Issue ic;  // issue cursor
  constexpr bool kPin = !(VAR == kContig && SF == kSfUE8M0);
  ic.t = decode_tile<T, VAR, DT, GRAN, kPin>(Sd, p, Li);
  long Lc = Li;
  TileCtx tc = ic.t;  // compute cursor
  if (!tc.valid) return;
  int si = 0, sc = 0;
  auto advance = [&](TileCtx& t, long& L, int& s) -> bool {
    if (t.valid && ++s >= t.nk) {
      L += grid;
      t = decode_tile<T, VAR, DT, GRAN, kPin>(Sd, p, L);
      s = 0;
      return true;
    }
    return false;
  };
  __syncthreads();  // scheduler scratch in stage memory is dead from here on
  if constexpr (ACC) {
    if (wave >= Lay::EPI0 && wave < Lay::COPY0) {
      accumulate_waves<T, VAR, DT, GRAN, Lay>(Sd, p, smem, tc, Lc, wave - Lay::EPI0, lane);
      return;
    }
  }
  if (wave >= Lay::COPY0) {
    // Copy waves (the last four): one barrier per item, like the MFMA waves. Before
    // barrier j the copies of item j have landed (the younger ones, per_wave(CW) per item
    // for S - 2 items, may still be in flight); after it the stage of item j + S - 1 is
    // free and is refilled. The MFMA waves therefore never wait to enter the memory
    // pipeline. The loop is instantiated per copy wave, so the small copies dealt to a
    // wave and its wait counts are compile-time constants.
    auto copy_loop = [&](auto cw) {
      constexpr int CW = decltype(cw)::value;
      prepare(ic);
#pragma unroll
      for (int k = 0; k < S - 1; ++k) {
        issue(ic, si, k, cw);
        if (advance(ic.t, Li, si)) prepare(ic);
      }
      TileCtx tm = tc;  // mirror of the compute cursor: the same number of barriers
      long Lm = Lc;
      int sm = 0, jt = 0;
      while (true) {
        vm_wait_imm<Lay::per_wave(CW) * (S - 2)>();
        lds_barrier();
        issue(ic, si, (jt + S - 1) % S, cw);
        if (advance(ic.t, Li, si)) prepare(ic);
        advance(tm, Lm, sm);
        if (!tm.valid) break;
        ++jt;
      }
      if constexpr (ACC) lds_barrier();  // the MFMA waves' final exchange barrier
      vm_wait_imm<0>();  // the last (idle) copies land before the workgroup's LDS is released
    };
    switch (cwave) {
      case 0: copy_loop(std::integral_constant<int, 0>{}); break;
      case 1: copy_loop(std::integral_constant<int, 1>{}); break;
      case 2: copy_loop(std::integral_constant<int, 2>{}); break;
      default: copy_loop(std::integral_constant<int, 3>{}); break;
    }
    return;
  }
  // MFMA waves
  int it = 0;
  int rx = 0;  // exchange buffer of the next finished tile (accumulating calls)
  while (true) {
    lds_barrier();
    const int stg = it % S;
    if (sc == 0) {
      if constexpr (FP8) {
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
          for (int j = 0; j < MJ; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};
      } else {
#pragma unroll
        for (int i = 0; i < NI2; ++i)
#pragma unroll
          for (int j = 0; j < MJ2; ++j) acc2[i][j] = (v16f){};
      }
    }
    // a wave whose columns all lie beyond N (the last n-tile of a ragged N) or whose rows
    // all lie at or past the tile's valid rows (the padding of an expert's last m-tile)
    // has nothing to compute: the epilogue stores none of its outputs
    if (ACC || (wn0 < tc.n_end - tc.n0 && tc.m0 + wm0 < tc.row_end)) compute(tc, sc, stg);
    const bool epi = sc == tc.nk - 1;
    if (epi) {
      epilogue(tc, stg, rx);
      rx ^= Lay::R_HALF;
    }
    advance(tc, Lc, sc);
    if (!tc.valid) break;
    ++it;
  }
  if constexpr (ACC) lds_barrier();  // publishes the last tile to the epilogue waves
}

}  // namespace mgg
