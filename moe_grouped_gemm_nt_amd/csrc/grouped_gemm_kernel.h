// grouped_gemm_kernel.h - the persistent grouped NT GEMM kernel template (see
// gemm_engine.h for the design). Included by exactly one translation unit, which
// instantiates it for every (variant, dtype, scale format, weight-scale granularity,
// tile) combination the host dispatcher can pick.
#pragma once

#include "gemm_engine.h"

namespace mgg {

// Everything a workgroup needs to run one output tile. All fields are uniform across
// the workgroup.
struct TileCtx {
  int valid;    // 0 once the workgroup has no more tiles
  int g;        // expert
  int m0, n0;   // first activation row / weight row of the tile
  int nk;       // 128-byte K slices to run (at least 1)
  int k_bytes;  // bytes of K in every operand row (0: nothing to load)
  int a_lim;    // activation rows < a_lim are loaded (others read as zero)
  int row_end;  // masked: valid rows end; contiguous/K-grouped: M
  long a_off;   // byte offset of the expert's activation block
  long b_off;   // byte offset of the expert's weight block
  int lda, ldb; // row strides in bytes
  long sfa_off; // element offset of scale group 0 for row 0
  int sfa_ld;   // elements between consecutive scale groups
  long sfb_off;
  int sfb_ld;
  long d_row0;  // output element offset of row 0 of the expert's output block
};

template <class T, int VAR>
struct Sched {
  // LDS scheduler arrays (allocated after the pipeline stages).
  int* s_a;    // masked: tile prefix [G]; contiguous: block flags/prefix; K-grouped: p_e
  int* s_b;    // masked: clamped counts; contiguous: block experts; K-grouped: usable k_e
  int* s_c;    // contiguous: list of valid blocks
  int* s_tmp;  // scan scratch [256]
  int total;   // number of tiles
  int ntn;     // n tiles per expert
  int mtn;     // K-grouped: m tiles per expert
};

template <class T, int VAR>
__device__ __forceinline__ void sched_init(Sched<T, VAR>& S, const Params& p) {
  const int tid = threadIdx.x;
  S.ntn = (p.N + T::BN - 1) / T::BN;
  if constexpr (VAR == kMasked) {
    for (int g = tid; g < p.G; g += kThreads) {
      int c = p.meta[g];
      c = c < 0 ? 0 : (c > p.rows ? p.rows : c);
      S.s_b[g] = c;
      S.s_a[g] = ((c + T::BM - 1) / T::BM) * S.ntn;
    }
    __syncthreads();
    S.total = block_exclusive_scan(S.s_a, p.G, S.s_tmp);
  } else if constexpr (VAR == kContig) {
    const int nb = (p.rows + kContigBlock - 1) / kContigBlock;
    for (int b = tid; b < nb; b += kThreads) {
      int e = p.meta[(long)b * kContigBlock];
      bool ok = e >= 0 && e < p.G;
      S.s_b[b] = ok ? e : -1;
      S.s_a[b] = ok ? 1 : 0;
    }
    __syncthreads();
    int nvalid = block_exclusive_scan(S.s_a, nb, S.s_tmp);
    for (int b = tid; b < nb; b += kThreads)
      if (S.s_b[b] >= 0) S.s_c[S.s_a[b]] = b;
    __syncthreads();
    S.total = nvalid * (kContigBlock / T::BM) * S.ntn;
  } else {
    S.mtn = (p.rows + T::BM - 1) / T::BM;
    for (int g = tid; g < p.G; g += kThreads) {
      int k = p.meta[g];
      S.s_b[g] = k;
      S.s_a[g] = k > 0 ? k : 0;
    }
    __syncthreads();
    block_exclusive_scan(S.s_a, p.G, S.s_tmp);
    for (int g = tid; g < p.G; g += kThreads) {
      const int k = S.s_b[g];
      const int pe = S.s_a[g];
      bool usable = k >= 0 && (k % p.k_granule) == 0 && (pe % p.k_granule) == 0 &&
                    (long)pe + k <= (long)p.K;
      S.s_b[g] = usable ? k : -1;
    }
    __syncthreads();
    S.total = p.G * S.mtn * S.ntn;
  }
}

// Logical index of the workgroup's first tile; its later tiles follow in steps of the
// grid size. Workgroups are dispatched to the 8 XCDs round-robin (block b runs on XCD
// b % 8); each XCD gets a contiguous range of logical tiles per round so that
// neighbouring tiles (same expert, same weight panel) share that XCD's L2.
__device__ __forceinline__ long logical_tile(int it) {
  const int grid = gridDim.x, b = blockIdx.x;
  if (grid % kXcds != 0) return (long)it * grid + b;
  const int per = grid / kXcds;
  return (long)it * grid + (long)(b % kXcds) * per + b / kXcds;
}

template <class T, int VAR, int DT, int GRAN>
__device__ __forceinline__ TileCtx decode_tile(const Sched<T, VAR>& S, const Params& p, long& L) {
  // Decodes logical tile L; tiles with nothing to do are skipped by advancing L in
  // steps of the grid size (the same workgroup's later tiles), and L is left at the
  // tile returned.
  TileCtx t;
  t.valid = 0;
  constexpr int esz = DT == kFP8 ? 1 : 2;
  const int Kd = p.K;  // masked/contiguous K (elements)
  if constexpr (VAR == kMasked) {
    while (L < S.total) {
      // largest g with prefix[g] <= L
      int lo = 0, hi = p.G - 1;
      while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (S.s_a[mid] <= L) lo = mid; else hi = mid - 1;
      }
      const int g = lo;
      const int c = S.s_b[g];
      const int mt_g = (c + T::BM - 1) / T::BM;
      const int local = (int)(L - S.s_a[g]);
      const int nt = local / mt_g, mt = local % mt_g;
      t.valid = 1;
      t.g = g;
      t.m0 = mt * T::BM;
      t.n0 = nt * T::BN;
      t.k_bytes = Kd * esz;
      t.nk = (t.k_bytes + kSliceBytes - 1) / kSliceBytes;
      t.a_lim = c;
      t.row_end = c;
      t.a_off = (long)g * p.rows * t.k_bytes;
      t.b_off = (long)g * p.N * t.k_bytes;
      t.lda = t.ldb = t.k_bytes;
      const int KB = Kd / 128;
      t.sfa_off = (long)g * KB * p.rows;
      t.sfa_ld = p.rows;
      if constexpr (GRAN == kSfbBlock) {
        t.sfb_off = (long)g * ((p.N + 127) / 128) * KB;
        t.sfb_ld = 1;  // consecutive scale groups of one block are adjacent
      } else {
        t.sfb_off = (long)g * KB * p.N;
        t.sfb_ld = p.N;
      }
      t.d_row0 = (long)g * p.rows * p.N;
      break;
    }
  } else if constexpr (VAR == kContig) {
    constexpr int SUB = kContigBlock / T::BM;
    while (L < S.total) {
      const int nt = (int)(L % S.ntn);
      const long rest = L / S.ntn;
      const int sub = (int)(rest % SUB);
      const int vb = (int)(rest / SUB);
      const int blk = S.s_c[vb];
      const int e = S.s_b[blk];
      const int m0 = blk * kContigBlock + sub * T::BM;
      // A sub-tile that starts on padding is padding throughout (valid rows come first
      // in a block); skip it without loading anything.
      if (m0 >= p.rows || (sub > 0 && p.meta[m0] != e)) { L += gridDim.x; continue; }
      t.valid = 1;
      t.g = e;
      t.m0 = m0;
      t.n0 = nt * T::BN;
      t.k_bytes = Kd * esz;
      t.nk = (t.k_bytes + kSliceBytes - 1) / kSliceBytes;
      t.a_lim = p.rows;
      t.row_end = p.rows;
      t.a_off = 0;
      t.b_off = (long)e * p.N * t.k_bytes;
      t.lda = t.ldb = t.k_bytes;
      const int KB = Kd / 128;
      t.sfa_off = 0;
      t.sfa_ld = p.rows;
      if constexpr (GRAN == kSfbBlock) {
        t.sfb_off = (long)e * ((p.N + 127) / 128) * KB;
        t.sfb_ld = 1;
      } else {
        t.sfb_off = (long)e * KB * p.N;
        t.sfb_ld = p.N;
      }
      t.d_row0 = 0;
      break;
    }
  } else {
    while (L < S.total) {
      const int per = S.mtn * S.ntn;
      const int e = (int)(L / per);
      const int local = (int)(L % per);
      const int k = S.s_b[e];
      if (k < 0 || (k == 0 && p.accumulate)) { L += gridDim.x; continue; }  // nothing to write
      const int nt = local / S.mtn, mt = local % S.mtn;
      const long pe = S.s_a[e];
      t.valid = 1;
      t.g = e;
      t.m0 = mt * T::BM;
      t.n0 = nt * T::BN;
      t.k_bytes = k * esz;
      t.nk = t.k_bytes > 0 ? (t.k_bytes + kSliceBytes - 1) / kSliceBytes : 1;
      t.a_lim = p.rows;
      t.row_end = p.rows;
      t.a_off = (long)p.rows * pe * esz;
      t.b_off = (long)p.N * pe * esz;
      t.lda = t.ldb = t.k_bytes;
      t.sfa_off = (pe / 128) * p.rows;
      t.sfa_ld = p.rows;
      t.sfb_off = (pe / 128) * p.N;
      t.sfb_ld = p.N;
      t.d_row0 = (long)e * p.rows * p.N;
      break;
    }
  }
  return t;
}

// ----------------------------------------------------------------------------- kernel

template <class T, int VAR, int DT, int SF, int GRAN>
struct Layout {
  static constexpr bool FP8 = DT == kFP8;
  static constexpr int A_BYTES = T::BM * kSliceBytes;
  static constexpr int B_BYTES = T::BN * kSliceBytes;
  static constexpr int SA_N = FP8 ? T::BM : 0;
  static constexpr int SB_N = FP8 ? (GRAN == kSfbChannel ? T::BN : (T::BN + 127) / 128) : 0;
  static constexpr int SA_OFF = A_BYTES + B_BYTES;
  static constexpr int SB_OFF = SA_OFF + SA_N * 4;
  static constexpr int STAGE = ((SB_OFF + SB_N * 4) + 15) / 16 * 16;
  static constexpr int PIPE = 2 * STAGE;
};

template <class T, int VAR, int DT, int SF, int GRAN>
__global__ __launch_bounds__(kThreads) void grouped_gemm_kernel(Params p) {
  using Lay = Layout<T, VAR, DT, SF, GRAN>;
  constexpr bool FP8 = Lay::FP8;
  constexpr int NI = T::NI, MJ = T::MJ;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int wave_m = wave / T::WN, wave_n = wave % T::WN;
  const int wm0 = wave_m * T::WTM, wn0 = wave_n * T::WTN;

  // ---- scheduler state in LDS after the two pipeline stages
  Sched<T, VAR> S;
  {
    int* base = reinterpret_cast<int*>(smem + Lay::PIPE);
    S.s_tmp = base;
    base += kThreads;
    const int n = (VAR == kContig) ? (p.rows + kContigBlock - 1) / kContigBlock : p.G;
    S.s_a = base;
    S.s_b = base + n;
    S.s_c = base + 2 * n;
  }
  sched_init<T, VAR>(S, p);

  // ---- per-lane constant LDS offsets of the MFMA fragments (XOR swizzle folded in)
  const int x_lo = ((lg) ^ (lr & 7)) << 4;
  const int x_hi = ((lg + 4) ^ (lr & 7)) << 4;
  int a_row_off[NI];  // weight fragment rows (first MFMA operand)
  int b_row_off[MJ];  // activation fragment rows (second MFMA operand)
#pragma unroll
  for (int i = 0; i < NI; ++i) a_row_off[i] = Lay::A_BYTES + (wn0 + 16 * i + lr) * kSliceBytes;
#pragma unroll
  for (int j = 0; j < MJ; ++j) b_row_off[j] = (wm0 + 16 * j + lr) * kSliceBytes;

  v4f acc[NI][MJ];
  v4i stage_regs[T::CH_PER_THREAD];
  float sa_reg = 0.f, sb_reg = 0.f;

  // Issue the global loads of slice `s` of tile `t` into registers.
  auto load_slice = [&](const TileCtx& t, int s) {
    const int kb0 = s * kSliceBytes;
#pragma unroll
    for (int u = 0; u < T::CH_PER_THREAD; ++u) {
      const int q = tid + u * kThreads;
      v4i v = {0, 0, 0, 0};
      if (q < T::CHUNKS) {
        const int row = q >> 3, c = q & 7;
        const int kb = kb0 + c * 16;
        const bool k_ok = kb + 16 <= t.k_bytes;
        if (row < T::BM) {
          const int m = t.m0 + row;
          if (k_ok && m < t.a_lim)
            v = *reinterpret_cast<const v4i*>(p.A + t.a_off + (long)m * t.lda + kb);
        } else {
          const int n = t.n0 + row - T::BM;
          if (k_ok && n < p.N)
            v = *reinterpret_cast<const v4i*>(p.B + t.b_off + (long)n * t.ldb + kb);
        }
      }
      stage_regs[u] = v;
    }
    if constexpr (FP8) {
      const bool k_ok = t.k_bytes > 0;
      if (tid < T::BM) {
        const int m = t.m0 + tid;
        sa_reg = (k_ok && m < t.a_lim)
                     ? load_scale<SF>(p.SFA, t.sfa_off + (long)s * t.sfa_ld + m) : 0.f;
      }
      if (tid < Lay::SB_N) {
        if constexpr (GRAN == kSfbChannel) {
          const int n = t.n0 + tid;
          sb_reg = (k_ok && n < p.N)
                       ? load_scale<SF>(p.SFB, t.sfb_off + (long)s * t.sfb_ld + n) : 0.f;
        } else {
          const int nb = t.n0 / 128 + tid;
          const int KB = p.K / 128;
          sb_reg = (k_ok && nb * 128 < p.N)
                       ? load_scale<SF>(p.SFB, t.sfb_off + (long)nb * KB + s) : 0.f;
        }
      }
    }
  };

  // Write the staged registers into LDS stage `buf`.
  auto store_slice = [&](int buf) {
    uint8_t* st = smem + buf * Lay::STAGE;
#pragma unroll
    for (int u = 0; u < T::CH_PER_THREAD; ++u) {
      const int q = tid + u * kThreads;
      if (q < T::CHUNKS) {
        const int row = q >> 3, c = q & 7;
        int off;
        if (row < T::BM) off = swz(row, c);
        else off = Lay::A_BYTES + swz(weight_lds_row<T>(row - T::BM), c);
        *reinterpret_cast<v4i*>(st + off) = stage_regs[u];
      }
    }
    if constexpr (FP8) {
      float* sA = reinterpret_cast<float*>(st + Lay::SA_OFF);
      float* sB = reinterpret_cast<float*>(st + Lay::SB_OFF);
      if (tid < T::BM) sA[tid] = sa_reg;
      if (tid < Lay::SB_N) sB[tid] = sb_reg;
    }
  };

  // MFMA work of one slice held in LDS stage `buf`.
  auto compute_slice = [&](int buf) {
    const uint8_t* st = smem + buf * Lay::STAGE;
    if constexpr (FP8) {
      const float* sA = reinterpret_cast<const float*>(st + Lay::SA_OFF);
      const float* sB = reinterpret_cast<const float*>(st + Lay::SB_OFF);
      v8i bfr[MJ];
      float sa[MJ];
#pragma unroll
      for (int j = 0; j < MJ; ++j) {
        v4i lo = *reinterpret_cast<const v4i*>(st + b_row_off[j] + x_lo);
        v4i hi = *reinterpret_cast<const v4i*>(st + b_row_off[j] + x_hi);
        bfr[j] = (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        sa[j] = sA[wm0 + 16 * j + lr];
      }
      float sbw = 0.f;
      if constexpr (GRAN == kSfbBlock) sbw = sB[wn0 / 128];
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        v4i lo = *reinterpret_cast<const v4i*>(st + a_row_off[i] + x_lo);
        v4i hi = *reinterpret_cast<const v4i*>(st + a_row_off[i] + x_hi);
        v8i afr = (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        v4f sbv = {sbw, sbw, sbw, sbw};
        if constexpr (GRAN == kSfbChannel)
          sbv = *reinterpret_cast<const v4f*>(sB + wn0 + lg * 4 * NI + 4 * i);
#pragma unroll
        for (int j = 0; j < MJ; ++j) {
          const v4f zero = {0.f, 0.f, 0.f, 0.f};
          // format 0 = FP8 E4M3 for both operands; scale exponent 127 = 2^0
          v4f part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(afr, bfr[j], zero, 0, 0,
                                                                       0, 127, 0, 127);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(part[r], sa[j] * sbv[r], acc[i][j][r]);
        }
      }
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int xo = h ? x_hi : x_lo;
        v8bf bfr[MJ];
#pragma unroll
        for (int j = 0; j < MJ; ++j) bfr[j] = *reinterpret_cast<const v8bf*>(st + b_row_off[j] + xo);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          v8bf afr = *reinterpret_cast<const v8bf*>(st + a_row_off[i] + xo);
#pragma unroll
          for (int j = 0; j < MJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, bfr[j], acc[i][j], 0, 0, 0);
        }
      }
    }
  };

  // Row-masked store of the finished tile.
  auto epilogue = [&](const TileCtx& t) {
#pragma unroll
    for (int j = 0; j < MJ; ++j) {
      const int m = t.m0 + wm0 + 16 * j + lr;
      bool row_ok = m < t.row_end;
      if constexpr (VAR == kContig) row_ok = row_ok && p.meta[m] == t.g;
      const int n_start = t.n0 + wn0 + lg * 4 * NI;
      if (!row_ok) continue;
      if constexpr (VAR == kKGrouped) {
        float* drow = reinterpret_cast<float*>(p.D) + t.d_row0 + (long)m * p.N + n_start;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          if (n_start + 4 * i + 4 <= p.N) {
            v4f v = acc[i][j];
            if (p.accumulate) v += *reinterpret_cast<const v4f*>(drow + 4 * i);
            *reinterpret_cast<v4f*>(drow + 4 * i) = v;
          }
        }
      } else {
        uint16_t* drow = reinterpret_cast<uint16_t*>(p.D) + t.d_row0 + (long)m * p.N + n_start;
#pragma unroll
        for (int h = 0; h < NI / 2; ++h) {
          if (n_start + 8 * h + 8 <= p.N) {
            const v4f x = acc[2 * h][j], y = acc[2 * h + 1][j];
            v4i w = {(int)pack_bf16x2(x[0], x[1]), (int)pack_bf16x2(x[2], x[3]),
                     (int)pack_bf16x2(y[0], y[1]), (int)pack_bf16x2(y[2], y[3])};
            *reinterpret_cast<v4i*>(drow + 8 * h) = w;
          }
        }
      }
    }
  };

  // ---- flat pipeline over (tile, slice) work items: the loads of the next item (which
  // may belong to the next tile) are in flight while the current one computes.
  const int grid = gridDim.x;
  long L = logical_tile(0);
  TileCtx cur = decode_tile<T, VAR, DT, GRAN>(S, p, L);
  if (!cur.valid) return;
  int s = 0;
  load_slice(cur, 0);
  store_slice(0);
  __syncthreads();
  int buf = 0;
  while (true) {
    TileCtx nxt = cur;
    int ns = s + 1;
    long Ln = L;
    if (ns >= cur.nk) {
      Ln = L + grid;
      nxt = decode_tile<T, VAR, DT, GRAN>(S, p, Ln);
      ns = 0;
    }
    if (nxt.valid) load_slice(nxt, ns);
    if (s == 0) {
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < MJ; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};
    }
    compute_slice(buf);
    if (s == cur.nk - 1) epilogue(cur);
    if (!nxt.valid) break;
    store_slice(buf ^ 1);
    __syncthreads();
    buf ^= 1;
    cur = nxt;
    L = Ln;
    s = ns;
  }
}

}  // namespace mgg
