// gemm_engine.h - the gfx950 grouped NT GEMM engine shared by the masked, contiguous
// and K-grouped entry points.
//
// One persistent kernel per call. Each workgroup (256 lanes = 4 wave64s):
//   1. reads the device-side routing (masked counts, contiguous row indices, K-grouped
//      token counts) into LDS and builds the tile prefix there, so nothing about the
//      expert distribution is baked into the launch (a captured hipGraph replays
//      correctly with new routing values);
//   2. walks its share of the (expert, m-tile, n-tile) list with an XCD-aware order;
//   3. per tile, streams 128-byte K slices of the activation rows and weight rows
//      through double-buffered, XOR-swizzled LDS with coalesced 16-byte loads and
//      feeds MFMA 16x16 instructions (FP8: 16x16x128 f8f6f4, one instruction per 128-K
//      scale group; BF16: 16x16x32 bf16);
//   4. FP8 only: promotes each 128-K partial sum into the FP32 accumulator with the
//      row scale times the weight scale (per-128-K promotion in registers);
//   5. stores rows under a per-row mask: a tile never writes past its expert's valid
//      rows, padding rows or another expert's rows.
//
// Operand roles. The MFMA's first operand is fed with WEIGHT rows (n) and its second
// with ACTIVATION rows (m), so each lane ends up holding 4 consecutive n of one m; the
// weight rows of a wave are further permuted so that one lane holds 4*NI consecutive
// n, which turns the epilogue into full 16-byte row-contiguous stores.
//
// K order. Inside one MFMA the K elements a lane supplies may be any fixed permutation
// as long as both operands use the same one; lanes 16g..16g+15 supply the 16-byte K
// chunks g and g+4 of each 128-byte slice. Across slices K ascends. The layout, the
// instruction and the promotion formula do not depend on the tile shape, so every
// tile configuration produces the same bits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mgg {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

enum Variant { kMasked = 0, kContig = 1, kKGrouped = 2 };
enum DType { kBF16 = 0, kFP8 = 1 };
enum SfFmt { kSfF32 = 0, kSfUE8M0 = 1 };
enum SfbGran { kSfbBlock = 0, kSfbChannel = 1 };

constexpr int kThreads = 256;
constexpr int kSliceBytes = 128;  // K bytes per row per pipeline stage
constexpr int kXcds = 8;          // MI355X: 8 accelerator dies, WGs dispatched round-robin
constexpr int kContigBlock = 128; // rows per contiguous-layout alignment block
constexpr int kMaxExperts = 4096;
constexpr int kMaxContigBlocks = 4096;

struct Params {
  const uint8_t* A;
  const uint8_t* B;
  const void* SFA;
  const void* SFB;
  void* D;
  const int32_t* meta;  // masked counts / contiguous row indices / K-grouped token counts
  int G;
  int rows;     // masked: capacity; contiguous and K-grouped: M
  int N;
  int K;        // masked, contiguous: K; K-grouped: K_total
  int accumulate;  // K-grouped: 1 adds the product to D
  int k_granule;   // K-grouped: required multiple of k_e (128 FP8, 8 BF16)
};

// Tile configuration: BM activation rows x BN weight rows per workgroup; 4 waves laid
// out WM (along m) x WN (along n).
template <int BM_, int BN_, int WM_, int WN_>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static_assert(WM * WN == 4, "four waves per workgroup");
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int MJ = WTM / 16, NI = WTN / 16;
  static_assert(MJ >= 1 && NI >= 1 && WTM % 16 == 0 && WTN % 16 == 0, "16x16 subtiles");
  static_assert(WTN <= 128 && 128 % WTN == 0, "a wave's n range stays in one 128-row block");
  static constexpr int CHUNKS = (BM + BN) * (kSliceBytes / 16);
  static constexpr int CH_PER_THREAD = (CHUNKS + kThreads - 1) / kThreads;
};

// ----------------------------------------------------------------------------- helpers

__device__ __forceinline__ float ue8m0_to_float(uint32_t u) {
  // 2^(u-127); u == 0 is the subnormal 2^-127; u == 255 is NaN.
  uint32_t bits = (u == 0) ? 0x00400000u : (u == 255 ? 0x7fc00000u : (u << 23));
  return __uint_as_float(bits);
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;  // NaN stays a quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

template <int SF>
__device__ __forceinline__ float load_scale(const void* base, long idx) {
  if constexpr (SF == kSfF32) {
    return reinterpret_cast<const float*>(base)[idx];
  } else {
    return ue8m0_to_float(reinterpret_cast<const uint8_t*>(base)[idx]);
  }
}

// Exclusive scan of `n` ints held in LDS `buf` (in place), block-wide; returns the total.
// Every thread of the block must call it.
__device__ int block_exclusive_scan(int* buf, int n, int* s_tmp) {
  const int tid = threadIdx.x;
  const int per = (n + kThreads - 1) / kThreads;
  const int lo = tid * per;
  const int hi = min(lo + per, n);
  int local = 0;
  for (int i = lo; i < hi; ++i) local += buf[i];
  s_tmp[tid] = local;
  __syncthreads();
  // Hillis-Steele inclusive scan over the 256 partial sums.
  for (int off = 1; off < kThreads; off <<= 1) {
    int v = (tid >= off) ? s_tmp[tid - off] : 0;
    __syncthreads();
    s_tmp[tid] += v;
    __syncthreads();
  }
  int run = s_tmp[tid] - local;  // exclusive prefix of this thread's range
  for (int i = lo; i < hi; ++i) {
    int v = buf[i];
    buf[i] = run;
    run += v;
  }
  int total = s_tmp[kThreads - 1];
  __syncthreads();
  return total;
}

// LDS row (within the weight tile) that holds tile-local weight row n. A wave's WTN
// rows are reordered so that MFMA subtile i reads 16 consecutive LDS rows while lane
// group q's outputs cover the contiguous n range [q*4*NI, (q+1)*4*NI) of the wave.
template <class T>
__device__ __forceinline__ int weight_lds_row(int n) {
  const int w = n / T::WTN, nl = n % T::WTN;
  const int q = nl / (4 * T::NI), rem = nl % (4 * T::NI);
  const int i = rem / 4, r = rem % 4;
  return w * T::WTN + 16 * i + 4 * q + r;
}

// Byte offset of (row, 16-byte chunk c) in a tile of 128-byte rows, XOR-swizzled so
// that 8 consecutive rows read at the same logical chunk hit 8 different bank groups.
__device__ __forceinline__ int swz(int row, int c) {
  return row * kSliceBytes + ((c ^ (row & 7)) << 4);
}

}  // namespace mgg
