// grouped_gemm.hip - host side of the C ABI declared in include/moe_grouped_gemm_nt.h:
// argument validation, tile-shape choice, grid sizing and kernel launch.
//
// The host never touches device data: the grid is sized from static shapes (experts,
// capacity or rows, N) and the CU count, and every workgroup reads the routing
// buffers itself, so a call captured into a hipGraph stays correct when the routing
// values change between replays.

#include <map>
#include <mutex>
#include <type_traits>
#include <string>
#include <unordered_map>
#include <utility>

#include "grouped_gemm_kernel.h"
#include "moe_grouped_gemm_nt.h"

using namespace mgg;

namespace {

thread_local std::string g_last_error;

mgg_status fail(mgg_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

// Tile shapes (BM activation rows x BN weight rows, 4 waves, S pipeline stages). The
// small-M shapes keep MFMA work proportional to the valid rows and put more
// workgroups on the weight stream when experts receive few tokens; all of them
// produce bitwise-identical results.
// FP8, <= 32 rows per expert; three stages (four measured 19 % slower on 32 experts of ~20
// rows with N = 1536, K = 2048, two 50 % slower)
using TileS8 = Tile<32, 64, 2, 2, 3>;
using TileS16 = Tile<32, 128, 1, 4, 4>;  // BF16 (32x32 subtiles), <= 32 rows per expert
using TileM = Tile<64, 128, 2, 2, 3>;    // <= 64 rows
using TileL = Tile<128, 256, 2, 2, 3>;   // larger experts, BF16
// larger experts, FP8 activations: eight MFMA waves of 64 x 64 (measured 13 % faster on
// the K = 256 contiguous shape, whose tiles are mostly epilogue, and 2-4 % on the
// MFMA-bound 6 x 4096 x 4096 shape; BF16 is better served by four)
using TileL8 = Tile<128, 256, 2, 4, 3>;
// ... except masked FP8 calls with 129-256 rows per expert (two m-tiles, the second partly
// padding, and a weight stream that sets the time): there four MFMA waves of 64 x 128 (the
// BF16 tile's shape) measured 3 % faster on the 32-expert N = 6144, K = 7168 shape, and
// 3-6 % slower on the 6-expert, FP4-weight and contiguous shapes (interleaved A/B runs)
// the fused SwiGLU tile: 128 output columns (their gate and up weight rows), eight waves
// of 16 rows x all 256 weight rows; the two-stage form takes over when the row-block table
// of a long contiguous layout (beyond ~2900 blocks) no longer fits next to three stages
using TileSwi = Tile<128, 256, 8, 1, 3, true>;
using TileSwi2 = Tile<128, 256, 8, 1, 2, true>;
using TileK = Tile<64, 128, 2, 2, 3>;    // K-grouped output tiles
template <class T>  // the same tile with streaming weight copies
using Streamed = Tile<T::BM, T::BN, T::WM, T::WN, T::S, T::SWI, true>;
// The 32-row tile of a dtype, and the 128x256 tile of a variant: contiguous FP8 calls with
// float32 per-channel weight scales take the four-wave tile (with eight waves they need
// more than the 168 registers three waves per SIMD leave).
template <int DT>
using SmallTile = std::conditional_t<DT == kBF16, TileS16, TileS8>;
template <int VAR, int DT, int SF, int GRAN>
using LargeTile = std::conditional_t<DT == kBF16 || (VAR == kContig && DT == kFP8 &&
                                                     SF == kSfF32 && GRAN == kSfbChannel),
                                     TileL, TileL8>;

enum TileId { kTileS = 0, kTileM = 1, kTileL = 2, kTileL4 = 3 };

struct DevInfo {
  int id = 0;
  int cus = 0;
};

std::mutex g_mu;
std::unordered_map<int, DevInfo> g_dev;
// (device, kernel) -> resident workgroups per CU; the LDS limit attribute is set once per
// pair, with that device current
std::map<std::pair<int, const void*>, int> g_occ;

bool dev_info(DevInfo* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  std::lock_guard<std::mutex> lk(g_mu);
  auto it = g_dev.find(dev);
  if (it != g_dev.end()) {
    *out = it->second;
    return true;
  }
  DevInfo d;
  d.id = dev;
  if (hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return false;
  g_dev[dev] = d;
  *out = d;
  return true;
}

long cdiv(long a, long b) { return (a + b - 1) / b; }

// Bytes of the weight operand of an M-grouped call ([G][N][K] elements), and the size from
// which a masked call whose experts fit one small m-tile streams its weights (below it the
// weights stay cache-resident from call to call, and the hint only costs).
long weight_bytes(mgg_dtype dt, int G, int N, int K) {
  const long e = (long)G * N * K;
  return dt == MGG_BF16 ? 2 * e : dt == MGG_FP8_FP4 ? e / 2 : e;
}
constexpr long kStreamWeightBytes = 64L << 20;

// Bytes the scheduler keeps in LDS after the pipeline stages, and the transient scan
// scratch it needs inside the stages.
template <int VAR>
void sched_bytes(const Params& p, long* persistent, long* transient) {
  if (VAR == kContig) {
    const long nb = cdiv(p.rows, kContigBlock);
    *persistent = nb * 4;
    *transient = (kThreads + 2 * nb) * 4;
  } else if (VAR == kKGrouped) {
    *persistent = (p.G + 1L) * 4;         // token prefixes and their total
    *transient = (kThreads + p.G) * 4L;  // scan scratch, clamped counts
  } else {
    *persistent = (VAR == kPsum ? 3L : 2L) * p.G * 4;
    *transient = kThreads * 4;
  }
}

template <class T, int VAR, int DT, int SF, int GRAN, bool ACC>
long lds_bytes(const Params& p) {
  long pers, trans;
  sched_bytes<VAR>(p, &pers, &trans);
  using Lay = Layout<T, VAR, DT, SF, GRAN, ACC>;
  if (trans > Lay::PIPE) return 1L << 40;
  return Lay::SCHED_OFF + pers;
}

template <class T, int VAR, int DT, int SF, int GRAN, bool ACC>
mgg_status launch(const Params& p, long max_tiles, hipStream_t stream) {
  auto kern = grouped_gemm_kernel<T, VAR, DT, SF, GRAN, ACC>;
  using Lay = Layout<T, VAR, DT, SF, GRAN, ACC>;
  const long lds = lds_bytes<T, VAR, DT, SF, GRAN, ACC>(p);
  if (lds > kLdsBytes)
    return fail(MGG_EUNSUPPORTED, "too many experts or row blocks for the LDS scheduler");
  DevInfo dev;
  if (!dev_info(&dev)) return fail(MGG_EHIP, "hipGetDevice/hipDeviceGetAttribute failed");
  int occ = 1;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    const std::pair<int, const void*> key(dev.id, (const void*)kern);
    auto it = g_occ.find(key);
    if (it == g_occ.end()) {
      if (hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                              kLdsBytes) != hipSuccess)
        return fail(MGG_EHIP, "hipFuncSetAttribute failed");
      // Residency at the pipeline's own footprint plus a typical scheduler table.
      int o = 0;
      const size_t lds_typ = (size_t)Lay::SCHED_OFF + 4096;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, kern, Lay::NT, lds_typ) !=
              hipSuccess || o < 1)
        o = 1;
      g_occ[key] = o;
      occ = o;
    } else {
      occ = it->second;
    }
  }
  const long resident = (long)dev.cus * occ;
  long grid = max_tiles < resident ? max_tiles : resident;
  if (grid >= kXcds) grid -= grid % kXcds;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(Lay::NT), (size_t)lds, stream, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MGG_EHIP, std::string("kernel launch: ") + hipGetErrorString(e));
  return MGG_OK;
}

template <class T, int VAR>
long m_tiles(const Params& p) {
  const long ntn = cdiv(p.N, T::BN);
  if (VAR == kMasked) return (long)p.G * cdiv(p.rows, T::BM) * ntn;
  if (VAR == kPsum) return (cdiv(p.rows, T::BM) + p.G) * ntn;  // one ragged tile per expert
  return cdiv(p.rows, kContigBlock) * (kContigBlock / T::BM) * ntn;
}

template <int VAR, int DT, int SF, int GRAN>
mgg_status launch_tile(TileId tile, const Params& p, hipStream_t s, bool stream_w) {
  // Calls that read every weight panel once stream their weight copies (stream_w, chosen
  // by the entry point): masked calls whose experts fit in one 32- or 64-row m-tile and
  // whose weights are large, and contiguous calls with at most 512 bytes of K (w2-like:
  // each expert's one or two m-tiles read their panel over a few slices while the output
  // writes are as large as the weight reads).
  if constexpr (VAR == kContig) {
    if (stream_w) {
      if (tile == kTileL4) tile = kTileL;
      using TLg = LargeTile<VAR, DT, SF, GRAN>;
      using TS = SmallTile<DT>;
      if (tile == kTileL && lds_bytes<TLg, VAR, DT, SF, GRAN, false>(p) > kLdsBytes) tile = kTileM;
      switch (tile) {
        case kTileS: return launch<Streamed<TS>, VAR, DT, SF, GRAN, false>(p, m_tiles<TS, VAR>(p), s);
        case kTileM: return launch<Streamed<TileM>, VAR, DT, SF, GRAN, false>(p, m_tiles<TileM, VAR>(p), s);
        default: return launch<Streamed<TLg>, VAR, DT, SF, GRAN, false>(p, m_tiles<TLg, VAR>(p), s);
      }
    }
  }
  if constexpr (VAR == kMasked) {
    if (stream_w && tile == kTileS) {
      using TS = SmallTile<DT>;
      return launch<Streamed<TS>, VAR, DT, SF, GRAN, false>(p, m_tiles<TS, VAR>(p), s);
    }
    if (stream_w && tile == kTileM)
      return launch<Streamed<TileM>, VAR, DT, SF, GRAN, false>(p, m_tiles<TileM, VAR>(p), s);
  }
  if constexpr (VAR == kMasked && DT == kFP8) {
    if (tile == kTileL4 && lds_bytes<TileL, VAR, DT, SF, GRAN, false>(p) <= kLdsBytes)
      return launch<TileL, VAR, DT, SF, GRAN, false>(p, m_tiles<TileL, VAR>(p), s);
  }
  if (tile == kTileL4) tile = kTileL;
  // The largest tile needs the most LDS; fall back to the middle one when the
  // scheduler table does not fit next to it.
  using TileLg = LargeTile<VAR, DT, SF, GRAN>;
  if (tile == kTileL && lds_bytes<TileLg, VAR, DT, SF, GRAN, false>(p) > kLdsBytes) tile = kTileM;
  using TileS = SmallTile<DT>;
  switch (tile) {
    case kTileS: return launch<TileS, VAR, DT, SF, GRAN, false>(p, m_tiles<TileS, VAR>(p), s);
    case kTileM: return launch<TileM, VAR, DT, SF, GRAN, false>(p, m_tiles<TileM, VAR>(p), s);
    default: return launch<TileLg, VAR, DT, SF, GRAN, false>(p, m_tiles<TileLg, VAR>(p), s);
  }
}

// Dispatch over the compile-time parameters of the M-grouped variants.
template <int VAR>
mgg_status dispatch_m(mgg_dtype dt, mgg_sf_fmt sf, mgg_sfb_gran gran, TileId tile, bool stream_w,
                      const Params& p, hipStream_t s) {
  if (dt == MGG_BF16) return launch_tile<VAR, kBF16, kSfF32, kSfbBlock>(tile, p, s, stream_w);
  if (dt == MGG_FP8_FP4) return launch_tile<VAR, kFP4W, kSfUE8M0, kSfbBlock32>(tile, p, s, stream_w);
  if (sf == MGG_SF_F32) {
    if (gran == MGG_SFB_BLOCK128) return launch_tile<VAR, kFP8, kSfF32, kSfbBlock>(tile, p, s, stream_w);
    return launch_tile<VAR, kFP8, kSfF32, kSfbChannel>(tile, p, s, stream_w);
  }
  if (gran == MGG_SFB_BLOCK128) return launch_tile<VAR, kFP8, kSfUE8M0, kSfbBlock>(tile, p, s, stream_w);
  return launch_tile<VAR, kFP8, kSfUE8M0, kSfbChannel>(tile, p, s, stream_w);
}

// The fused SwiGLU tile with three stages, or with two when the contiguous layout's
// row-block table does not fit next to three (the bits are the same either way).
template <int DT, int SF, int GRAN>
mgg_status launch_swi(const Params& p, hipStream_t s) {
  if (lds_bytes<TileSwi, kContig, DT, SF, GRAN, false>(p) <= kLdsBytes)
    return launch<TileSwi, kContig, DT, SF, GRAN, false>(p, m_tiles<TileSwi, kContig>(p), s);
  return launch<TileSwi2, kContig, DT, SF, GRAN, false>(p, m_tiles<TileSwi2, kContig>(p), s);
}

TileId pick_tile(int expected_m, int fallback) {
  const int em = expected_m > 0 ? expected_m : fallback;
  if (em <= 32) return kTileS;
  if (em <= 64) return kTileM;
  return kTileL;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// Every buffer resource the kernels address must be below 2 GiB so that a 32-bit
// out-of-range offset can mask a lane. Operand and output resources start at a tile's
// first row, so the limit applies to one tile's rows (at most kTileRowsA activation or
// output rows, kTileRowsB weight rows; the fused SwiGLU tile gathers its weight rows from
// the whole expert), while scale and routing tensors are addressed whole.
constexpr long kMaxBuffer = (1L << 31) - 1;
constexpr long kTileRowsA = 128;
constexpr long kTileRowsB = 256;

uint32_t scale_bytes(long count, mgg_sf_fmt sf) {
  // UE8M0 buffers are read in whole dwords: the caller's allocation must be readable up
  // to the next multiple of 4 bytes.
  return (uint32_t)(sf == MGG_SF_F32 ? count * 4 : (count + 3) / 4 * 4);
}

mgg_status check_common(mgg_dtype dt, int N, int K, const void* A, const void* SFA,
                        const void* B, const void* SFB, mgg_sf_fmt sf, const void* D,
                        const void* meta) {
  if (dt != MGG_BF16 && dt != MGG_FP8_E4M3 && dt != MGG_FP8_FP4)
    return fail(MGG_EINVAL, "unknown dtype");
  if (N < 1 || N % 8 != 0) return fail(MGG_EINVAL, "N must be a positive multiple of 8");
  if (K < 1) return fail(MGG_EINVAL, "K must be positive");
  if (dt == MGG_BF16 && K % 8 != 0) return fail(MGG_EINVAL, "BF16 needs K % 8 == 0");
  if (dt != MGG_BF16 && K % 128 != 0) return fail(MGG_EINVAL, "FP8 needs K % 128 == 0");
  if (K > (1 << 28)) return fail(MGG_EUNSUPPORTED, "K too large");
  if (!A || !B || !D || !meta) return fail(MGG_EINVAL, "null pointer");
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(D, 16))
    return fail(MGG_EINVAL, "A, B and D must be 16-byte aligned");
  if (dt != MGG_BF16) {
    if (!SFA || !SFB) return fail(MGG_EINVAL, "FP8 needs SFA and SFB");
    if (sf != MGG_SF_F32 && sf != MGG_SF_UE8M0) return fail(MGG_EINVAL, "unknown scale format");
    if (!aligned(SFA, 4) || !aligned(SFB, 4)) return fail(MGG_EINVAL, "scales must be 4-byte aligned");
    if (dt == MGG_FP8_FP4 && sf != MGG_SF_UE8M0)
      return fail(MGG_EUNSUPPORTED, "FP8 x FP4 takes UE8M0 scales");
  }
  if (!aligned(meta, 4)) return fail(MGG_EINVAL, "routing buffer must be 4-byte aligned");
  return MGG_OK;
}

// Weight-scale entries of an M-grouped call and weight bytes per row, after checking
// that the weight-scale granularity fits the element type.
mgg_status weight_layout(mgg_dtype dt, mgg_sfb_gran gran, long G, long N, long K, long* sfb_n,
                         long* b_row) {
  const long KB = K / 128, NB = cdiv(N, 128);
  *b_row = dt == MGG_BF16 ? 2 * K : (dt == MGG_FP8_FP4 ? K / 2 : K);
  *sfb_n = 0;
  if (dt == MGG_FP8_E4M3) {
    if (gran == MGG_SFB_BLOCK128) *sfb_n = G * NB * KB;
    else if (gran == MGG_SFB_CHANNEL) *sfb_n = G * KB * N;
    else return fail(MGG_EINVAL, "unknown weight-scale granularity");
  } else if (dt == MGG_FP8_FP4) {
    if (gran != MGG_SFB_BLOCK32) return fail(MGG_EINVAL, "FP4 weights take MGG_SFB_BLOCK32 scales");
    *sfb_n = G * KB * N * 4;
  }
  return MGG_OK;
}

mgg_status check_sizes(std::initializer_list<long> sizes) {
  for (long s : sizes)
    if (s > kMaxBuffer) return fail(MGG_EUNSUPPORTED, "an operand block exceeds 2 GiB");
  return MGG_OK;
}

}  // namespace

namespace {
mgg_status kgrouped_impl(mgg_dtype dt, int G, int M, int N, int K_total, const void* A,
                         const void* SFA, const void* B, const void* SFB, mgg_sf_fmt sf,
                         float* D, const int32_t* ks, int accumulate, int meta_psum,
                         hipStream_t stream);
}  // namespace

extern "C" {

const char* mgg_status_string(mgg_status s) {
  switch (s) {
    case MGG_OK: return "ok";
    case MGG_EINVAL: return "invalid argument";
    case MGG_EUNSUPPORTED: return "unsupported argument combination";
    case MGG_EHIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* mgg_last_error(void) { return g_last_error.c_str(); }

mgg_status quantize_fp8_1x128_impl(int M, int K, const void* X, void* Q, void* SF,
                                   mgg_sf_fmt sf, float sf_zero, hipStream_t stream,
                                   const char** err) __attribute__((visibility("hidden")));

mgg_status quantize_fp8_1x128(int M, int K, const void* X, void* Q, void* SF, mgg_sf_fmt sf,
                              float sf_zero, hipStream_t stream) {
  g_last_error.clear();
  const char* err = "";
  const mgg_status st = quantize_fp8_1x128_impl(M, K, X, Q, SF, sf, sf_zero, stream, &err);
  if (st != MGG_OK) return fail(st, err);
  return MGG_OK;
}

mgg_status swiglu_quant_fp8_1x128_impl(int M, int I, const void* H, void* Q, void* SF,
                                       mgg_sf_fmt sf, float sf_zero, hipStream_t stream,
                                       const char** err) __attribute__((visibility("hidden")));

mgg_status swiglu_quant_fp8_1x128(int M, int I, const void* H, void* Q, void* SF,
                                  mgg_sf_fmt sf, float sf_zero, hipStream_t stream) {
  g_last_error.clear();
  const char* err = "";
  const mgg_status st = swiglu_quant_fp8_1x128_impl(M, I, H, Q, SF, sf, sf_zero, stream, &err);
  if (st != MGG_OK) return fail(st, err);
  return MGG_OK;
}

mgg_status grouped_gemm_masked(mgg_dtype dt, int G, int cap, int N, int K, const void* A,
                               const void* SFA, const void* B, const void* SFB,
                               mgg_sf_fmt sf, mgg_sfb_gran gran, void* D,
                               const int32_t* masked_m, int expected_m, hipStream_t stream) {
  g_last_error.clear();
  mgg_status st = check_common(dt, N, K, A, SFA, B, SFB, sf, D, masked_m);
  if (st != MGG_OK) return st;
  if (G < 1 || G > kMaxExperts) return fail(MGG_EINVAL, "G must be in [1, 4096]");
  if (cap < 1) return fail(MGG_EINVAL, "cap must be positive");
  long sfb_n, b_row;
  st = weight_layout(dt, gran, G, N, K, &sfb_n, &b_row);
  if (st != MGG_OK) return st;
  const long esz = dt == MGG_BF16 ? 2 : 1, KB = K / 128;
  const long sfa_n = (long)G * KB * cap;
  st = check_sizes({kTileRowsA * K * esz, kTileRowsB * b_row, kTileRowsA * N * 2, sfa_n * 4,
                    sfb_n * 4, (long)G * cdiv(cap, 32) * cdiv(N, 64)});
  if (st != MGG_OK) return st;
  Params p{};
  p.A = (const uint8_t*)A;
  p.B = (const uint8_t*)B;
  p.SFA = SFA;
  p.SFB = SFB;
  p.D = D;
  p.meta = masked_m;
  p.G = G;
  p.rows = cap;
  p.N = N;
  p.K = K;
  p.sfa_bytes = dt != MGG_BF16 ? scale_bytes(sfa_n, sf) : 0;
  p.sfb_bytes = dt != MGG_BF16 ? scale_bytes(sfb_n, sf) : 0;
  p.meta_bytes = (uint32_t)G * 4;
  TileId tile = pick_tile(expected_m, cap);
  if (tile == kTileL && expected_m > 128 && expected_m <= 256) tile = kTileL4;
  return dispatch_m<kMasked>(dt, sf, gran, tile, weight_bytes(dt, G, N, K) >= kStreamWeightBytes,
                            p, stream);
}

mgg_status grouped_gemm_contiguous(mgg_dtype dt, int G, int M, int N, int K, const void* A,
                                   const void* SFA, const void* B, const void* SFB,
                                   mgg_sf_fmt sf, mgg_sfb_gran gran, void* D,
                                   const int32_t* m_indices, int expected_m,
                                   hipStream_t stream) {
  g_last_error.clear();
  mgg_status st = check_common(dt, N, K, A, SFA, B, SFB, sf, D, m_indices);
  if (st != MGG_OK) return st;
  if (G < 1 || G > kMaxExperts) return fail(MGG_EINVAL, "G must be in [1, 4096]");
  if (M < 1 || M > kMaxContigBlocks * kContigBlock)
    return fail(M < 1 ? MGG_EINVAL : MGG_EUNSUPPORTED, "M must be in [1, 524288]");
  long sfb_n, b_row;
  st = weight_layout(dt, gran, G, N, K, &sfb_n, &b_row);
  if (st != MGG_OK) return st;
  const long esz = dt == MGG_BF16 ? 2 : 1, KB = K / 128;
  const long sfa_n = KB * M;
  st = check_sizes({kTileRowsA * K * esz, kTileRowsB * b_row, kTileRowsA * N * 2, sfa_n * 4,
                    sfb_n * 4});
  if (st != MGG_OK) return st;
  Params p{};
  p.A = (const uint8_t*)A;
  p.B = (const uint8_t*)B;
  p.SFA = SFA;
  p.SFB = SFB;
  p.D = D;
  p.meta = m_indices;
  p.G = G;
  p.rows = M;
  p.N = N;
  p.K = K;
  p.sfa_bytes = dt != MGG_BF16 ? scale_bytes(sfa_n, sf) : 0;
  p.sfb_bytes = dt != MGG_BF16 ? scale_bytes(sfb_n, sf) : 0;
  p.meta_bytes = (uint32_t)M * 4;
  const bool short_k = (long)K * (dt == MGG_BF16 ? 2 : 1) <= 512;
  return dispatch_m<kContig>(dt, sf, gran, pick_tile(expected_m, kContigBlock), short_k, p,
                             stream);
}

mgg_status grouped_gemm_contiguous_psum(mgg_dtype dt, int G, int M, int N, int K,
                                        const void* A, const void* SFA, const void* B,
                                        const void* SFB, mgg_sf_fmt sf, mgg_sfb_gran gran,
                                        void* D, const int32_t* psum, int expected_m,
                                        hipStream_t stream) {
  g_last_error.clear();
  mgg_status st = check_common(dt, N, K, A, SFA, B, SFB, sf, D, psum);
  if (st != MGG_OK) return st;
  if (G < 1 || G > kMaxExperts) return fail(MGG_EINVAL, "G must be in [1, 4096]");
  if (M < 1) return fail(MGG_EINVAL, "M must be positive");
  long sfb_n, b_row;
  st = weight_layout(dt, gran, G, N, K, &sfb_n, &b_row);
  if (st != MGG_OK) return st;
  const long esz = dt == MGG_BF16 ? 2 : 1, KB = K / 128;
  const long sfa_n = KB * M;
  st = check_sizes({kTileRowsA * K * esz, kTileRowsB * b_row, kTileRowsA * N * 2, sfa_n * 4,
                    sfb_n * 4, (cdiv(M, 32) + G) * cdiv(N, 64)});
  if (st != MGG_OK) return st;
  Params p{};
  p.A = (const uint8_t*)A;
  p.B = (const uint8_t*)B;
  p.SFA = SFA;
  p.SFB = SFB;
  p.D = D;
  p.meta = psum;
  p.G = G;
  p.rows = M;
  p.N = N;
  p.K = K;
  p.sfa_bytes = dt != MGG_BF16 ? scale_bytes(sfa_n, sf) : 0;
  p.sfb_bytes = dt != MGG_BF16 ? scale_bytes(sfb_n, sf) : 0;
  p.meta_bytes = (uint32_t)G * 4;
  return dispatch_m<kPsum>(dt, sf, gran, pick_tile(expected_m, kContigBlock), false, p, stream);
}

mgg_status grouped_gemm_contiguous_swiglu_quant(mgg_dtype dt, int G, int M, int I, int K,
                                               const void* A, const void* SFA, const void* B,
                                               const void* SFB, mgg_sf_fmt sf,
                                               mgg_sfb_gran gran, void* Q, void* SFQ,
                                               mgg_sf_fmt sfq, float sf_zero,
                                               const int32_t* m_indices, hipStream_t stream) {
  g_last_error.clear();
  if (dt == MGG_BF16)
    return fail(MGG_EUNSUPPORTED, "the fused SwiGLU epilogue takes FP8 activations");
  if (I < 128 || I % 128 != 0) return fail(MGG_EINVAL, "I must be a positive multiple of 128");
  if (I > (1 << 27)) return fail(MGG_EUNSUPPORTED, "I too large");
  mgg_status st = check_common(dt, 2 * I, K, A, SFA, B, SFB, sf, Q, m_indices);
  if (st != MGG_OK) return st;
  if (G < 1 || G > kMaxExperts) return fail(MGG_EINVAL, "G must be in [1, 4096]");
  if (M < 1 || M > kMaxContigBlocks * kContigBlock)
    return fail(M < 1 ? MGG_EINVAL : MGG_EUNSUPPORTED, "M must be in [1, 524288]");
  if (dt == MGG_FP8_E4M3 && gran == MGG_SFB_CHANNEL && sf == MGG_SF_UE8M0)
    return fail(MGG_EUNSUPPORTED, "the fused SwiGLU epilogue takes UE8M0 weight scales per 128x128 block");
  if (!SFQ) return fail(MGG_EINVAL, "null pointer");
  if (sfq != MGG_SF_F32 && sfq != MGG_SF_UE8M0) return fail(MGG_EINVAL, "unknown scale format");
  if (sfq == MGG_SF_F32 && !aligned(SFQ, 4))
    return fail(MGG_EINVAL, "float32 output scales must be 4-byte aligned");
  if (!(sf_zero > 0.f) || !(sf_zero < 3.0e38f))
    return fail(MGG_EINVAL, "sf_zero must be a positive finite float");
  long sfb_n, b_row;
  st = weight_layout(dt, gran, G, 2L * I, K, &sfb_n, &b_row);
  if (st != MGG_OK) return st;
  const long KB = K / 128;
  const long sfa_n = KB * M, sfq_n = (long)(I / 128) * M;
  st = check_sizes({kTileRowsA * K, 2L * I * b_row, kTileRowsA * I, sfa_n * 4, sfb_n * 4,
                    sfq_n * 4});
  if (st != MGG_OK) return st;
  Params p{};
  p.A = (const uint8_t*)A;
  p.B = (const uint8_t*)B;
  p.SFA = SFA;
  p.SFB = SFB;
  p.D = Q;
  p.meta = m_indices;
  p.G = G;
  p.rows = M;
  p.N = 2 * I;
  p.K = K;
  p.sfa_bytes = scale_bytes(sfa_n, sf);
  p.sfb_bytes = scale_bytes(sfb_n, sf);
  p.meta_bytes = (uint32_t)M * 4;
  p.SFQ = SFQ;
  p.sfq_ue8m0 = sfq == MGG_SF_UE8M0;
  p.sf_zero = sf_zero;
  p.sfq_bytes = scale_bytes(sfq_n, sfq);
  if (dt == MGG_FP8_FP4)
    return launch_swi<kFP4W, kSfUE8M0, kSfbBlock32>(p, stream);
  if (sf == MGG_SF_UE8M0) return launch_swi<kFP8, kSfUE8M0, kSfbBlock>(p, stream);
  if (gran == MGG_SFB_BLOCK128) return launch_swi<kFP8, kSfF32, kSfbBlock>(p, stream);
  return launch_swi<kFP8, kSfF32, kSfbChannel>(p, stream);
}

mgg_status grouped_gemm_kgrouped(mgg_dtype dt, int G, int M, int N, int K_total, const void* A,
                                 const void* SFA, const void* B, const void* SFB,
                                 mgg_sf_fmt sf, float* D, const int32_t* ks, int accumulate,
                                 hipStream_t stream) {
  return kgrouped_impl(dt, G, M, N, K_total, A, SFA, B, SFB, sf, D, ks, accumulate, 0, stream);
}

mgg_status grouped_gemm_kgrouped_psum(mgg_dtype dt, int G, int M, int N, int K_total,
                                      const void* A, const void* SFA, const void* B,
                                      const void* SFB, mgg_sf_fmt sf, float* D,
                                      const int32_t* psum, int accumulate, hipStream_t stream) {
  return kgrouped_impl(dt, G, M, N, K_total, A, SFA, B, SFB, sf, D, psum, accumulate, 1, stream);
}

}  // extern "C"

namespace {

// K-grouped call; `meta_psum` selects cumulative token ends instead of per-expert counts.
mgg_status kgrouped_impl(mgg_dtype dt, int G, int M, int N, int K_total, const void* A,
                         const void* SFA, const void* B, const void* SFB, mgg_sf_fmt sf,
                         float* D, const int32_t* ks, int accumulate, int meta_psum,
                         hipStream_t stream) {
  g_last_error.clear();
  if (K_total < 0) return fail(MGG_EINVAL, "K_total must be non-negative");
  // check_common wants K >= 1; an empty token axis is still a valid call.
  mgg_status st = check_common(dt, N, K_total > 0 ? K_total : (dt == MGG_FP8_E4M3 ? 128 : 8),
                               A, SFA, B, SFB, sf, D, ks);
  if (st != MGG_OK) return st;
  if (dt == MGG_FP8_FP4) return fail(MGG_EUNSUPPORTED, "FP4 weights are M-grouped only");
  if (G < 1 || G > kMaxExperts) return fail(MGG_EINVAL, "G must be in [1, 4096]");
  if (M < 1) return fail(MGG_EINVAL, "M must be positive");
  if (accumulate != 0 && accumulate != 1) return fail(MGG_EINVAL, "accumulate must be 0 or 1");
  const long esz = dt == MGG_FP8_E4M3 ? 1 : 2, KB = K_total / 128;
  const long tiles = (long)G * cdiv(M, TileK::BM) * cdiv(N, TileK::BN);
  st = check_sizes({kTileRowsA * K_total * esz, kTileRowsB * K_total * esz, kTileRowsA * N * 4,
                    KB * M * 4, KB * N * 4, tiles});
  if (st != MGG_OK) return st;
  Params p{};
  p.A = (const uint8_t*)A;
  p.B = (const uint8_t*)B;
  p.SFA = SFA;
  p.SFB = SFB;
  p.D = D;
  p.meta = ks;
  p.G = G;
  p.rows = M;
  p.N = N;
  p.K = K_total;
  p.accumulate = accumulate;
  p.k_granule = dt == MGG_FP8_E4M3 ? 128 : 8;
  p.meta_psum = meta_psum;
  p.sfa_bytes = dt == MGG_FP8_E4M3 ? scale_bytes(KB * M, sf) : 0;
  p.sfb_bytes = dt == MGG_FP8_E4M3 ? scale_bytes(KB * N, sf) : 0;
  p.meta_bytes = (uint32_t)G * 4;
#define MGG_KG(DT_, SF_)                                                              \
  return accumulate ? launch<TileK, kKGrouped, DT_, SF_, kSfbChannel, true>(p, tiles, stream) \
                    : launch<TileK, kKGrouped, DT_, SF_, kSfbChannel, false>(p, tiles, stream)
  if (dt == MGG_BF16) { MGG_KG(kBF16, kSfF32); }
  if (sf == MGG_SF_F32) { MGG_KG(kFP8, kSfF32); }
  MGG_KG(kFP8, kSfUE8M0);
#undef MGG_KG
}

}  // namespace
