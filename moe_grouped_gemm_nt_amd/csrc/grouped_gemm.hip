// grouped_gemm.hip - host side of the C ABI declared in include/moe_grouped_gemm_nt.h:
// argument validation, tile-shape choice, grid sizing and kernel launch.
//
// The host never touches device data: the grid is sized from static shapes (experts,
// capacity or rows, N) and the CU count, and every workgroup reads the routing
// buffers itself, so a call captured into a hipGraph stays correct when the routing
// values change between replays.

#include <mutex>
#include <string>
#include <unordered_map>

#include "grouped_gemm_kernel.h"
#include "moe_grouped_gemm_nt.h"

using namespace mgg;

namespace {

thread_local std::string g_last_error;

mgg_status fail(mgg_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

// Tile shapes. Small-M tiles keep the MFMA work proportional to the valid rows when
// experts receive few tokens; all of them produce bitwise-identical results.
using TileS = Tile<32, 256, 1, 4>;   // <= 32 rows per expert: weight streaming
using TileM = Tile<64, 256, 1, 4>;   // <= 64 rows
using TileL = Tile<128, 256, 2, 2>;  // larger experts
using TileK = Tile<128, 128, 2, 2>;  // K-grouped output tiles

enum TileId { kTileS = 0, kTileM = 1, kTileL = 2 };

struct DevInfo {
  int cus = 0;
  int max_lds = 0;
};

std::mutex g_mu;
std::unordered_map<int, DevInfo> g_dev;
std::unordered_map<const void*, int> g_occ;  // (kernel) -> resident workgroups per CU

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
  if (hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return false;
  if (hipDeviceGetAttribute(&d.max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) !=
      hipSuccess)
    return false;
  g_dev[dev] = d;
  *out = d;
  return true;
}

template <class T, int VAR, int DT, int SF, int GRAN>
constexpr int pipe_bytes() {
  return Layout<T, VAR, DT, SF, GRAN>::PIPE;
}

template <class T, int VAR, int DT, int SF, int GRAN>
mgg_status launch(const Params& p, long max_tiles, int sched_n, hipStream_t stream) {
  auto kern = grouped_gemm_kernel<T, VAR, DT, SF, GRAN>;
  const size_t lds = (size_t)pipe_bytes<T, VAR, DT, SF, GRAN>() +
                     (size_t)(kThreads + 3 * sched_n) * sizeof(int);
  DevInfo dev;
  if (!dev_info(&dev)) return fail(MGG_EHIP, "hipGetDevice/hipDeviceGetAttribute failed");
  if ((long)lds > 160 * 1024)
    return fail(MGG_EUNSUPPORTED, "too many experts or row blocks for the LDS scheduler");
  int occ = 1;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    auto it = g_occ.find((const void*)kern);
    if (it == g_occ.end()) {
      hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                          160 * 1024);
      int o = 0;
      // Occupancy at the pipeline's own LDS footprint; the scheduler arrays are small
      // for typical expert counts.
      const size_t lds_typ = (size_t)pipe_bytes<T, VAR, DT, SF, GRAN>() + 4096;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, kern, kThreads, lds_typ) !=
              hipSuccess || o < 1)
        o = 1;
      g_occ[(const void*)kern] = o;
      occ = o;
    } else {
      occ = it->second;
    }
  }
  const long resident = (long)dev.cus * occ;
  long grid = max_tiles < resident ? max_tiles : resident;
  if (grid >= kXcds) grid -= grid % kXcds;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), lds, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MGG_EHIP, std::string("kernel launch: ") + hipGetErrorString(e));
  return MGG_OK;
}

// Dispatch over the compile-time parameters of the M-grouped variants.
template <int VAR>
mgg_status dispatch_m(mgg_dtype dt, mgg_sf_fmt sf, mgg_sfb_gran gran, TileId tile,
                      const Params& p, long tiles_s, long tiles_m, long tiles_l, int sched_n,
                      hipStream_t s) {
#define MGG_TILE_SWITCH(DT_, SF_, GR_)                                                  \
  switch (tile) {                                                                       \
    case kTileS: return launch<TileS, VAR, DT_, SF_, GR_>(p, tiles_s, sched_n, s);      \
    case kTileM: return launch<TileM, VAR, DT_, SF_, GR_>(p, tiles_m, sched_n, s);      \
    default: return launch<TileL, VAR, DT_, SF_, GR_>(p, tiles_l, sched_n, s);          \
  }
  if (dt == MGG_BF16) {
    MGG_TILE_SWITCH(kBF16, kSfF32, kSfbBlock)
  }
  if (sf == MGG_SF_F32) {
    if (gran == MGG_SFB_BLOCK128) { MGG_TILE_SWITCH(kFP8, kSfF32, kSfbBlock) }
    MGG_TILE_SWITCH(kFP8, kSfF32, kSfbChannel)
  }
  if (gran == MGG_SFB_BLOCK128) { MGG_TILE_SWITCH(kFP8, kSfUE8M0, kSfbBlock) }
  MGG_TILE_SWITCH(kFP8, kSfUE8M0, kSfbChannel)
#undef MGG_TILE_SWITCH
}

TileId pick_tile(int expected_m, int fallback) {
  const int em = expected_m > 0 ? expected_m : fallback;
  if (em <= 32) return kTileS;
  if (em <= 64) return kTileM;
  return kTileL;
}

long cdiv(long a, long b) { return (a + b - 1) / b; }

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

mgg_status check_common(mgg_dtype dt, int N, int K, const void* A, const void* SFA,
                        const void* B, const void* SFB, mgg_sf_fmt sf, const void* D,
                        const void* meta) {
  if (dt != MGG_BF16 && dt != MGG_FP8_E4M3) return fail(MGG_EINVAL, "unknown dtype");
  if (N < 1 || N % 8 != 0) return fail(MGG_EINVAL, "N must be a positive multiple of 8");
  if (K < 1) return fail(MGG_EINVAL, "K must be positive");
  if (dt == MGG_BF16 && K % 8 != 0) return fail(MGG_EINVAL, "BF16 needs K % 8 == 0");
  if (dt == MGG_FP8_E4M3 && K % 128 != 0) return fail(MGG_EINVAL, "FP8 needs K % 128 == 0");
  if (K > (1 << 28)) return fail(MGG_EUNSUPPORTED, "K too large");
  if (!A || !B || !D || !meta) return fail(MGG_EINVAL, "null pointer");
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(D, 16))
    return fail(MGG_EINVAL, "A, B and D must be 16-byte aligned");
  if (dt == MGG_FP8_E4M3) {
    if (!SFA || !SFB) return fail(MGG_EINVAL, "FP8 needs SFA and SFB");
    if (sf != MGG_SF_F32 && sf != MGG_SF_UE8M0) return fail(MGG_EINVAL, "unknown scale format");
    if (sf == MGG_SF_F32 && (!aligned(SFA, 4) || !aligned(SFB, 4)))
      return fail(MGG_EINVAL, "float32 scales must be 4-byte aligned");
  }
  if (!aligned(meta, 4)) return fail(MGG_EINVAL, "routing buffer must be 4-byte aligned");
  return MGG_OK;
}

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

mgg_status grouped_gemm_masked(mgg_dtype dt, int G, int cap, int N, int K, const void* A,
                               const void* SFA, const void* B, const void* SFB,
                               mgg_sf_fmt sf, mgg_sfb_gran gran, void* D,
                               const int32_t* masked_m, int expected_m, hipStream_t stream) {
  g_last_error.clear();
  mgg_status st = check_common(dt, N, K, A, SFA, B, SFB, sf, D, masked_m);
  if (st != MGG_OK) return st;
  if (G < 1 || G > kMaxExperts) return fail(MGG_EINVAL, "G must be in [1, 4096]");
  if (cap < 1) return fail(MGG_EINVAL, "cap must be positive");
  if (dt == MGG_FP8_E4M3 && gran != MGG_SFB_BLOCK128 && gran != MGG_SFB_CHANNEL)
    return fail(MGG_EINVAL, "unknown weight-scale granularity");
  const long ntn_s = cdiv(N, TileS::BN), ntn_l = cdiv(N, TileL::BN);
  const long tiles_s = (long)G * cdiv(cap, TileS::BM) * ntn_s;
  const long tiles_m = (long)G * cdiv(cap, TileM::BM) * ntn_s;
  const long tiles_l = (long)G * cdiv(cap, TileL::BM) * ntn_l;
  if (tiles_s >= (1L << 31)) return fail(MGG_EUNSUPPORTED, "problem too large");
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
  const TileId tile = pick_tile(expected_m, cap);
  return dispatch_m<kMasked>(dt, sf, gran, tile, p, tiles_s, tiles_m, tiles_l, G, stream);
}

mgg_status grouped_gemm_contiguous(mgg_dtype dt, int G, int M, int N, int K, const void* A,
                                   const void* SFA, const void* B, const void* SFB,
                                   mgg_sf_fmt sf, mgg_sfb_gran gran, void* D,
                                   const int32_t* m_indices, int expected_m,
                                   hipStream_t stream) {
  g_last_error.clear();
  mgg_status st = check_common(dt, N, K, A, SFA, B, SFB, sf, D, m_indices);
  if (st != MGG_OK) return st;
  if (G < 1) return fail(MGG_EINVAL, "G must be positive");
  if (M < 1 || M > kMaxContigBlocks * kContigBlock)
    return fail(M < 1 ? MGG_EINVAL : MGG_EUNSUPPORTED, "M must be in [1, 524288]");
  if (dt == MGG_FP8_E4M3 && gran != MGG_SFB_BLOCK128 && gran != MGG_SFB_CHANNEL)
    return fail(MGG_EINVAL, "unknown weight-scale granularity");
  const long nb = cdiv(M, kContigBlock);
  const long ntn_s = cdiv(N, TileS::BN), ntn_l = cdiv(N, TileL::BN);
  const long tiles_s = nb * (kContigBlock / TileS::BM) * ntn_s;
  const long tiles_m = nb * (kContigBlock / TileM::BM) * ntn_s;
  const long tiles_l = nb * (kContigBlock / TileL::BM) * ntn_l;
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
  const TileId tile = pick_tile(expected_m, kContigBlock);
  return dispatch_m<kContig>(dt, sf, gran, tile, p, tiles_s, tiles_m, tiles_l, (int)nb, stream);
}

mgg_status grouped_gemm_kgrouped(mgg_dtype dt, int G, int M, int N, int K_total, const void* A,
                                 const void* SFA, const void* B, const void* SFB,
                                 mgg_sf_fmt sf, float* D, const int32_t* ks, int accumulate,
                                 hipStream_t stream) {
  g_last_error.clear();
  if (K_total < 0) return fail(MGG_EINVAL, "K_total must be non-negative");
  // check_common wants K >= 1; an empty token axis is still a valid call.
  mgg_status st = check_common(dt, N, K_total > 0 ? K_total : (dt == MGG_FP8_E4M3 ? 128 : 8),
                               A, SFA, B, SFB, sf, D, ks);
  if (st != MGG_OK) return st;
  if (G < 1 || G > kMaxExperts) return fail(MGG_EINVAL, "G must be in [1, 4096]");
  if (M < 1) return fail(MGG_EINVAL, "M must be positive");
  if (accumulate != 0 && accumulate != 1) return fail(MGG_EINVAL, "accumulate must be 0 or 1");
  const long tiles = (long)G * cdiv(M, TileK::BM) * cdiv(N, TileK::BN);
  if (tiles >= (1L << 31)) return fail(MGG_EUNSUPPORTED, "problem too large");
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
  if (dt == MGG_BF16)
    return launch<TileK, kKGrouped, kBF16, kSfF32, kSfbChannel>(p, tiles, G, stream);
  if (sf == MGG_SF_F32)
    return launch<TileK, kKGrouped, kFP8, kSfF32, kSfbChannel>(p, tiles, G, stream);
  return launch<TileK, kKGrouped, kFP8, kSfUE8M0, kSfbChannel>(p, tiles, G, stream);
}

}  // extern "C"
