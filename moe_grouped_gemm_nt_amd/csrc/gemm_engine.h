// gemm_engine.h - the gfx950 grouped NT GEMM engine shared by the masked, contiguous
// and K-grouped entry points.
//
// One persistent kernel per call. Each workgroup (four copy waves, four or eight MFMA
// waves, and four epilogue waves when an accumulation input is read; see
// grouped_gemm_kernel.h):
//   1. reads the device-side routing (masked counts, contiguous row indices, K-grouped
//      token counts) into LDS and builds the tile prefix there, so nothing about the
//      expert distribution is baked into the launch (a captured hipGraph replays
//      correctly with new routing values);
//   2. walks its share of the (expert, m-tile, n-tile) list with an XCD-aware order;
//   3. per tile, streams 128-byte K slices of the activation rows and weight rows
//      through an S-stage ring of XOR-swizzled LDS buffers filled by direct global ->
//      LDS copies, and feeds MFMAs (FP8: 16x16x128 f8f6f4, one instruction per 128-K
//      scale group; BF16: 32x32x16 bf16);
//   4. FP8 only: promotes each 128-K partial sum into the FP32 accumulator with the
//      row scale times the weight scale (per-128-K promotion in registers);
//   5. stores rows under a per-row mask: a tile never writes past its expert's valid
//      rows, padding rows or another expert's rows.
// With an accumulation input (K-grouped D = C + A B^T) four more waves own the
// epilogue: they prefetch C tiles several tiles ahead straight into registers, add the
// MFMA waves' results handed over through LDS, and store D.
//
// Operand roles. The MFMA's first operand is fed with WEIGHT rows (n) and its second
// with ACTIVATION rows (m), so each lane ends up holding 4 consecutive n of one m; the
// weight rows of a wave are further permuted so that one lane holds 4*NI consecutive
// n, which turns the epilogue into full 16-byte row-contiguous stores.
//
// K order. The 16x16x128 FP8 operand of lanes 16g..16g+15 holds K 16g..16g+15 in its
// first four registers and K 64+16g..64+16g+15 in the last four, so those lanes read
// the 16-byte chunks g and g+4 of each 128-byte slice; an FP4 operand's lanes
// 16g..16g+15 hold K 32g..32g+31 (the 16-byte chunk g of a 64-byte FP4 slice), and the
// MX scale a lane passes covers exactly those 32 elements. Across slices K ascends. The layout,
// the instruction and the promotion formula do not depend on the tile shape, so every
// tile configuration produces the same bits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace mgg {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

enum Variant { kMasked = 0, kContig = 1, kKGrouped = 2, kPsum = 3 };
// kFP4W: FP8 E4M3 activations times FP4 E2M1 weights (two per byte, even K element in
// the low nibble) with one UE8M0 scale per 32 K of a weight row.
enum DType { kBF16 = 0, kFP8 = 1, kFP4W = 2 };
enum SfFmt { kSfF32 = 0, kSfUE8M0 = 1 };
enum SfbGran { kSfbBlock = 0, kSfbChannel = 1, kSfbBlock32 = 2 };

constexpr int kThreads = 256;     // one group of four waves
// Tiles of accumulation input in flight per epilogue wave. Deeper prefetch measured
// slower on the K-grouped wgrad shape: the extra C loads queue in front of the MFMA
// waves' operand copies in the CU's memory pipeline.
constexpr int kCPrefetch = 2;
constexpr int kSliceBytes = 128;  // K bytes per row per pipeline stage
constexpr int kXcds = 8;          // MI355X: 8 accelerator dies, WGs dispatched round-robin
constexpr int kContigBlock = 128; // rows per contiguous-layout alignment block
constexpr int kMaxExperts = 4096;  // the expert index shares an int with the block index
constexpr int kMaxContigBlocks = 4096;
constexpr int kLdsBytes = 160 * 1024;  // per workgroup on gfx950
// Flag on a K-grouped expert's scheduler entry (its token prefix, at most 2^28 + 1):
// the expert is outside the routing contract and is skipped.
constexpr int kKUnusable = 1 << 30;

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
  int meta_psum;   // K-grouped: the routing holds cumulative token ends, not counts
  // Fused SwiGLU epilogue (contiguous): D receives E4M3 codes [rows][N/2] of
  // silu(gate) * up and SFQ their 1x128 scales [N/256][rows] (float32, or UE8M0 bytes
  // when sfq_ue8m0); an all-zero group takes sf_zero.
  void* SFQ;
  int sfq_ue8m0;
  float sf_zero;
  uint32_t sfq_bytes;
  uint32_t sfa_bytes, sfb_bytes;  // readable bytes of the scale tensors (FP8)
  uint32_t meta_bytes;            // bytes of the routing tensor
};

// Tile configuration: BM activation rows x BN weight rows per workgroup; WM x WN MFMA
// waves (four or eight) laid out WM along m and WN along n; S pipeline stages of
// 128-byte K slices in LDS. SWI: the fused SwiGLU tile of the contiguous product, whose
// 256 weight rows are the gate rows and then the up rows of 128 output columns, one
// wave row-band covering all of them (so a row's 1x128 output group stays in one wave).
// STREAMW: the weight copies take the streaming cache policy (every weight panel of the
// call is read once).
template <int BM_, int BN_, int WM_, int WN_, int S_, bool SWI_ = false, bool STREAMW_ = false>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, S = S_;
  static constexpr bool SWI = SWI_;
  static constexpr bool STREAMW = STREAMW_;
  static_assert(!SWI || (BN == 256 && WN == 1), "fused SwiGLU tile: 256 weight rows, one wave column");
  static constexpr int NMW = WM * WN;  // MFMA waves
  static_assert(NMW == 4 || NMW == 8, "four or eight MFMA waves");
  static_assert(S >= 2 && S <= 6, "pipeline depth");
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  // FP8 runs 16x16x128 MFMAs (MJ x NI subtiles per wave); BF16 runs 32x32x16 MFMAs
  // (MJ2 x NI2 subtiles), the BF16 shape with the full matrix-core rate on gfx950.
  static constexpr int MJ = WTM / 16, NI = WTN / 16;
  static constexpr int MJ2 = WTM / 32, NI2 = WTN / 32;
  static_assert(MJ >= 1 && NI >= 2 && WTM % 16 == 0 && WTN % 16 == 0, "16x16 subtiles");
  static_assert(SWI || (WTN <= 128 && 128 % WTN == 0),
                "a wave's n range stays in one 128-row block");
  static_assert((BM + BN) % 32 == 0 && BM % 8 == 0, "whole 8-row copies, 4 waves");
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

// Inclusive running maximum of `n` ints held in LDS `buf` (in place), block-wide over NT
// threads; same structure as the scan below (every thread must call it, `s_tmp` needs
// NT / 64 ints, two barriers).
template <int NT>
__device__ void block_inclusive_max(int* buf, int n, int* s_tmp) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = (n + NT - 1) / NT;
  const int lo = tid * per;
  const int hi = min(lo + per, n);
  int local = INT_MIN;
  for (int i = lo; i < hi; ++i) local = max(local, buf[i]);
  int incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off, 64);
    if (lane >= off) incl = max(incl, v);
  }
  if (lane == 63) s_tmp[wave] = incl;
  __syncthreads();
  int run = INT_MIN;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) run = w < wave ? max(run, s_tmp[w]) : run;
  const int before_lane = __shfl_up(incl, 1, 64);
  if (lane > 0) run = max(run, before_lane);  // maximum of everything before this chunk
  for (int i = lo; i < hi; ++i) {
    run = max(run, buf[i]);
    buf[i] = run;
  }
  __syncthreads();
}

// Exclusive scan like block_exclusive_scan, for values in [0, cap] with every partial
// sum saturating at cap (min(a + b, cap) is associative on non-negative values, so the
// result is the exact prefix clamped to cap); 2 * cap must fit an int. Returns the
// saturated total.
template <int NT>
__device__ int block_exclusive_scan_sat(int* buf, int n, int* s_tmp, int cap) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = (n + NT - 1) / NT;
  const int lo = tid * per;
  const int hi = min(lo + per, n);
  int local = 0;
  for (int i = lo; i < hi; ++i) local = min(local + buf[i], cap);
  int incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off, 64);
    if (lane >= off) incl = min(incl + v, cap);
  }
  int excl = __shfl_up(incl, 1, 64);  // saturated sums do not subtract: shift instead
  if (lane == 0) excl = 0;
  if (lane == 63) s_tmp[wave] = incl;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    if (w < wave) before = min(before + s_tmp[w], cap);
    total = min(total + s_tmp[w], cap);
  }
  int run = min(before + excl, cap);
  for (int i = lo; i < hi; ++i) {
    const int v = buf[i];
    buf[i] = run;
    run = min(run + v, cap);
  }
  __syncthreads();
  return total;
}

// Exclusive scan of `n` ints held in LDS `buf` (in place), block-wide over NT threads;
// returns the total. Every thread of the block must call it; `s_tmp` needs NT / 64
// ints. Each thread sums a contiguous chunk, waves scan their 64 partial sums with
// cross-lane shuffles, and the wave totals are combined through LDS (two barriers).
template <int NT>
__device__ int block_exclusive_scan(int* buf, int n, int* s_tmp) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = (n + NT - 1) / NT;
  const int lo = tid * per;
  const int hi = min(lo + per, n);
  int local = 0;
  for (int i = lo; i < hi; ++i) local += buf[i];
  int incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off, 64);
    if (lane >= off) incl += v;
  }
  if (lane == 63) s_tmp[wave] = incl;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    before += w < wave ? s_tmp[w] : 0;
    total += s_tmp[w];
  }
  int run = before + incl - local;  // exclusive prefix of this thread's chunk
  for (int i = lo; i < hi; ++i) {
    const int v = buf[i];
    buf[i] = run;
    run += v;
  }
  __syncthreads();
  return total;
}

// Weight-row order inside LDS. The first MFMA operand is fed with weight rows in LDS
// order; the rows are permuted so that each lane's outputs cover contiguous weight
// columns, which makes the epilogue 16-byte row-contiguous stores.
//
// FP8 (16x16 outputs: lane group q holds MFMA rows 4q..4q+3): a wave's WTN rows are
// stored so that subtile i reads 16 consecutive LDS rows while lane group q covers the
// contiguous range [q*4*NI, (q+1)*4*NI) of the wave.
// BF16 (32x32 outputs: lane group g = lane / 32 holds MFMA rows 8t + 4g + r, t, r in
// 0..3): MFMA row i of subtile s is weight row 32 s + 16 ((i >> 2) & 1) + 4 (i >> 3) +
// (i & 3), so lane group g covers 16 contiguous rows of each subtile.
template <class T, bool BF16>
__device__ __forceinline__ int weight_row_of_lds(int R) {
  const int w = R / T::WTN, rl = R % T::WTN;
  if constexpr (BF16) {
    const int s = rl / 32, i = rl % 32;
    return w * T::WTN + 32 * s + 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3);
  } else {
    const int i = rl / 16, q = (rl % 16) / 4, r = rl % 4;
    return w * T::WTN + q * 4 * T::NI + 4 * i + r;
  }
}

// ----------------------------------------------------------------------------- buffers
//
// Global memory is read through buffer resources (base, size in bytes): a lane whose
// byte offset is at or beyond the size reads zeros and its stores are dropped. Every
// out-of-range row, column or K chunk is expressed that way (offset kOOB), so nothing
// outside an expert's block is ever touched and the instruction stream is the same for
// every lane and every tile.

constexpr uint32_t kOOB = 0x80000000u;  // beyond any resource size (sizes are < 2^31)

__device__ __forceinline__ v4i make_rsrc(const void* base, uint32_t nbytes) {
  const unsigned long long a = reinterpret_cast<unsigned long long>(base);
  v4i r;
  r.x = __builtin_amdgcn_readfirstlane((int)(a & 0xffffffffu));
  r.y = __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xffffu));  // stride 0
  r.z = __builtin_amdgcn_readfirstlane((int)nbytes);
  r.w = 0x00020000;  // raw 32-bit data, gfx9 buffer format
  return r;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
}

// Direct global -> LDS copies: each lane's 16 (or 4) bytes land at lds + 16 * lane
// (or 4 * lane). The s_nops cover the SGPR-write -> VMEM-read and M0-write -> LDS-DMA
// wait states, which the compiler cannot see inside the asm.
// The LDS address is uniform by construction; readfirstlane makes that explicit. A
// batch of copies starts with dma_fence(), which covers the wait states between a
// VALU write of an SGPR (resource descriptors come from readfirstlane) and a vector
// memory instruction reading it; each copy then only needs the M0 -> LDS-DMA gap.
__device__ __forceinline__ void dma_fence() { asm volatile("s_nop 4" ::: "memory"); }
__device__ __forceinline__ void dma_x4(uint32_t lds, v4i rsrc, uint32_t voff) {
  const uint32_t l = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(l), "v"(voff), "s"(rsrc) : "memory");
}
// The same copy with the streaming (non-temporal) cache policy, for operand bytes that
// are read once.
__device__ __forceinline__ void dma_x4_nt(uint32_t lds, v4i rsrc, uint32_t voff) {
  const uint32_t l = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
               :: "s"(l), "v"(voff), "s"(rsrc) : "memory");
}
// The same copies with a wave-uniform byte offset `soff` added to every lane's address (the
// instruction's scalar offset operand): lanes whose voff is out of range stay out of range.
__device__ __forceinline__ void dma_x4_so(uint32_t lds, v4i rsrc, uint32_t voff, uint32_t soff) {
  const uint32_t l = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(l), "v"(voff), "s"(rsrc), "s"(soff) : "memory");
}
__device__ __forceinline__ void dma_x4_nt_so(uint32_t lds, v4i rsrc, uint32_t voff,
                                             uint32_t soff) {
  const uint32_t l = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen nt lds"
               :: "s"(l), "v"(voff), "s"(rsrc), "s"(soff) : "memory");
}
__device__ __forceinline__ void dma_x1(uint32_t lds, v4i rsrc, uint32_t voff) {
  const uint32_t l = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :: "s"(l), "v"(voff), "s"(rsrc) : "memory");
}
// Calls f(std::integral_constant<int, I>) for I = B .. E - 1 in order.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Pins a uniform value in SGPRs at this point of the program.
__device__ __forceinline__ void pin_sgpr(v4i& r) { asm volatile("" : "+s"(r)); }

// Workgroup barrier that orders LDS: all of this wave's LDS reads have returned and no
// memory access is moved across it by the compiler.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// s_waitcnt vmcnt(N): at most N of this wave's vector-memory operations outstanding.
template <int N>
__device__ __forceinline__ void vm_wait_imm() {
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N < 63 ? N : 63) : "memory");
}

// The LLVM raw buffer store intrinsic, declared with the 128-bit resource as a plain
// int vector so the same descriptor serves the asm copies above.
extern "C" __device__ void mgg_raw_buffer_store_v4i32(v4i vdata, v4i rsrc, int voffset,
                                                     int soffset, int aux)
    __asm("llvm.amdgcn.raw.buffer.store.v4i32");

// Cache-policy operand of the buffer intrinsics: bit 1 is the gfx950 "nt" (streaming)
// hint, for data touched once per call.
constexpr int kCacheDefault = 0;
constexpr int kCacheStream = 2;

template <int AUX = kCacheDefault>
__device__ __forceinline__ void store_b128(v4i rsrc, uint32_t voff, v4i v) {
  mgg_raw_buffer_store_v4i32(v, rsrc, (int)voff, 0, AUX);
}

// The matching load into registers; the compiler tracks its completion like any load.
extern "C" __device__ v4i mgg_raw_buffer_load_v4i32(v4i rsrc, int voffset, int soffset, int aux)
    __asm("llvm.amdgcn.raw.buffer.load.v4i32");

template <int AUX = kCacheDefault>
__device__ __forceinline__ v4i load_b128(v4i rsrc, uint32_t voff) {
  return mgg_raw_buffer_load_v4i32(rsrc, (int)voff, 0, AUX);
}

// 4-byte and 1-byte stores (per-row scales of a fused epilogue).
extern "C" __device__ void mgg_raw_buffer_store_i32(int vdata, v4i rsrc, int voffset,
                                                    int soffset, int aux)
    __asm("llvm.amdgcn.raw.buffer.store.i32");
extern "C" __device__ void mgg_raw_buffer_store_i8(char vdata, v4i rsrc, int voffset,
                                                   int soffset, int aux)
    __asm("llvm.amdgcn.raw.buffer.store.i8");

__device__ __forceinline__ void store_b32(v4i rsrc, uint32_t voff, uint32_t v) {
  mgg_raw_buffer_store_i32((int)v, rsrc, (int)voff, 0, kCacheDefault);
}
__device__ __forceinline__ void store_b8(v4i rsrc, uint32_t voff, uint32_t v) {
  mgg_raw_buffer_store_i8((char)v, rsrc, (int)voff, 0, kCacheDefault);
}

}  // namespace mgg
