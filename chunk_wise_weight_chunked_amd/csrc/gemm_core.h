// gemm_core.h -- the MFMA/LDS GEMM mainloop shared by the four contractions of
// the TTT-MLP layer on CDNA4 (gfx950).
//
// Every contraction of the layer is put in "both operands K-contiguous" form,
//     acc[m][n] += sum_k A[m][k] * B[n][k],
// so one mainloop serves all of them; the kernels differ only in how the
// operand rows are found (row loaders) and what happens to the accumulator
// (epilogues).
//
// Tile geometry (one workgroup = 4 wave64s in a 2 x 2 grid):
//   * BM x BN output tile, each wave owns (BM/2) x (BN/2) as 32x32 MFMA blocks;
//   * one k-tile = 128 bytes of K per operand row (64 bf16 or 32 fp32 values);
//   * LDS holds two stages of A (BM x 128 B) and B (BN x 128 B); each 128-byte
//     row is eight 16-byte chunks stored at chunk ^ (row & 7), so both the
//     16-byte row-wise global->LDS stores and the column-wise fragment reads of
//     32 consecutive rows are free of bank conflicts;
//   * bf16 uses v_mfma_f32_32x32x16_bf16 (each lane feeds 8 consecutive K
//     values of one row); fp32 uses v_mfma_f32_32x32x2_f32, eight of them per
//     16 K values, with A and B lanes agreeing on which K each one covers.
// Accumulator element r of block (i, j) in lane l sits at
//     row = 32 i + 8 (r / 4) + 4 (l / 32) + (r % 4),   col = 32 j + (l % 32)
// of the wave's sub-tile (the MFMA 32x32 result layout).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ttt {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;     // 4 waves
constexpr int kRowBytes = 128;    // bytes of K per operand row per k-tile
constexpr int kChunks = 8;        // 16-byte chunks per row per k-tile
constexpr int kTokenAlign = 64;   // chunk padding in the token-major layouts

// ----------------------------------------------------------------- numbers
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16, round to nearest even; NaN stays NaN (quiet).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kPerChunk = 4;  // values per 16-byte chunk
  __device__ __forceinline__ static float to_f32(float v) { return v; }
  __device__ __forceinline__ static void store(float* p, float v) { *p = v; }
};
template <> struct Elem<uint16_t> {  // bf16 stored as raw bits
  static constexpr int kPerChunk = 8;
  __device__ __forceinline__ static float to_f32(uint16_t v) { return bf16_bits_to_f32(v); }
  __device__ __forceinline__ static void store(uint16_t* p, float v) { *p = f32_to_bf16_bits(v); }
};

// Value i (0..kPerChunk-1) of a 16-byte chunk, as float.
template <typename T>
__device__ __forceinline__ float chunk_value(const uint4& c, int i);
template <>
__device__ __forceinline__ float chunk_value<float>(const uint4& c, int i) {
  const uint32_t w = i == 0 ? c.x : i == 1 ? c.y : i == 2 ? c.z : c.w;
  return __uint_as_float(w);
}
template <>
__device__ __forceinline__ float chunk_value<uint16_t>(const uint4& c, int i) {
  const uint32_t w = (i >> 1) == 0 ? c.x : (i >> 1) == 1 ? c.y : (i >> 1) == 2 ? c.z : c.w;
  return bf16_bits_to_f32((i & 1) ? (w >> 16) : (w & 0xffffu));
}

// --------------------------------------------------------------- LDS layout
__device__ __forceinline__ uint32_t lds_offset(int row, int chunk) {
  return (uint32_t)row * kRowBytes + (uint32_t)((chunk ^ (row & 7)) << 4);
}

// ------------------------------------------------------------- tile shapes
template <int BM_, int BN_>
struct TileShape {
  static constexpr int BM = BM_;
  static constexpr int BN = BN_;
  static constexpr int WM = BM / 2;   // wave sub-tile rows
  static constexpr int WN = BN / 2;   // wave sub-tile cols
  static constexpr int MB = WM / 32;  // 32x32 blocks per wave, rows
  static constexpr int NB = WN / 32;  // 32x32 blocks per wave, cols
  static constexpr int kStageBytes = (BM + BN) * kRowBytes;
  static constexpr int kLdsBytes = 2 * kStageBytes;
  static_assert(BM % 64 == 0 && BN % 64 == 0, "tile must hold 2x2 waves of 32x32 blocks");
};

template <class S>
struct Accum {
  floatx16_t v[S::MB][S::NB];
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < S::MB; ++i)
#pragma unroll
      for (int j = 0; j < S::NB; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) v[i][j][r] = 0.0f;
  }
};

// Position of accumulator element (i, j, r) of this lane inside the BM x BN tile.
struct LanePos {
  int wave_m0, wave_n0, lane;
  __device__ __forceinline__ int row(int i, int r) const {
    return wave_m0 + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
  }
  __device__ __forceinline__ int col(int j) const { return wave_n0 + 32 * j + (lane & 31); }
};

template <class S>
__device__ __forceinline__ LanePos lane_pos() {
  const int wave = threadIdx.x >> 6;
  LanePos p;
  p.wave_m0 = (wave >> 1) * S::WM;
  p.wave_n0 = (wave & 1) * S::WN;
  p.lane = threadIdx.x & 63;
  return p;
}

// ---------------------------------------------------------- fragment + MFMA
template <typename T, class S>
struct Mma;

template <class S>
struct Mma<uint16_t, S> {
  static constexpr int kSteps = 4;  // 16 K values per step, 64 per k-tile
  __device__ __forceinline__ static void ktile(Accum<S>& acc, const char* sA, const char* sB,
                                               const LanePos& p) {
    const int r = p.lane & 31, h = p.lane >> 5;
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      bf16x8_t a[S::MB], b[S::NB];
#pragma unroll
      for (int i = 0; i < S::MB; ++i)
        a[i] = *reinterpret_cast<const bf16x8_t*>(sA + lds_offset(p.wave_m0 + 32 * i + r, 2 * s + h));
#pragma unroll
      for (int j = 0; j < S::NB; ++j)
        b[j] = *reinterpret_cast<const bf16x8_t*>(sB + lds_offset(p.wave_n0 + 32 * j + r, 2 * s + h));
#pragma unroll
      for (int i = 0; i < S::MB; ++i)
#pragma unroll
        for (int j = 0; j < S::NB; ++j)
          acc.v[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc.v[i][j], 0, 0, 0);
    }
  }
};

template <class S>
struct Mma<float, S> {
  static constexpr int kSteps = 2;  // 16 K values per step, 32 per k-tile
  __device__ __forceinline__ static void ktile(Accum<S>& acc, const char* sA, const char* sB,
                                               const LanePos& p) {
    const int r = p.lane & 31, h = p.lane >> 5;
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      floatx4_t a[S::MB][2], b[S::NB][2];
#pragma unroll
      for (int i = 0; i < S::MB; ++i)
#pragma unroll
        for (int q = 0; q < 2; ++q)
          a[i][q] = *reinterpret_cast<const floatx4_t*>(
              sA + lds_offset(p.wave_m0 + 32 * i + r, 4 * s + 2 * h + q));
#pragma unroll
      for (int j = 0; j < S::NB; ++j)
#pragma unroll
        for (int q = 0; q < 2; ++q)
          b[j][q] = *reinterpret_cast<const floatx4_t*>(
              sB + lds_offset(p.wave_n0 + 32 * j + r, 4 * s + 2 * h + q));
#pragma unroll
      for (int i = 0; i < S::MB; ++i)
#pragma unroll
        for (int j = 0; j < S::NB; ++j)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            acc.v[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i][e >> 2][e & 3],
                                                               b[j][e >> 2][e & 3],
                                                               acc.v[i][j], 0, 0, 0);
    }
  }
};

// ------------------------------------------------------------- row loaders
// A row loader moves one operand's k-tile (ROWS rows x 128 bytes) from global
// memory to LDS in two phases: load(kt) issues the global loads into
// registers, store(lds) writes them to the swizzled LDS stage.  Thread t owns
// chunk (t & 7) of rows (t >> 3) + 32 q, q = 0 .. ROWS/32 - 1.
template <int ROWS>
struct RowLoader {
  static constexpr int kPer = ROWS / 32;
  const char* ptr[kPer];  // row base (byte address of this thread's chunk at k = 0)
  uint4 reg[kPer];

  // row_base(q) returns the byte address of row (t>>3)+32q at K index 0, or
  // nullptr when that row lies outside the operand (it then loads zeros).
  template <class F>
  __device__ __forceinline__ void init(F&& row_base) {
    const int c = threadIdx.x & 7;
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const char* b = row_base(q);
      ptr[q] = b ? b + c * 16 : nullptr;
    }
  }
  __device__ __forceinline__ void load(int64_t kt) {
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      if (ptr[q])
        reg[q] = *reinterpret_cast<const uint4*>(ptr[q] + kt * kRowBytes);
      else
        reg[q] = make_uint4(0u, 0u, 0u, 0u);
    }
  }
  __device__ __forceinline__ void store(char* lds) const {
    const int c = threadIdx.x & 7, r0 = threadIdx.x >> 3;
#pragma unroll
    for (int q = 0; q < kPer; ++q)
      *reinterpret_cast<uint4*>(lds + lds_offset(r0 + 32 * q, c)) = reg[q];
  }
};

// ---------------------------------------------------------------- mainloop
// Runs k-tiles [0, nk) through a two-stage LDS pipeline: while the MFMAs work
// on stage kt&1, the global loads of k-tile kt+1 are in flight; one barrier
// per k-tile separates the LDS writes of the next stage from the reads of the
// current one.  after_ktile(kt) runs once every wave has finished k-tile kt
// (it may touch registers and global memory, not LDS).
template <typename T, class S, class LA, class LB, class Hook>
__device__ __forceinline__ void mainloop(Accum<S>& acc, LA& la, LB& lb, int64_t nk, char* smem,
                                         const LanePos& p, Hook&& after_ktile) {
  char* stage[2] = {smem, smem + S::kStageBytes};
  if (nk <= 0) return;
  la.load(0);
  lb.load(0);
  la.store(stage[0]);
  lb.store(stage[0] + S::BM * kRowBytes);
  __syncthreads();
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int cur = (int)(kt & 1);
    const bool more = kt + 1 < nk;
    if (more) {
      la.load(kt + 1);
      lb.load(kt + 1);
    }
    Mma<T, S>::ktile(acc, stage[cur], stage[cur] + S::BM * kRowBytes, p);
    if (more) {
      la.store(stage[cur ^ 1]);
      lb.store(stage[cur ^ 1] + S::BM * kRowBytes);
    }
    __syncthreads();
    after_ktile(kt);
  }
}

// ------------------------------------------------------- block -> tile map
// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2): hardware block b runs on XCD b % 8.  xcd_remap gives every XCD a
// contiguous range of logical block indices (a bijection on [0, nblocks)), so
// the tiles resident on one XCD at a time are neighbours in logical order.
__device__ __forceinline__ int xcd_remap(int b, int nblocks) {
  const int x = b & 7, k = b >> 3;
  const int q = nblocks >> 3, rem = nblocks & 7;
  return x * q + min(x, rem) + k;
}

// Logical index -> (tile row, tile col), walking `group_m` tile-rows at a time
// so that consecutive logical tiles share operand rows.
struct TileCoord {
  int m, n;
};
__device__ __forceinline__ TileCoord grouped_tile(int L, int tiles_m, int tiles_n, int group_m) {
  const int per_group = group_m * tiles_n;
  const int g = L / per_group;
  const int first_m = g * group_m;
  const int gm = min(group_m, tiles_m - first_m);
  const int in = L - g * per_group;
  TileCoord t;
  t.m = first_m + in % gm;
  t.n = in / gm;
  return t;
}

}  // namespace ttt
