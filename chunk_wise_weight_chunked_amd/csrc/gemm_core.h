// gemm_core.h -- the MFMA/LDS GEMM mainloop shared by the four contractions of
// the TTT-MLP layer on CDNA4 (gfx950).
//
// Every contraction of the layer is put in "both operands K-contiguous" form,
//     acc[m][n] += sum_k A[m][k] * B[n][k],
// so one mainloop serves all of them; the kernels differ only in how the
// operand rows are found (row loaders) and what happens to the accumulator
// (epilogues).
//
// Tile geometry (one workgroup = WAVES_M x WAVES_N wave64s):
//   * BM x BN output tile, each wave owns (BM/WAVES_M) x (BN/WAVES_N) as 32x32
//     MFMA blocks;
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

constexpr int kRowBytes = 128;    // bytes of K per operand row per k-tile
constexpr int kChunks = 8;        // 16-byte chunks per row per k-tile
constexpr int kTokenAlign = 64;   // chunk padding in the token-major layouts

// ----------------------------------------------------------------- numbers
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
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
// LDS is addressed through address-space-3 pointers so that every access
// compiles to ds_read / ds_write (a generic pointer would give flat accesses,
// which also count against the vector-memory counter and serialise the
// global prefetch with the LDS reads).
typedef __attribute__((address_space(3))) char lds_char;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// V: a scalar or clang ext_vector type (HIP's vector classes are not
// address-space aware; convert with the helpers below).
template <typename V>
__device__ __forceinline__ V lds_load(const lds_char* p) {
  return *(const __attribute__((address_space(3))) V*)p;
}
template <typename V>
__device__ __forceinline__ void lds_store(lds_char* p, V v) {
  *(__attribute__((address_space(3))) V*)p = v;
}
__device__ __forceinline__ u32x4_t as_u32x4(const uint4& v) { return u32x4_t{v.x, v.y, v.z, v.w}; }
__device__ __forceinline__ uint4 as_uint4(const u32x4_t& v) { return make_uint4(v[0], v[1], v[2], v[3]); }

#ifndef TTT_LDS_SWZ_SHIFT
#define TTT_LDS_SWZ_SHIFT 1
#endif
__device__ __forceinline__ int lds_swz(int row) { return (row >> TTT_LDS_SWZ_SHIFT) & 7; }
__device__ __forceinline__ uint32_t lds_offset(int row, int chunk) {
  return (uint32_t)row * kRowBytes + (uint32_t)((chunk ^ lds_swz(row)) << 4);
}

// A k-major operand tile (rows = k, 128-byte rows of 64 m-values) is read with
// transposed loads that take four consecutive rows at a time; this swizzle
// puts rows r and r + 2 (same bank half) on opposite halves of the 8 chunk
// slots, so each half-wave of such a load hits every bank once.
__device__ __forceinline__ int lds_swz_tr(int row) {
  return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

// ------------------------------------------------------------- tile shapes
template <int BM_, int BN_, int WAVES_M_, int WAVES_N_>
struct TileShape {
  static constexpr int BM = BM_;
  static constexpr int BN = BN_;
  static constexpr int WAVES_M = WAVES_M_;
  static constexpr int WAVES_N = WAVES_N_;
  static constexpr int kWaves = WAVES_M * WAVES_N;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int WM = BM / WAVES_M;  // wave sub-tile rows
  static constexpr int WN = BN / WAVES_N;  // wave sub-tile cols
  static constexpr int MB = WM / 32;       // 32x32 blocks per wave, rows
  static constexpr int NB = WN / 32;       // 32x32 blocks per wave, cols
  static constexpr int kStageBytes = (BM + BN) * kRowBytes;
  static constexpr int kLdsBytes = 2 * kStageBytes;
  static_assert(WM % 32 == 0 && WN % 32 == 0, "waves hold whole 32x32 blocks");
  static_assert(BM % (8 * kWaves) == 0 && BN % (8 * kWaves) == 0,
                "each wave loads whole 8-row groups");
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
  p.wave_m0 = (wave / S::WAVES_N) * S::WM;
  p.wave_n0 = (wave % S::WAVES_N) * S::WN;
  p.lane = threadIdx.x & 63;
  return p;
}

// ---------------------------------------------------------- fragment + MFMA
template <typename T, class S>
struct Mma;

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

// A fragment i of step s from a k-major A tile: stage row R = (m / 64) * 64 + k
// holds the 64 m-values [64 (m / 64), + 64) of k-tile column k, chunk c at
// c ^ lds_swz_tr(R).  ds_read_b64_tr_b16 works on groups of 16 lanes: lane j
// of a group gives the address of 4 consecutive values, and lane j receives
// value j % 4 of the words lanes j / 4, 4 + j / 4, 8 + j / 4 and 12 + j / 4
// addressed.  With lane j addressing k-row kb + j / 4 at m-values
// mb + 4 (j % 4) .. + 3, lane j receives k-rows kb .. kb + 3 of column mb + j.
// Lane l of the wave needs row m = l % 32 of the fragment and k values
// 8 (l / 32) .. + 7: group g = l / 16 takes mb = 16 (g % 2) and kb = 8 (g / 2),
// two loads (kb and kb + 4) per fragment.
__device__ __forceinline__ bf16x8_t read_a_tr(const lds_char* sA, int m0, int lane, int s) {
  const int g = lane >> 4, j = lane & 15;
  const int m = m0 + 16 * (g & 1) + 4 * (j & 3);  // m-values m .. m + 3 of this lane's word
  const int k = 16 * s + 8 * (g >> 1) + (j >> 2);
  bf16x4_t v[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int R = (m >> 6) * 64 + k + 4 * h;
    const uint32_t off = (uint32_t)R * kRowBytes +
                         (uint32_t)(((((m & 63) >> 3) ^ lds_swz_tr(R))) << 4) + (uint32_t)((m & 7) * 2);
    v[h] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (__attribute__((address_space(3))) bf16x4_t*)(sA + off));
  }
  return bf16x8_t{v[0][0], v[0][1], v[0][2], v[0][3], v[1][0], v[1][1], v[1][2], v[1][3]};
}

template <class S, bool kTrA = false, bool kTrB = false>
struct Mma16 {
  static constexpr int kSteps = 4;  // 16 K values per step, 64 per k-tile
  struct Frag {
    bf16x8_t a[S::MB], b[S::NB];
  };
  __device__ __forceinline__ static bf16x8_t read_a(const lds_char* sA, const LanePos& p, int i,
                                                    int s) {
    if constexpr (kTrA)
      return read_a_tr(sA, p.wave_m0 + 32 * i, p.lane, s);
    else
      return lds_load<bf16x8_t>(sA + lds_offset(p.wave_m0 + 32 * i + (p.lane & 31),
                                                2 * s + (p.lane >> 5)));
  }
  __device__ __forceinline__ static bf16x8_t read_b(const lds_char* sB, const LanePos& p, int j,
                                                    int s) {
    if constexpr (kTrB)
      return read_a_tr(sB, p.wave_n0 + 32 * j, p.lane, s);
    else
      return lds_load<bf16x8_t>(sB + lds_offset(p.wave_n0 + 32 * j + (p.lane & 31),
                                                2 * s + (p.lane >> 5)));
  }
  __device__ __forceinline__ static void read(Frag& f, const lds_char* sA, const lds_char* sB,
                                              const LanePos& p, int s) {
#pragma unroll
    for (int i = 0; i < S::MB; ++i) f.a[i] = read_a(sA, p, i, s);
#pragma unroll
    for (int j = 0; j < S::NB; ++j) f.b[j] = read_b(sB, p, j, s);
  }
  // The fragments of step s+1 are read while the MFMAs of step s run.  The
  // scheduling barriers pin that order (otherwise the compiler sinks each read
  // down to its first use and the MFMAs wait on LDS latency every time).
  // mid() runs between the two halves of the steps (the mainloop stages the
  // next k-tile there).
  template <class Mid>
  __device__ __forceinline__ static void ktile(Accum<S>& acc, const lds_char* sA,
                                               const lds_char* sB, const LanePos& p, Mid&& mid) {
    Frag f[2];
    read(f[0], sA, sB, p, 0);
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      if (s + 1 < kSteps) read(f[(s + 1) & 1], sA, sB, p, s + 1);
      __builtin_amdgcn_sched_barrier(0);
      const Frag& c = f[s & 1];
#pragma unroll
      for (int i = 0; i < S::MB; ++i)
#pragma unroll
        for (int j = 0; j < S::NB; ++j)
          acc.v[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(c.a[i], c.b[j], acc.v[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (s == kSteps / 2 - 1) {
        mid();
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  // The same k-tile with the fragment reads of step s+1 spread between the
  // MFMAs of step s (read m after MFMA m) and a hook after every MFMA, called
  // with the MFMA's index in the k-tile (a constant once unrolled); the
  // mainloop issues the next k-tile's global reads from it.  Issued in one
  // group, the reads and loads of all eight waves queue behind each other and
  // hold up the MFMAs that follow them.
  template <class Hook>
  __device__ __forceinline__ static void ktile_spread(Accum<S>& acc, const lds_char* sA,
                                                      const lds_char* sB, const LanePos& p,
                                                      Hook&& after_mfma) {
    constexpr int kPerStep = S::MB * S::NB;
    Frag f[2];
    read(f[0], sA, sB, p, 0);
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      __builtin_amdgcn_sched_barrier(0);
      const Frag& c = f[s & 1];
      Frag& n = f[(s + 1) & 1];
#pragma unroll
      for (int i = 0; i < S::MB; ++i)
#pragma unroll
        for (int j = 0; j < S::NB; ++j) {
          acc.v[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(c.a[i], c.b[j], acc.v[i][j], 0, 0, 0);
          const int m = i * S::NB + j;
          if (s + 1 < kSteps) {
            // fragment reads of step s+1 due after this MFMA (the last MFMA
            // of the step takes whatever is left)
#pragma unroll
            for (int q = 0; q < S::MB + S::NB; ++q) {
              if (q == m || (m == kPerStep - 1 && q > m)) {
                if (q < S::MB)
                  n.a[q] = read_a(sA, p, q, s + 1);
                else
                  n.b[q - S::MB] = read_b(sB, p, q - S::MB, s + 1);
              }
            }
          }
          after_mfma(s * kPerStep + m);
          __builtin_amdgcn_sched_barrier(0);
        }
    }
  }
};

template <class S>
struct Mma<uint16_t, S> : Mma16<S, false> {};

// fp32: v_mfma_f32_32x32x2_f32, eight per 16 K values; lane l feeds K value
// 16 s + 8 (l / 32) + e of its row to MFMA e of step s, on both sides.  A
// k-major tile (rows = k, 128-byte rows of 32 m-values: stage row
// R = (m / 32) * 32 + k, chunk c at c ^ lds_swz_tr(R)) is read one value per
// lane and MFMA.
template <class S, bool kTrA = false, bool kTrB = false>
struct Mma32 {
  static constexpr int kSteps = 2;  // 16 K values per step, 32 per k-tile
  template <bool kKMajor>
  __device__ __forceinline__ static void read8(float v[8], const lds_char* sX, int row, int lane,
                                               int s) {
    const int h = lane >> 5;
    if constexpr (kKMajor) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int R = (row >> 5) * 32 + 16 * s + 8 * h + e;
        v[e] = lds_load<float>(sX + (uint32_t)R * kRowBytes +
                               (uint32_t)((((row & 31) >> 2) ^ lds_swz_tr(R)) << 4) +
                               (uint32_t)((row & 3) * 4));
      }
    } else {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const floatx4_t x = lds_load<floatx4_t>(sX + lds_offset(row, 4 * s + 2 * h + q));
#pragma unroll
        for (int e = 0; e < 4; ++e) v[4 * q + e] = x[e];
      }
    }
  }
  template <class Mid>
  __device__ __forceinline__ static void ktile(Accum<S>& acc, const lds_char* sA,
                                               const lds_char* sB, const LanePos& p, Mid&& mid) {
    const int r = p.lane & 31;
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      float a[S::MB][8], b[S::NB][8];
#pragma unroll
      for (int i = 0; i < S::MB; ++i) read8<kTrA>(a[i], sA, p.wave_m0 + 32 * i + r, p.lane, s);
#pragma unroll
      for (int j = 0; j < S::NB; ++j) read8<kTrB>(b[j], sB, p.wave_n0 + 32 * j + r, p.lane, s);
#pragma unroll
      for (int i = 0; i < S::MB; ++i)
#pragma unroll
        for (int j = 0; j < S::NB; ++j)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            acc.v[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i][e], b[j][e], acc.v[i][j], 0, 0, 0);
      if (s == kSteps / 2 - 1) mid();
    }
  }
};

template <class S>
struct Mma<float, S> : Mma32<S, false, false> {};

// The fragment reader of element type T with the given operand forms.
template <typename T, class S, bool kTrA, bool kTrB>
struct MmaSel;
template <class S, bool kTrA, bool kTrB>
struct MmaSel<uint16_t, S, kTrA, kTrB> {
  using type = Mma16<S, kTrA, kTrB>;
};
template <class S, bool kTrA, bool kTrB>
struct MmaSel<float, S, kTrA, kTrB> {
  using type = Mma32<S, kTrA, kTrB>;
};

// ------------------------------------------------------------- row loaders
// Global reads use buffer loads: a scalar resource (base, byte range) per
// operand and k-tile, a per-lane 32-bit offset.  Reads at or beyond the range
// return zero, which is how rows outside the operand are masked (no branches),
// and buffer loads are counted by vmcnt only, so the next k-tile's loads stay
// in flight while the MFMAs consume LDS.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOobOffset = 0x80000000u;  // beyond any range used here

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int64_t n = bytes < 0 ? 0 : (bytes > 0x7fffffffLL ? 0x7fffffffLL : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n,
                                           0x00020000);
}

// s_waitcnt on the vector-memory counter only: vmcnt(N), N a constant.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Loader interface used by the mainloops: issue(kt, stage) starts the
// direct-to-LDS reads of k-tile kt into `stage`; rsrc(kt, live) and
// issue_one(r, stage, q) issue them one instruction at a time.
//
// DirectLoader moves one operand's k-tile (ROWS rows x 128 bytes) with
// buffer_load ... lds (no registers): wave w of WAVES fills rows
// [w ROWS/WAVES, (w+1) ROWS/WAVES) of the stage, 8 rows (1 KB) per instruction, lane l writing 16 bytes at
// lane * 16 of that KB.  The swizzled layout (row r, chunk c at c ^ (r & 7)) is
// produced by choosing the source: lane l reads chunk (l & 7) ^ (l >> 3) of
// row l >> 3 of its group.  Addressing, in bytes and uniform across the
// workgroup:
//   row r, k-tile kt  ->  base + kt * kt_stride + r * row_stride + chunk * 16,
//   valid while the offset from base + kt * kt_stride is below
//   valid_bytes - kt * kt_shrink (reads beyond return zero).
// Row-major operands use row_stride = row length, kt_stride = kt_shrink = 128;
// k-blocked operands ([K/kt][rows][128 B]) use row_stride = 128,
// kt_stride = rows * 128, kt_shrink = 0.
template <int ROWS, int WAVES>
struct DirectLoader {
  static constexpr int kRowsPerWave = ROWS / WAVES;
  static constexpr int kPer = kRowsPerWave / 8;  // instructions per wave per k-tile
  const char* base;
  int64_t kt_stride, valid_bytes, kt_shrink;
  uint32_t voff[kPer];
  uint32_t lds_row0;  // first stage row of this wave

  __device__ __forceinline__ void init(const void* base_, int64_t row_stride, int64_t kt_stride_,
                                       int64_t valid_bytes_, int64_t kt_shrink_) {
    base = static_cast<const char*>(base_);
    kt_stride = kt_stride_;
    valid_bytes = valid_bytes_;
    kt_shrink = kt_shrink_;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    lds_row0 = (uint32_t)(wave * kRowsPerWave);
    const int rr = lane >> 3;
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int row = (int)lds_row0 + 8 * q + rr;
      const int c = (lane & 7) ^ lds_swz(row);  // source chunk landing at chunk lane & 7
      voff[q] = (uint32_t)(row * row_stride + c * 16);
    }
  }
  // Rows grouped in blocks of `block_rows` rows of 128 bytes each, blocks
  // `block_stride` bytes apart (tiled operands): row r at
  // (r / block_rows) block_stride + (r % block_rows) 128.
  __device__ __forceinline__ void init_blocked(const void* base_, int block_rows,
                                               int64_t block_stride, int64_t kt_stride_,
                                               int64_t valid_bytes_, int64_t kt_shrink_) {
    base = static_cast<const char*>(base_);
    kt_stride = kt_stride_;
    valid_bytes = valid_bytes_;
    kt_shrink = kt_shrink_;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    lds_row0 = (uint32_t)(wave * kRowsPerWave);
    const int rr = lane >> 3;
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int row = (int)lds_row0 + 8 * q + rr;
      const int c = (lane & 7) ^ lds_swz(row);
      voff[q] = (uint32_t)((row / block_rows) * block_stride + (row % block_rows) * kRowBytes +
                           c * 16);
    }
  }
  // Descriptor of k-tile kt; live = false gives an empty range (every read
  // returns zero).
  __device__ __forceinline__ rsrc_t rsrc(int64_t kt, bool live = true) const {
    return make_rsrc(base + kt * kt_stride, live ? valid_bytes - kt * kt_shrink : 0);
  }
  // Instruction q (0..kPer-1) of a k-tile: 8 rows into `stage`.
  __device__ __forceinline__ void issue_one(rsrc_t r, lds_char* stage, int q) const {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void*)(stage + (lds_row0 + 8 * q) * kRowBytes), 16,
        voff[q], 0, 0, 0);
  }
  __device__ __forceinline__ void issue(int64_t kt, lds_char* stage) {
    const rsrc_t r = rsrc(kt);
#pragma unroll
    for (int q = 0; q < kPer; ++q) issue_one(r, stage, q);
  }
};

// KMajorLoader: a k-major operand tile of 256 m-values (m: the tile's output
// rows or columns) and one k-tile of TB = 128 / sizeof(T) k-values.  Stage
// row R = (m / TB) * TB + k holds the TB values m = TB (R / TB) .. + TB - 1 of
// k-tile row k (128 bytes), chunk c at c ^ lds_swz_tr(R); the fragment readers
// with kTrA / kTrB read it.  Source addressing, in bytes from base:
//   m-block mb = m / TB, k-tile kt, row k  ->  mb * block_stride + kt * kt_stride
//                                             + k * row_stride,
// e.g. a row-major [K][ld] matrix: block_stride = 128, row_stride = ld bytes,
// kt_stride = TB * row_stride; the k-blocked token-major layouts (blocks of
// 64 token columns, R rows of 128 bytes each): block_stride = R * 128,
// row_stride = 128, kt_stride = 64 * 128.  Reads at or beyond valid_bytes -
// kt * kt_stride from base + kt * kt_stride return zero.
template <typename T, int WAVES>
struct KMajorLoader {
  static constexpr int TB = kRowBytes / (int)sizeof(T);
  static constexpr int kRowsPerWave = 256 / WAVES;
  static constexpr int kPer = kRowsPerWave / 8;
  const char* base;
  int64_t kt_stride, valid_bytes;
  uint32_t voff[kPer];
  uint32_t lds_row0;

  __device__ __forceinline__ void init(const void* base_, int64_t block_stride,
                                       int64_t row_stride, int64_t kt_stride_,
                                       int64_t valid_bytes_) {
    base = static_cast<const char*>(base_);
    kt_stride = kt_stride_;
    valid_bytes = valid_bytes_;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    lds_row0 = (uint32_t)(wave * kRowsPerWave);
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int row = (int)lds_row0 + 8 * q + (lane >> 3);
      const int c = (lane & 7) ^ lds_swz_tr(row);
      voff[q] = (uint32_t)((row / TB) * block_stride + (row % TB) * row_stride + c * 16);
    }
  }
  __device__ __forceinline__ rsrc_t rsrc(int64_t kt, bool live = true) const {
    return make_rsrc(base + kt * kt_stride, live ? valid_bytes - kt * kt_stride : 0);
  }
  __device__ __forceinline__ void issue_one(rsrc_t r, lds_char* stage, int q) const {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void*)(stage + (lds_row0 + 8 * q) * kRowBytes), 16,
        voff[q], 0, 0, 0);
  }
  __device__ __forceinline__ void issue(int64_t kt, lds_char* stage) {
    const rsrc_t r = rsrc(kt);
#pragma unroll
    for (int q = 0; q < kPer; ++q) issue_one(r, stage, q);
  }
};

// ---------------------------------------------------------------- mainloop
// Runs k-tiles [0, nk) through a two-stage LDS pipeline.  Entering k-tile kt
// (after a barrier), stage kt&1 holds k-tile kt and the other stage is free:
// the loaders start k-tile kt+1 into it (bf16 with kSpread: spread over kt's
// MFMAs; otherwise at once, in one group).  Before the closing barrier every
// wave waits for its own reads of k-tile kt+1.  after_ktile(kt) runs once
// every wave has finished k-tile kt and no read is in flight (it may use
// registers and global memory, not LDS).
// kTrA (bf16 only): the A tile is k-major (see read_a_tr) and its fragments
// are read with transposed loads.  kEveryWant (bf16 spread issue): one load
// every kEveryWant MFMAs; 0 takes every second MFMA when the loads then still
// end in the first half of the k-tile, else every MFMA.
template <typename T, class S, bool kSpread = true, bool kTrA = false, bool kTrB = false,
          int kEveryWant = 0, class LA, class LB, class Hook>
__device__ __forceinline__ void mainloop(Accum<S>& acc, LA& la, LB& lb, int64_t nk, lds_char* smem,
                                         const LanePos& p, Hook&& after_ktile) {
  static_assert(sizeof(T) == 4 || !(kTrA || kTrB) || kSpread,
                "bf16 k-major fragments: spread issue");
  if (nk <= 0) return;
  if constexpr (kSpread && sizeof(T) == 2) {
    // bf16: k-tile kt+1's load instructions are spread over
    // k-tile kt's MFMAs, one every kEvery MFMAs from the first.  After the
    // last k-tile they read an empty range into the idle stage; the closing
    // wait drains them before the caller touches LDS.
    using M = Mma16<S, kTrA, kTrB>;
    constexpr int kLoads = LA::kPer + LB::kPer;
    constexpr int kMfmas = M::kSteps * S::MB * S::NB;
    constexpr int kEvery = kEveryWant > 0 ? kEveryWant : (2 * kLoads <= kMfmas / 2 ? 2 : 1);
    static_assert(kLoads * kEvery <= kMfmas, "the loads fit the k-tile's MFMAs");
    la.issue(0, smem);
    lb.issue(0, smem + S::BM * kRowBytes);
    wait_vmcnt<0>();
    __syncthreads();
    for (int64_t kt = 0; kt < nk; ++kt) {
      const lds_char* cur = smem + (kt & 1) * S::kStageBytes;
      lds_char* nxt = smem + ((kt + 1) & 1) * S::kStageBytes;
      const bool more = kt + 1 < nk;
      const rsrc_t ra = la.rsrc(kt + 1, more), rb = lb.rsrc(kt + 1, more);
      M::ktile_spread(acc, cur, cur + S::BM * kRowBytes, p, [&](int idx) {
        if (idx % kEvery == 0 && idx / kEvery < kLoads) {
          const int q = idx / kEvery;
          if (q < LA::kPer)
            la.issue_one(ra, nxt, q);
          else
            lb.issue_one(rb, nxt + S::BM * kRowBytes, q - LA::kPer);
        }
      });
      wait_vmcnt<0>();
      __syncthreads();
      after_ktile(kt);
    }
    return;
  }
  // fp32, or bf16 without kSpread: k-tile kt+1's loads in one group at the
  // start of k-tile kt
  la.issue(0, smem);
  lb.issue(0, smem + S::BM * kRowBytes);
  wait_vmcnt<0>();
  __syncthreads();
  for (int64_t kt = 0; kt < nk; ++kt) {
    const lds_char* cur = smem + (kt & 1) * S::kStageBytes;
    lds_char* nxt = smem + ((kt + 1) & 1) * S::kStageBytes;
    if (kt + 1 < nk) {
      la.issue(kt + 1, nxt);
      lb.issue(kt + 1, nxt + S::BM * kRowBytes);
    }
    MmaSel<T, S, kTrA, kTrB>::type::ktile(acc, cur, cur + S::BM * kRowBytes, p, [] {});
    wait_vmcnt<0>();
    __syncthreads();
    after_ktile(kt);
  }
}

// A workgroup barrier for LDS only.  __syncthreads() also releases global
// memory, and the compiler puts a wait for every outstanding vector memory
// operation (stores included) in front of it.  Here: this wave's LDS
// operations complete (lgkmcnt(0)), then s_barrier, with compiler-level
// memory barriers on both sides so no access moves across.  Direct-to-LDS
// loads are not covered: callers wait for them (vmcnt) before calling.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt not waited
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The mainloop of a tile that stores part of its accumulator to global memory
// between k-tiles (the prefix scan's weight slots).  before_ktile(kt) runs
// before k-tile kt's MFMAs, while the accumulator holds the sum over k-tiles
// [0, kt), and issues the stores when kt starts a chunk.  bf16: k-tile kt+1's
// loads are then spread over kt's MFMAs (one every kEvery MFMAs, as in
// mainloop); fp32: issued in one group before the stores.  Every k-tile ends
// with vmcnt(0): the stores drain within the k-tile that issues them and no
// vector-memory operation is in flight at the barrier.  kmap(kt) is the
// loaders' k-tile for step kt (the identity, or another order of the same
// k-tiles).
template <typename T, class S, class LA, class LB, class Hook, class KMap>
__device__ __forceinline__ void mainloop_with_stores(Accum<S>& acc, LA& la, LB& lb, int64_t nk,
                                                     lds_char* smem, const LanePos& p,
                                                     Hook&& before_ktile, KMap&& kmap) {
  if (nk <= 0) return;
  la.issue(kmap(0), smem);
  lb.issue(kmap(0), smem + S::BM * kRowBytes);
  wait_vmcnt<0>();
  __syncthreads();
  for (int64_t kt = 0; kt < nk; ++kt) {
    const lds_char* cur = smem + (kt & 1) * S::kStageBytes;
    lds_char* nxt = smem + ((kt + 1) & 1) * S::kStageBytes;
    const bool more = kt + 1 < nk;
    if constexpr (sizeof(T) == 2) {
      using M = Mma16<S, false, false>;
      constexpr int kLoads = LA::kPer + LB::kPer;
      constexpr int kMfmas = M::kSteps * S::MB * S::NB;
      constexpr int kEvery = 2 * kLoads <= kMfmas / 2 ? 2 : 1;
      static_assert(kLoads <= kMfmas, "one load instruction per MFMA at most");
      before_ktile(kt);
      const rsrc_t ra = la.rsrc(kmap(kt + 1), more), rb = lb.rsrc(kmap(kt + 1), more);
      M::ktile_spread(acc, cur, cur + S::BM * kRowBytes, p, [&](int idx) {
        if (idx % kEvery == 0 && idx / kEvery < kLoads) {
          const int q = idx / kEvery;
          if (q < LA::kPer)
            la.issue_one(ra, nxt, q);
          else
            lb.issue_one(rb, nxt + S::BM * kRowBytes, q - LA::kPer);
        }
      });
    } else {
      if (more) {
        la.issue(kmap(kt + 1), nxt);
        lb.issue(kmap(kt + 1), nxt + S::BM * kRowBytes);
      }
      before_ktile(kt);
      Mma<T, S>::ktile(acc, cur, cur + S::BM * kRowBytes, p, [] {});
    }
    wait_vmcnt<0>();
    lds_barrier();
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
