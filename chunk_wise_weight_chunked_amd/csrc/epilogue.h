// epilogue.h -- device helpers shared by the GEMM epilogues of the layer's
// kernels: the token-column map of the chunk-padded token-major layouts, the
// k-blocked index, the LDS stage that turns a tile's columns into token runs
// (or column runs), and SiLU.
#pragma once

#include <hip/hip_runtime.h>

#include "gemm_core.h"
#include "layer.h"

namespace ttt {

// ------------------------------------------------------------ chunk columns
// Token row -> column of the token-major layouts (chunks padded to Cp
// columns).  ident: no padding and whole chunks (Cp = C, N C = T), where the
// column is the row itself.
struct ChunkMap {
  int32_t T, C, N, Cp;
  bool ident;
  __device__ __forceinline__ int64_t col(int32_t row) const {
    const int32_t b = row / T, s = row - b * T, i = s / C;
    return ((int64_t)b * N + i) * Cp + (s - i * C);
  }
};

__device__ __forceinline__ ChunkMap chunk_map(const Dims& dm) {
  ChunkMap m;
  m.T = (int32_t)dm.T;
  m.C = (int32_t)dm.C;
  m.N = (int32_t)dm.N;
  m.Cp = (int32_t)dm.Cp;
  m.ident = chunk_map_is_identity(dm);
  return m;
}

// Element index of (row n, token column p) in a k-blocked token-major matrix
// of R rows.
template <typename T>
__device__ __forceinline__ int64_t kblock_index(int64_t n, int64_t p, int64_t R) {
  constexpr int TB = kRowBytes / (int)sizeof(T);
  return ((p / TB) * R + n) * TB + (p % TB);
}

// LDS staging for the epilogues: a slice of COLS output columns x 256 tile
// rows (tokens), put by lanes 4 rows at a time, read back either as token runs
// (token-major outputs) or as column runs (row-major outputs).  Row stride of
// 260 elements keeps the 4-element puts of 16 lanes on distinct banks.  bf16
// results leave with non-temporal stores: nothing reads them back before L2
// would evict them anyway, and streaming them measured 3% faster on S1.
template <typename T, int NTHREADS, int COLS = 64>
struct Stage {
  static constexpr int kCols = COLS;
  static constexpr int kToks = 256;
  static constexpr int kStride = (kToks + 4) * (int)sizeof(T);  // bytes per LDS row
  static constexpr int TB = kRowBytes / (int)sizeof(T);
  static constexpr int kBytes = kCols * kStride;

  __device__ __forceinline__ static void put4(lds_char* lds, int col, int tok, const float v[4]) {
    lds_char* q = lds + col * kStride + tok * (int)sizeof(T);
    if constexpr (sizeof(T) == 2) {
      lds_store<u32x2_t>(q, u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])});
    } else {
      lds_store<floatx4_t>(q, floatx4_t{v[0], v[1], v[2], v[3]});
    }
  }

  // Two consecutive tokens (tok even) of one column.
  __device__ __forceinline__ static void put2(lds_char* lds, int col, int tok, float v0, float v1) {
    lds_char* q = lds + col * kStride + tok * (int)sizeof(T);
    if constexpr (sizeof(T) == 2) {
      lds_store<uint32_t>(q, pack_bf16x2(v0, v1));
    } else {
      lds_store<u32x2_t>(q, u32x2_t{__float_as_uint(v0), __float_as_uint(v1)});
    }
  }

  // Token-major, k-blocked output of R rows: tile token t of column c goes to
  // dst[kblock_index(col_base + c, column(row0 + t), R)].  Consecutive lanes
  // take 8-token runs of one column, then the next column, so a wave writes
  // contiguous 128-byte block rows.
  __device__ __forceinline__ static void flush_tokens(const lds_char* lds, T* __restrict__ dst,
                                                      int64_t R, int64_t col_base, int ncols,
                                                      int32_t row0, int32_t rows_total,
                                                      const ChunkMap& cm) {
    constexpr int GPB = TB / 8;  // 8-token runs per block row
    for (int it = threadIdx.x; it < kCols * (kToks / 8); it += NTHREADS) {
      const int g = it % GPB, c = (it / GPB) % kCols, tb = it / (GPB * kCols);
      const int tok = tb * TB + g * 8;
      const int32_t row = row0 + tok;
      if (c >= ncols || row >= rows_total) continue;
      const lds_char* src = lds + c * kStride + tok * (int)sizeof(T);
      const int64_t n = col_base + c;
      int64_t p0 = row;  // identity map: 8 rows of a whole chunk (T and C multiples of 64)
      int32_t room = 8;
      if (!cm.ident) {
        const int32_t b = row / cm.T, sq = row - b * cm.T, i = sq / cm.C, j = sq - i * cm.C;
        p0 = ((int64_t)b * cm.N + i) * cm.Cp + j;
        room = min(cm.C - j, cm.T - sq);
      }
      if (room >= 8 && (p0 & 7) == 0) {
        T* d = dst + kblock_index<T>(n, p0, R);
        if constexpr (sizeof(T) == 2) {
          const u32x2_t lo = lds_load<u32x2_t>(src);
          const u32x2_t hi = lds_load<u32x2_t>(src + 8);
          __builtin_nontemporal_store(u32x4_t{lo[0], lo[1], hi[0], hi[1]},
                                      reinterpret_cast<u32x4_t*>(d));
        } else {
          *reinterpret_cast<uint4*>(d) = as_uint4(lds_load<u32x4_t>(src));
          *reinterpret_cast<uint4*>(d + 4) = as_uint4(lds_load<u32x4_t>(src + 16));
        }
      } else {
        for (int e = 0; e < 8 && row + e < rows_total; ++e)
          dst[kblock_index<T>(n, cm.col(row + e), R)] = lds_load<T>(src + e * (int)sizeof(T));
      }
    }
  }

  // Row-major output: tile row t, column c goes to
  // dst[(dst_row0 + t) * ld + col_base + c] for rows_lo <= t < rows_valid,
  // c < ncols (a multiple of 8); 8 columns per store.
  __device__ __forceinline__ static void flush_rows(const lds_char* lds, T* __restrict__ dst,
                                                    int64_t dst_row0, int64_t ld,
                                                    int64_t col_base, int ncols, int32_t rows_lo,
                                                    int32_t rows_valid) {
    constexpr int kRuns = kCols / 8;  // 8-column runs per row
    for (int it = threadIdx.x; it < kToks * kRuns; it += NTHREADS) {
      const int t = it / kRuns, c = (it % kRuns) * 8;
      if (t < rows_lo || t >= rows_valid || c >= ncols) continue;
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        v[e] = Elem<T>::to_f32(lds_load<T>(lds + (c + e) * kStride + t * (int)sizeof(T)));
      T* d = dst + (dst_row0 + t) * ld + col_base + c;
      if constexpr (sizeof(T) == 2) {
        __builtin_nontemporal_store(u32x4_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                            pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])},
                                    reinterpret_cast<u32x4_t*>(d));
      } else {
        *reinterpret_cast<float4*>(d) = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4*>(d + 4) = make_float4(v[4], v[5], v[6], v[7]);
      }
    }
  }
};

// SiLU in fp32: x * sigmoid(x), with the hardware reciprocal (1 ulp).
__device__ __forceinline__ float silu(float x) {
  return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

}  // namespace ttt
