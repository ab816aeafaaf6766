// gemm.hip -- batched GEMM on the library's MFMA mainloop (gemm_core.h), for
// the plain products of the layer's backward pass.
//
// C[b] = alpha * A[b] B[b]ᵀ (or C[b] += ...), with A [M][K] and B [N][K] in
// the mainloop's "both operands K-contiguous" sense.  Either operand may
// instead be stored k-major -- [K][M] (resp. [K][N]) row-major, or in TB x TB
// tiles of such a matrix -- and is then loaded as k-major tiles
// (KMajorLoader) and read with transposed fragment loads (bf16) or one value
// per lane (fp32).  The layouts are listed with GemmLayout (layer.h).  A
// second product of the same output shape can share the accumulators:
// C[b] = alpha (A[b] B[b]ᵀ + alpha2 A2[b] B2[b]ᵀ), written once.  The batch index walks independent products (the chunks of
// a sequence, or the K slices of a split product whose partial results the
// caller adds in order).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "epilogue.h"
#include "gemm_core.h"
#include "layer.h"

namespace ttt {
namespace {

using GTile = TileShape<256, 256, 2, 4>;

// Rows [0, 256) x columns [64 q, 64 q + 64) of the accumulator into an LDS
// stage of fp32 values, then out to C in 8-element runs.  Row stride 72
// floats: the two half-waves of a put (rows 4 apart) land on opposite halves
// of the 64 banks.
constexpr int kEpiCols = 64;
constexpr int kEpiStride = kEpiCols + 8;  // floats per staged row

template <typename Tc>
__device__ __forceinline__ void store8(Tc* dst, const float v[8], bool accumulate);
template <>
__device__ __forceinline__ void store8<float>(float* dst, const float v[8], bool accumulate) {
  float4 lo = make_float4(v[0], v[1], v[2], v[3]), hi = make_float4(v[4], v[5], v[6], v[7]);
  if (accumulate) {
    const float4 a = *reinterpret_cast<const float4*>(dst);
    const float4 b = *reinterpret_cast<const float4*>(dst + 4);
    lo = make_float4(a.x + lo.x, a.y + lo.y, a.z + lo.z, a.w + lo.w);
    hi = make_float4(b.x + hi.x, b.y + hi.y, b.z + hi.z, b.w + hi.w);
  }
  *reinterpret_cast<float4*>(dst) = lo;
  *reinterpret_cast<float4*>(dst + 4) = hi;
}
template <>
__device__ __forceinline__ void store8<uint16_t>(uint16_t* dst, const float v[8], bool) {
  *reinterpret_cast<uint4*>(dst) = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                              pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
}

template <class S, typename Tc>
__device__ __forceinline__ void gemm_epilogue(const Accum<S>& acc, const LanePos& p, lds_char* smem,
                                              Tc* __restrict__ C, int64_t ldc, int64_t m0,
                                              int64_t n0, int64_t M, int64_t N, float alpha,
                                              bool accumulate) {
  for (int q = 0; q < S::BN / kEpiCols; ++q) {
    __syncthreads();  // the mainloop's (or the previous pass's) reads of LDS are done
#pragma unroll
    for (int j = 0; j < S::NB; ++j) {
      const int col = p.wave_n0 + 32 * j;
      if (col < kEpiCols * q || col >= kEpiCols * q + kEpiCols) continue;
      const int c = col - kEpiCols * q + (p.lane & 31);
#pragma unroll
      for (int i = 0; i < S::MB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          lds_store<float>(smem + ((uint32_t)p.row(i, r) * kEpiStride + c) * 4,
                           alpha * acc.v[i][j][r]);
    }
    __syncthreads();
    const int64_t cb = n0 + kEpiCols * q;
    for (int it = threadIdx.x; it < S::BM * (kEpiCols / 8); it += S::kThreads) {
      const int t = it / (kEpiCols / 8), c = (it % (kEpiCols / 8)) * 8;
      if (m0 + t >= M || cb + c >= N) continue;
      const floatx4_t lo = lds_load<floatx4_t>(smem + ((uint32_t)t * kEpiStride + c) * 4);
      const floatx4_t hi = lds_load<floatx4_t>(smem + ((uint32_t)t * kEpiStride + c + 4) * 4);
      const float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      store8<Tc>(C + (m0 + t) * ldc + cb + c, v, accumulate);
    }
  }
}

// Operand loaders of batch b for a tile starting at row r0 (m0 for A, n0 for
// B), contracting K values:
// row-major [rows][ld] with K contiguous: rows beyond the operand's row count
// read zero (K is a multiple of TB here); k-major [K][ld]: rows beyond K read
// zero -- the range ends with row K - 1 of the batch's matrix, whose first
// column may sit partway across a stored row (a batch offset that is not
// whole rows); k-blocked: rows beyond the block's ld rows read zero (a
// batch's row offset counted), K is whole blocks; tiled (TB x TB tiles of
// 128-byte rows, whole matrices per batch, row count and ld multiples of TB):
// K-contiguous -- a k-tile of the tile's rows is one tile from each of its
// TB-row blocks; k-major -- a k-tile is consecutive tiles of one tile row.
template <typename T, int kL, int kRows>
__device__ __forceinline__ auto make_loader(const char* X, int64_t ld, int64_t sx, int64_t b,
                                            int64_t r0, int64_t rows, int64_t K) {
  constexpr int64_t es = sizeof(T);
  constexpr int TB = kRowBytes / (int)sizeof(T);
  constexpr int64_t kTileBytes = (int64_t)TB * kRowBytes;
  constexpr int kWaves = GTile::kWaves;
  if constexpr (kL == kKMajor) {
    const int64_t col = (b * sx) % ld + r0;  // column of the tile's first row
    KMajorLoader<T, kWaves> l;
    l.init(X + r0 * es, kRowBytes, ld * es, TB * ld * es, (K * ld - col) * es);
    return l;
  } else if constexpr (kL == kTiledKMajor) {
    KMajorLoader<T, kWaves> l;
    l.init(X + (r0 / TB) * kTileBytes, kTileBytes, kRowBytes, ld * kRowBytes,
           (K * ld - r0 * TB) * es);
    return l;
  } else if constexpr (kL == kKBlocked) {
    const int64_t row = (b * sx / TB) % ld + r0;
    DirectLoader<kRows, kWaves> l;
    l.init(X + r0 * kRowBytes, kRowBytes, ld * kRowBytes, (ld - row) * kRowBytes, 0);
    return l;
  } else if constexpr (kL == kTiledRowK) {
    DirectLoader<kRows, kWaves> l;
    l.init_blocked(X + (r0 / TB) * ld * kRowBytes, TB, ld * kRowBytes, kTileBytes,
                   ((rows - r0) / TB) * ld * kRowBytes, kTileBytes);
    return l;
  } else {
    DirectLoader<kRows, kWaves> l;
    l.init(X + r0 * ld * es, ld * es, kRowBytes, (rows - r0) * ld * es, kRowBytes);
    return l;
  }
}

constexpr bool is_kmajor(int l) { return l == kKMajor || l == kTiledKMajor; }

// The batched products issue one next-k-tile load per MFMA: their operands
// (per-chunk weights and gradient sums, k-blocked copies) mostly stream from
// HBM, and issuing the loads early measured faster (the 32K backward 22.41 ->
// 21.86 ms) than one every second MFMA.
constexpr int kGemmEvery = 1;

// The tile's position: batch b and the first row and column of the tile.
struct GemmTilePos {
  int64_t b, m0, n0;
};

template <class S>
__device__ __forceinline__ GemmTilePos gemm_tile_pos(const GemmArgs& g) {
  const int tiles_m = (int)((g.M + S::BM - 1) / S::BM);
  const int tiles_n = (int)((g.N + S::BN - 1) / S::BN);
  const int per_batch = tiles_m * tiles_n;
  const int L = xcd_remap(blockIdx.x, (int)gridDim.x);
  const int64_t b = L / per_batch;
  const TileCoord tc = grouped_tile(L - (int)b * per_batch, tiles_m, tiles_n, 8);
  return GemmTilePos{b, (int64_t)tc.m * S::BM, (int64_t)tc.n * S::BN};
}

// acc = A[b] B[b]ᵀ of g for the tile at t; with kLA2 >= 0, the second
// product (g2's A, B, K and alpha; g's M, N and batch) runs first on the
// same accumulators, which are then scaled by g2.alpha.
template <typename T, int kLA, int kLB, int kLA2, int kLB2, class S>
__device__ __forceinline__ void gemm_accumulate(const GemmArgs& g, const GemmArgs& g2,
                                                const GemmTilePos& t, Accum<S>& acc,
                                                lds_char* smem, const LanePos& p) {
  constexpr int64_t es = sizeof(T);
  constexpr int TB = kRowBytes / (int)sizeof(T);
  const int64_t b = t.b;
  acc.zero();
  if constexpr (kLA2 >= 0) {
    const int64_t K2 = b + 1 == g2.batch ? g2.K_last : g2.K;
    auto la = make_loader<T, kLA2, S::BM>(static_cast<const char*>(g2.A) + b * g2.sa * es, g2.lda,
                                          g2.sa, b, t.m0, g.M, K2);
    auto lb = make_loader<T, kLB2, S::BN>(static_cast<const char*>(g2.B) + b * g2.sb * es, g2.ldb,
                                          g2.sb, b, t.n0, g.N, K2);
    mainloop<T, S, true, is_kmajor(kLA2), is_kmajor(kLB2), kGemmEvery>(acc, la, lb, (K2 + TB - 1) / TB, smem,
                                                           p, [](int64_t) {});
#pragma unroll
    for (int i = 0; i < S::MB; ++i)
#pragma unroll
      for (int j = 0; j < S::NB; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc.v[i][j][r] *= g2.alpha;
  }
  const int64_t K = b + 1 == g.batch ? g.K_last : g.K;
  auto la = make_loader<T, kLA, S::BM>(static_cast<const char*>(g.A) + b * g.sa * es, g.lda, g.sa,
                                       b, t.m0, g.M, K);
  auto lb = make_loader<T, kLB, S::BN>(static_cast<const char*>(g.B) + b * g.sb * es, g.ldb, g.sb,
                                       b, t.n0, g.N, K);
  mainloop<T, S, true, is_kmajor(kLA), is_kmajor(kLB), kGemmEvery>(acc, la, lb, (K + TB - 1) / TB, smem, p,
                                                       [](int64_t) {});
}

template <typename T, int kLA, int kLB>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_kernel(
    GemmArgs g) {
  using S = GTile;
  static_assert(S::kLdsBytes >= S::BM * kEpiStride * 4, "epilogue stage fits the pipeline's LDS");
  __shared__ __attribute__((aligned(16))) char smem_raw[S::kLdsBytes];
  lds_char* smem = (lds_char*)smem_raw;
  const GemmTilePos t = gemm_tile_pos<S>(g);
  Accum<S> acc;
  const LanePos p = lane_pos<S>();
  gemm_accumulate<T, kLA, kLB, -1, -1>(g, g, t, acc, smem, p);
  if (g.c_f32)
    gemm_epilogue<S, float>(acc, p, smem, static_cast<float*>(g.C) + t.b * g.sc, g.ldc, t.m0, t.n0,
                            g.M, g.N, g.alpha, g.accumulate != 0);
  else
    gemm_epilogue<S, T>(acc, p, smem, static_cast<T*>(g.C) + t.b * g.sc, g.ldc, t.m0, t.n0, g.M,
                        g.N, g.alpha, false);
}

// dZ = dO_j W^(j-1) + eta V^_j S_j in the accumulators (g: dO_j and the
// transposed weight slot, both K-contiguous; g2: V^_j and S_j read as k-major
// tiles), then the SwiGLU derivative per element: dZ never leaves the tile.
// Epilogue per pass of kPass columns: dZ staged in fp32; each thread takes
// two token rows x 8 columns, reads A_g and A_u (fp32) for them, writes the
// row-major dA runs and puts the values into two token-major stages (dA_g,
// dA_u), which then leave as k-blocked block rows.  The derivative is the
// plain formula in fp32 (sigmoid as 1 / (1 + exp(-A_g))).
template <typename T>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void dz_swiglu_kernel(
    GemmArgs g, GemmArgs g2, Dims dm, int64_t row0, int64_t row_stride,
    const float* __restrict__ Ag, T* __restrict__ dA, T* __restrict__ dAk) {
  using S = GTile;
  constexpr int kPass = sizeof(T) == 2 ? 64 : 32;  // columns per epilogue pass
  constexpr int kStride = kPass + 8;               // floats per staged dZ row
  using St = Stage<T, S::kThreads, kPass>;
  constexpr int kDzBytes = S::BM * kStride * 4;
  constexpr int kEpiBytes = kDzBytes + 2 * St::kBytes;
  constexpr int kLds = S::kLdsBytes > kEpiBytes ? S::kLdsBytes : kEpiBytes;
  static_assert(St::kToks == S::BM && S::BN % kPass == 0 && kPass % 32 == 0,
                "passes cover whole 32-column blocks of the tile's rows");
  __shared__ __attribute__((aligned(16))) char smem_raw[kLds];
  lds_char* smem = (lds_char*)smem_raw;
  const GemmTilePos t = gemm_tile_pos<S>(g);
  Accum<S> acc;
  const LanePos p = lane_pos<S>();
  gemm_accumulate<T, kRowK, kRowK, kRowK, kTiledKMajor>(g, g2, t, acc, smem, p);

  const int64_t f = dm.f, f2 = 2 * dm.f;
  const int64_t grow0 = row0 + t.b * row_stride + t.m0;  // token row of tile row 0
  const int rows_valid = (int)min<int64_t>(S::BM, g.M - t.m0);
  const ChunkMap cm = chunk_map(dm);
  lds_char* const dz = smem;
  lds_char* const stage_g = smem + kDzBytes;
  lds_char* const stage_u = stage_g + St::kBytes;
  constexpr int kGroups = kPass / 8;
  for (int q = 0; q < S::BN / kPass; ++q) {
    __syncthreads();  // the mainloop's (or the previous pass's) reads of LDS are done
#pragma unroll
    for (int j = 0; j < S::NB; ++j) {
      const int col = p.wave_n0 + 32 * j;
      if (col < kPass * q || col >= kPass * q + kPass) continue;
      const int c = col - kPass * q + (p.lane & 31);
#pragma unroll
      for (int i = 0; i < S::MB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          lds_store<float>(dz + ((uint32_t)p.row(i, r) * kStride + c) * 4, g.alpha * acc.v[i][j][r]);
    }
    __syncthreads();
    const int64_t cb = t.n0 + kPass * q;
    const int ncols = (int)max<int64_t>(0, min<int64_t>(kPass, g.N - cb));
    for (int it = threadIdx.x; it < (S::BM / 2) * kGroups; it += S::kThreads) {
      const int t0 = 2 * (it / kGroups), c = (it % kGroups) * 8;
      if (t0 >= rows_valid || c >= ncols) continue;
      float dag[2][8], dau[2][8];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int tr = t0 + h;
        if (tr >= rows_valid) {
#pragma unroll
          for (int e = 0; e < 8; ++e) dag[h][e] = dau[h][e] = 0.0f;
          continue;
        }
        const uint32_t srow = (uint32_t)tr * kStride + c;
        const floatx4_t z0 = lds_load<floatx4_t>(dz + srow * 4);
        const floatx4_t z1 = lds_load<floatx4_t>(dz + (srow + 4) * 4);
        const float* a = Ag + (grow0 + tr) * f2 + cb + c;
        const float4 g0 = *reinterpret_cast<const float4*>(a);
        const float4 g1 = *reinterpret_cast<const float4*>(a + 4);
        const float4 u0 = *reinterpret_cast<const float4*>(a + f);
        const float4 u1 = *reinterpret_cast<const float4*>(a + f + 4);
        const float zz[8] = {z0[0], z0[1], z0[2], z0[3], z1[0], z1[1], z1[2], z1[3]};
        const float gg[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
        const float uu[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float sg = 1.0f / (1.0f + __expf(-gg[e]));
          dag[h][e] = zz[e] * uu[e] * sg * (1.0f + gg[e] * (1.0f - sg));
          dau[h][e] = zz[e] * gg[e] * sg;
        }
        T* const out = dA + (grow0 + tr) * f2 + cb + c;
        store8<T>(out, dag[h], false);
        store8<T>(out + f, dau[h], false);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        St::put2(stage_g, c + e, t0, dag[0][e], dag[1][e]);
        St::put2(stage_u, c + e, t0, dau[0][e], dau[1][e]);
      }
    }
    __syncthreads();
    const int32_t r0 = (int32_t)grow0, r1 = (int32_t)(grow0 + rows_valid);
    St::flush_tokens(stage_g, dAk, f2, cb, ncols, r0, r1, cm);
    St::flush_tokens(stage_u, dAk, f2, f + cb, ncols, r0, r1, cm);
  }
}

// [A_g | A_u] = H [W_gate; W_up]ᵀ in fp32 and Z = SiLU(A_g) * A_u in one
// launch.  B is the interleaved weight WgU ([f/32][2][32][d]: 32 gate rows,
// then the 32 up rows of the same features; in TB x TB tiles when
// wgu_tiled(d, es)), so each 64-column pass of a tile holds the gate and up
// sums of 32 features.  Row t of Ag holds A_g at
// [0, f) and A_u at [f, 2f); Z is [BT][f] in the activation type, computed
// from the same fp32 values as SiLU(g) * u (the forward's arithmetic).
template <typename T>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void preact_kernel(
    const T* __restrict__ H, const T* __restrict__ WgU, int64_t BT, int64_t d, int64_t f,
    float* __restrict__ Ag, T* __restrict__ Z) {
  using S = GTile;
  __shared__ __attribute__((aligned(16))) char smem_raw[S::kLdsBytes];
  lds_char* smem = (lds_char*)smem_raw;
  constexpr int TB = kRowBytes / (int)sizeof(T);
  const int tiles_m = (int)((BT + S::BM - 1) / S::BM);
  const int tiles_n = (int)((2 * f + S::BN - 1) / S::BN);
  const TileCoord tc = grouped_tile(xcd_remap(blockIdx.x, (int)gridDim.x), tiles_m, tiles_n, 8);
  const int64_t m0 = (int64_t)tc.m * S::BM, n0 = (int64_t)tc.n * S::BN;
  Accum<S> acc;
  acc.zero();
  const LanePos p = lane_pos<S>();
  auto la = make_loader<T, kRowK, S::BM>(reinterpret_cast<const char*>(H), d, 0, 0, m0, BT, d);
  const char* const wgu = reinterpret_cast<const char*>(WgU);
  auto lb = wgu_tiled(d, (int64_t)sizeof(T)) ? make_loader<T, kTiledRowK, S::BN>(wgu, d, 0, 0, n0, 2 * f, d)
                                             : make_loader<T, kRowK, S::BN>(wgu, d, 0, 0, n0, 2 * f, d);
  mainloop<T, S>(acc, la, lb, (d + TB - 1) / TB, smem, p, [](int64_t) {});

  for (int q = 0; q < S::BN / kEpiCols; ++q) {
    __syncthreads();  // the mainloop's (or the previous pass's) reads of LDS are done
#pragma unroll
    for (int j = 0; j < S::NB; ++j) {
      const int col = p.wave_n0 + 32 * j;
      if (col < kEpiCols * q || col >= kEpiCols * q + kEpiCols) continue;
      const int c = col - kEpiCols * q + (p.lane & 31);
#pragma unroll
      for (int i = 0; i < S::MB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          lds_store<float>(smem + ((uint32_t)p.row(i, r) * kEpiStride + c) * 4, acc.v[i][j][r]);
    }
    __syncthreads();
    const int64_t pair = (n0 + kEpiCols * q) / 64;  // gate/up block pair: features 32 pair ..
    if (64 * pair >= 2 * f) continue;
    const int64_t feat = 32 * pair;
    for (int it = threadIdx.x; it < S::BM * 4; it += S::kThreads) {
      const int t = it / 4, c = (it % 4) * 8;
      if (m0 + t >= BT) continue;
      const uint32_t row = (uint32_t)t * kEpiStride;
      const floatx4_t g0 = lds_load<floatx4_t>(smem + (row + c) * 4);
      const floatx4_t g1 = lds_load<floatx4_t>(smem + (row + c + 4) * 4);
      const floatx4_t u0 = lds_load<floatx4_t>(smem + (row + 32 + c) * 4);
      const floatx4_t u1 = lds_load<floatx4_t>(smem + (row + 32 + c + 4) * 4);
      const float g[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
      const float u[8] = {u0[0], u0[1], u0[2], u0[3], u1[0], u1[1], u1[2], u1[3]};
      float* ag = Ag + (m0 + t) * 2 * f + feat + c;
      store8<float>(ag, g, false);
      store8<float>(ag + f, u, false);
      float z[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) z[e] = g[e] * __builtin_amdgcn_rcpf(1.0f + __expf(-g[e])) * u[e];
      store8<T>(Z + (m0 + t) * f + feat + c, z, false);
    }
  }
}

template <typename T>
hipError_t launch_gemm_t(const GemmArgs& g, hipStream_t s) {
  const int64_t tiles = ((g.M + 255) / 256) * ((g.N + 255) / 256) * g.batch;
  const dim3 grid((unsigned)tiles), block(512);
  const int32_t combo = g.a_layout * 8 + g.b_layout;
  switch (combo) {
    case kRowK * 8 + kRowK:
      hipLaunchKernelGGL((gemm_kernel<T, kRowK, kRowK>), grid, block, 0, s, g);
      break;
    case kRowK * 8 + kKMajor:
      hipLaunchKernelGGL((gemm_kernel<T, kRowK, kKMajor>), grid, block, 0, s, g);
      break;
    case kRowK * 8 + kTiledRowK:
      hipLaunchKernelGGL((gemm_kernel<T, kRowK, kTiledRowK>), grid, block, 0, s, g);
      break;
    case kRowK * 8 + kTiledKMajor:
      hipLaunchKernelGGL((gemm_kernel<T, kRowK, kTiledKMajor>), grid, block, 0, s, g);
      break;
    case kKMajor * 8 + kRowK:
      hipLaunchKernelGGL((gemm_kernel<T, kKMajor, kRowK>), grid, block, 0, s, g);
      break;
    case kKMajor * 8 + kKMajor:
      hipLaunchKernelGGL((gemm_kernel<T, kKMajor, kKMajor>), grid, block, 0, s, g);
      break;
    case kKBlocked * 8 + kKBlocked:
      hipLaunchKernelGGL((gemm_kernel<T, kKBlocked, kKBlocked>), grid, block, 0, s, g);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Layout and size rules of one product (see GemmLayout).
bool gemm_args_ok(const GemmArgs& g) {
  const int64_t tb = 128 / (int64_t)dtype_bytes(g.dt);
  // K-contiguous, k-blocked and tiled operands are read in whole k-tiles; the
  // N runs of the epilogue are 8 wide
  if ((g.a_layout != kKMajor || g.b_layout != kKMajor) && (g.K % tb != 0 || g.K_last % tb != 0))
    return false;
  if (g.N % 8 != 0 || g.K <= 0 || g.K_last <= 0) return false;
  // tiled operands (B only): whole TB x TB tiles
  if (g.a_layout == kTiledRowK || g.a_layout == kTiledKMajor) return false;
  if ((g.b_layout == kTiledRowK || g.b_layout == kTiledKMajor) &&
      (g.N % tb != 0 || g.ldb % tb != 0 || g.K_last != g.K))
    return false;
  return true;
}

// dst[j][col0 + i] = src[i][j], through a 64 x 64 LDS tile (padded against
// bank conflicts); 256 threads, 4 rows per pass.  dst has ld_dst columns,
// row-major, or (tb > 0) in tb x tb tiles: element (r, c) at
// ((r / tb) (ld_dst / tb) + c / tb) tb^2 + (r % tb) tb + c % tb.
template <typename T>
__global__ __launch_bounds__(256) void transpose_rect_kernel(T* __restrict__ dst,
                                                             const T* __restrict__ src,
                                                             int64_t rows, int64_t cols,
                                                             int64_t ld_dst, int64_t col0,
                                                             int32_t tb) {
  __shared__ T tile[64][65];
  const int64_t i0 = (int64_t)blockIdx.y * 64, j0 = (int64_t)blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int r = ty; r < 64; r += 4) {
    const int64_t i = i0 + r, j = j0 + tx;
    if (i < rows && j < cols) tile[r][tx] = src[i * cols + j];
  }
  __syncthreads();
  for (int r = ty; r < 64; r += 4) {
    const int64_t j = j0 + r, i = i0 + tx;
    if (i >= rows || j >= cols) continue;
    const int64_t c = col0 + i;
    const int64_t at = tb > 0 ? ((j / tb) * (ld_dst / tb) + c / tb) * tb * tb + (j % tb) * tb + c % tb
                              : j * ld_dst + c;
    dst[at] = tile[tx][r];
  }
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0 || g.batch <= 0) return hipSuccess;
  if (!gemm_args_ok(g)) return hipErrorInvalidValue;
  if (g.dt == Dtype::BF16) return launch_gemm_t<uint16_t>(g, s);
  return launch_gemm_t<float>(g, s);
}

hipError_t launch_dz_swiglu(const GemmArgs& g, const GemmArgs& g2, const Dims& dm, int64_t row0,
                            int64_t row_stride, const float* Ag, void* dA, void* dAk,
                            hipStream_t s) {
  if (g.M <= 0 || g.N <= 0 || g.batch <= 0) return hipSuccess;
  if (!gemm_args_ok(g) || !gemm_args_ok(g2) || g2.dt != g.dt || g.dt != dm.dt || g2.M != g.M ||
      g2.N != g.N || g2.batch != g.batch || g.N != dm.f || g.a_layout != kRowK ||
      g.b_layout != kRowK || g2.a_layout != kRowK || g2.b_layout != kTiledKMajor ||
      row0 < 0 || row0 + (g.batch - 1) * row_stride + g.M > dm.B * dm.T)
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)(((g.M + 255) / 256) * ((g.N + 255) / 256) * g.batch)), block(512);
  if (g.dt == Dtype::BF16)
    hipLaunchKernelGGL(dz_swiglu_kernel<uint16_t>, grid, block, 0, s, g, g2, dm, row0, row_stride,
                       Ag, static_cast<uint16_t*>(dA), static_cast<uint16_t*>(dAk));
  else
    hipLaunchKernelGGL(dz_swiglu_kernel<float>, grid, block, 0, s, g, g2, dm, row0, row_stride, Ag,
                       static_cast<float*>(dA), static_cast<float*>(dAk));
  return hipGetLastError();
}

hipError_t launch_preact_swiglu(Dtype dt, const void* H, const void* WgU, int64_t BT, int64_t d,
                                int64_t f, float* Ag, void* Z, hipStream_t s) {
  if (BT <= 0) return hipSuccess;
  if (d % 64 != 0 || f % 64 != 0) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(((BT + 255) / 256) * ((2 * f + 255) / 256)));
  if (dt == Dtype::BF16)
    hipLaunchKernelGGL(preact_kernel<uint16_t>, grid, dim3(512), 0, s,
                       static_cast<const uint16_t*>(H), static_cast<const uint16_t*>(WgU), BT, d,
                       f, Ag, static_cast<uint16_t*>(Z));
  else
    hipLaunchKernelGGL(preact_kernel<float>, grid, dim3(512), 0, s, static_cast<const float*>(H),
                       static_cast<const float*>(WgU), BT, d, f, Ag, static_cast<float*>(Z));
  return hipGetLastError();
}

hipError_t launch_transpose(const void* src, void* dst, int64_t rows, int64_t cols, Dtype dt,
                            hipStream_t s, int64_t ld_dst, int64_t col0, bool tiled) {
  if (ld_dst < 0) ld_dst = rows;
  const int32_t tb = tiled ? (int32_t)(kRowBytes / dtype_bytes(dt)) : 0;
  if (col0 < 0 || col0 + rows > ld_dst) return hipErrorInvalidValue;
  if (tiled && (ld_dst % tb != 0 || cols % tb != 0)) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((cols + 63) / 64), (unsigned)((rows + 63) / 64));
  if (dt == Dtype::BF16)
    hipLaunchKernelGGL(transpose_rect_kernel<uint16_t>, grid, dim3(256), 0, s,
                       static_cast<uint16_t*>(dst), static_cast<const uint16_t*>(src), rows, cols,
                       ld_dst, col0, tb);
  else
    hipLaunchKernelGGL(transpose_rect_kernel<float>, grid, dim3(256), 0, s,
                       static_cast<float*>(dst), static_cast<const float*>(src), rows, cols,
                       ld_dst, col0, tb);
  return hipGetLastError();
}

}  // namespace ttt
