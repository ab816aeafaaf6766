// kernels.hip -- HIP kernels of the In-Place TTT fast-weight MLP layer for
// CDNA4 (gfx950).
//
// The layer (In-Place TTT page, zhichai.net, sections 3.1-3.3): for chunk i of
// C tokens,
//   Z_i   = SiLU(H_i W_gate^T) (.) (H_i W_up^T)                      (S1, swiglu_kernel)
//   V^_i  = Conv1D(X0)_i W_target, Conv1D depthwise over X0[t+1-k]   (S2, target_kernel)
//   O_i   = Z_i (W^(i-1))^T                                          (S3, down_proj_kernel)
//   W^(i) = W^(i-1) + eta V^_i^T Z_i                                 (S4, prefix_update_kernel)
// S1 and S2 do not depend on the fast weight and run over all tokens at once.
// S4 walks the chunks of a group of G chunks in order, keeping the fp32
// fast-weight tile in the MFMA accumulators, and emits the weight each chunk
// must use (the exclusive prefix W^(0) + eta sum_{j<i} V^_j^T Z_j) into one
// slot per chunk; S3 then applies all slots of the group at once.  With G = 1
// this is the sequential scan (one fp32 read-modify-write of the state per
// chunk); with G = N it is the three-step chunk-parallel form (section 3.2)
// with the prefix streamed through the accumulators.
//
// Operand layouts the kernels agree on (row-major):
//   H, X0, O   [B*T][d]      activations (T = bf16 bits or fp32)
//   Z          [B*T][f]      gated activations
//   Zt         [f][P]        Z transposed, token columns chunk-padded
//   Vt         [d][P]        eta * V^ transposed, same columns
//   WtT        [d][d]        W_target transposed ([j_out][c_in])
//   tapsT      [8][d] fp32   taps transposed, zero for k >= K
//   W_state    [B][d][f]     fp32 fast weight
//   slots      [G][B][d][f]  weight used by each chunk of the group
// Token t of sequence b sits in column (b N + i) Cp + j of Zt/Vt, with
// i = t / C, j = t % C; columns j >= (chunk length) hold zeros.
#include <math.h>

#include <algorithm>

#include "gemm_core.h"
#include "layer.h"

namespace ttt {

using Tile = TileShape<256, 256>;

// ------------------------------------------------------------ chunk columns
struct ChunkMap {
  int32_t T, C, N, Cp;
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
  return m;
}

// LDS staging for the token-major outputs (Zt, Vt): a slice of 64 output
// columns x 256 tokens is gathered from the accumulators (each lane puts 4
// consecutive tokens of one column), then every thread copies 8-token runs to
// dst[col][column of token] with 16-byte stores where the 8 tokens lie in one
// chunk, element stores otherwise.  Row stride 260 tokens keeps the 4-token
// writes of 16 lanes on distinct banks.
template <typename T>
struct TokStage {
  static constexpr int kCols = 64;
  static constexpr int kToks = 256;
  static constexpr int kStride = (kToks + 4) * (int)sizeof(T);  // bytes per LDS row

  __device__ __forceinline__ static void put4(char* lds, int col, int tok, const float v[4]) {
    char* q = lds + col * kStride + tok * (int)sizeof(T);
    if constexpr (sizeof(T) == 2) {
      uint2 w;
      w.x = (uint32_t)f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16);
      w.y = (uint32_t)f32_to_bf16_bits(v[2]) | ((uint32_t)f32_to_bf16_bits(v[3]) << 16);
      *reinterpret_cast<uint2*>(q) = w;
    } else {
      *reinterpret_cast<float4*>(q) = make_float4(v[0], v[1], v[2], v[3]);
    }
  }

  // Copy columns [0, ncols) of the staged slice; token row0 + t of the tile
  // goes to dst[(col_base + c) * ld + column(row0 + t)].
  __device__ __forceinline__ static void flush(const char* lds, T* dst, int64_t ld,
                                               int64_t col_base, int ncols, int32_t row0,
                                               int32_t rows_total, const ChunkMap& cm) {
    for (int it = threadIdx.x; it < kCols * (kToks / 8); it += kThreads) {
      const int c = it >> 5, tok = (it & 31) * 8;
      const int32_t row = row0 + tok;
      if (c >= ncols || row >= rows_total) continue;
      const char* src = lds + c * kStride + tok * (int)sizeof(T);
      T* drow = dst + (col_base + c) * ld;
      const int32_t b = row / cm.T, sq = row - b * cm.T, i = sq / cm.C, j = sq - i * cm.C;
      const int64_t c0 = ((int64_t)b * cm.N + i) * cm.Cp + j;
      const int32_t room = min(cm.C - j, cm.T - sq);
      if (room >= 8 && (c0 & 7) == 0) {
        if constexpr (sizeof(T) == 2) {
          const uint2 lo = *reinterpret_cast<const uint2*>(src);
          const uint2 hi = *reinterpret_cast<const uint2*>(src + 8);
          *reinterpret_cast<uint4*>(drow + c0) = make_uint4(lo.x, lo.y, hi.x, hi.y);
        } else {
          *reinterpret_cast<uint4*>(drow + c0) = *reinterpret_cast<const uint4*>(src);
          *reinterpret_cast<uint4*>(drow + c0 + 4) = *reinterpret_cast<const uint4*>(src + 16);
        }
      } else {
        for (int e = 0; e < 8 && row + e < rows_total; ++e)
          drow[cm.col(row + e)] = reinterpret_cast<const T*>(src)[e];
      }
    }
  }

  // Copy the staged slice row-major: token row0 + t, column c goes to
  // dst[(row0 + t) * ld + col_base + c] for c < ncols (a multiple of 8),
  // 8 columns (16 bytes for bf16) per store.
  __device__ __forceinline__ static void flush_rows(const char* lds, T* dst, int64_t ld,
                                                    int64_t col_base, int ncols, int32_t row0,
                                                    int32_t rows_valid) {
    for (int it = threadIdx.x; it < kToks * (kCols / 8); it += kThreads) {
      const int t = it >> 3, c = (it & 7) * 8;
      if (t >= rows_valid || c >= ncols) continue;
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        v[e] = Elem<T>::to_f32(*reinterpret_cast<const T*>(lds + (c + e) * kStride + t * (int)sizeof(T)));
      T* d = dst + (int64_t)(row0 + t) * ld + col_base + c;
      if constexpr (sizeof(T) == 2) {
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          w[q] = (uint32_t)f32_to_bf16_bits(v[2 * q]) | ((uint32_t)f32_to_bf16_bits(v[2 * q + 1]) << 16);
        *reinterpret_cast<uint4*>(d) = make_uint4(w[0], w[1], w[2], w[3]);
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

// ===================================================================== S1
// Z = SiLU(H W_gate^T) (.) (H W_up^T) over all B*T token rows.  The B tile
// interleaves 32-row blocks of W_gate and W_up (block 2q: gate features
// f0+32q.., block 2q+1: the same up features), so each wave holds the gate and
// up sums of the same (token, feature) in the same lane and register.
template <typename T>
__global__ __launch_bounds__(kThreads) void swiglu_kernel(Dims dm, const T* __restrict__ H,
                                                          const T* __restrict__ Wg,
                                                          const T* __restrict__ Wu,
                                                          T* __restrict__ Z, T* __restrict__ Zt) {
  using S = Tile;
  __shared__ __attribute__((aligned(16))) char smem[S::kLdsBytes];
  const int32_t BT = (int32_t)(dm.B * dm.T);
  const int64_t d = dm.d, f = dm.f;
  constexpr int kFeat = S::BN / 2;
  const int tiles_m = (BT + S::BM - 1) / S::BM;
  const int tiles_n = (int)((f + kFeat - 1) / kFeat);
  const TileCoord tc =
      grouped_tile(xcd_remap(blockIdx.x, tiles_m * tiles_n), tiles_m, tiles_n, 8);
  const int32_t row0 = tc.m * S::BM;
  const int64_t feat0 = (int64_t)tc.n * kFeat;
  const int tr = threadIdx.x >> 3;

  RowLoader<S::BM> la;
  la.init([&](int q) -> const char* {
    const int32_t row = row0 + tr + 32 * q;
    return row < BT ? reinterpret_cast<const char*>(H + (int64_t)row * d) : nullptr;
  });
  RowLoader<S::BN> lb;
  lb.init([&](int q) -> const char* {
    const int64_t feat = feat0 + 32 * (q >> 1) + tr;
    if (feat >= f) return nullptr;
    return reinterpret_cast<const char*>(((q & 1) ? Wu : Wg) + feat * d);
  });

  Accum<S> acc;
  acc.zero();
  const LanePos p = lane_pos<S>();
  const int64_t nk = d * (int64_t)sizeof(T) / kRowBytes;
  mainloop<T, S>(acc, la, lb, nk, smem, p, [](int64_t) {});

  // Epilogue: z = silu(gate) * up, staged in LDS in two passes of 64
  // features (those of wave column 0, then of wave column 1), then copied to
  // Zt (token-major) and Z (row-major).
  const ChunkMap cm = chunk_map(dm);
  const int wn = (threadIdx.x >> 6) & 1;
  using Stage = TokStage<T>;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if (wn == h) {
#pragma unroll
      for (int jp = 0; jp < S::NB / 2; ++jp)
#pragma unroll
        for (int i = 0; i < S::MB; ++i)
#pragma unroll
          for (int rq = 0; rq < 4; ++rq) {
            float z[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
              z[e] = silu(acc.v[i][2 * jp][4 * rq + e]) * acc.v[i][2 * jp + 1][4 * rq + e];
            Stage::put4(smem, 32 * jp + (p.lane & 31), p.row(i, 4 * rq), z);
          }
    }
    __syncthreads();
    const int64_t cb = feat0 + 64 * h;
    const int ncols = (int)max<int64_t>(0, min<int64_t>(64, f - cb));
    Stage::flush(smem, Zt, dm.P, cb, ncols, row0, BT, cm);
    Stage::flush_rows(smem, Z, f, cb, ncols, row0, min(BT - row0, S::BM));
    __syncthreads();
  }
}

// ===================================================================== S2
// A operand of the target GEMM: U[t][c] = sum_k taps[c][k] X0[t+1-k][c]
// (zero outside the token's own sequence), computed in fp32 while staging
// the k-tile and rounded once to T.  Thread t owns the 16-byte channel chunk
// (t & 7) of the 8 consecutive rows 8 (t >> 3) .. +7 and keeps the window of
// X0 rows r0-(KMAX-2) .. r0+8 in registers.  Taps come from the fp32 [8][d]
// copy (zero for k >= K).
template <typename T, int KMAX>
struct ConvLoader {
  static constexpr int kWin = 7 + KMAX;
  static constexpr int EPC = Elem<T>::kPerChunk;
  const char* x0;      // X0 base + this thread's chunk offset
  const float* taps;   // tapsT base
  int64_t row_bytes;   // d * sizeof(T)
  int64_t d;
  int32_t r0, BT, T_seq;
  uint4 win[kWin];

  __device__ __forceinline__ void load(int64_t kt) {
#pragma unroll
    for (int w = 0; w < kWin; ++w) {
      const int32_t g = r0 - (KMAX - 2) + w;
      if (g >= 0 && g < BT)
        win[w] = *reinterpret_cast<const uint4*>(x0 + (int64_t)g * row_bytes + kt * kRowBytes);
      else
        win[w] = make_uint4(0u, 0u, 0u, 0u);
    }
  }
  __device__ __forceinline__ void store_kt(char* lds, int64_t kt) const {
    const int c = threadIdx.x & 7;
    const int64_t ch0 = kt * (kRowBytes / (int)sizeof(T)) + c * EPC;
    float tp[KMAX][EPC];
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
#pragma unroll
      for (int e = 0; e < EPC; e += 4) {
        const float4 t4 = *reinterpret_cast<const float4*>(taps + k * d + ch0 + e);
        tp[k][e] = t4.x;
        tp[k][e + 1] = t4.y;
        tp[k][e + 2] = t4.z;
        tp[k][e + 3] = t4.w;
      }
    const int lrow0 = (threadIdx.x >> 3) * 8;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int32_t o = r0 + jj;
      const int32_t s = o - (o / T_seq) * T_seq;  // position inside its sequence
      float u[EPC];
#pragma unroll
      for (int e = 0; e < EPC; ++e) u[e] = 0.0f;
      if (o < BT) {
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
          const int32_t src = s + 1 - k;  // X0 row of this tap, inside the sequence
          if (src < 0 || src >= T_seq) continue;
#pragma unroll
          for (int e = 0; e < EPC; ++e)
            u[e] = fmaf(tp[k][e], chunk_value<T>(win[jj + KMAX - 1 - k], e), u[e]);
        }
      }
      uint4 out;
      if constexpr (sizeof(T) == 2) {
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          w[q] = (uint32_t)f32_to_bf16_bits(u[2 * q]) |
                 ((uint32_t)f32_to_bf16_bits(u[2 * q + 1]) << 16);
        out = make_uint4(w[0], w[1], w[2], w[3]);
      } else {
        out = make_uint4(__float_as_uint(u[0]), __float_as_uint(u[1]), __float_as_uint(u[2]),
                         __float_as_uint(u[3]));
      }
      *reinterpret_cast<uint4*>(lds + lds_offset(lrow0 + jj, c)) = out;
    }
  }
};

// Adapts ConvLoader to the mainloop's load/store interface (the store needs
// the k-tile index for the taps).
template <typename T, int KMAX>
struct ConvLoaderRef {
  ConvLoader<T, KMAX>& l;
  int64_t pending;
  __device__ __forceinline__ void load(int64_t kt) {
    l.load(kt);
    pending = kt;
  }
  __device__ __forceinline__ void store(char* lds) const { l.store_kt(lds, pending); }
};

// eta * V^ = eta * U W_target over all token rows, written transposed into Vt.
template <typename T, int KMAX>
__global__ __launch_bounds__(kThreads) void target_kernel(Dims dm, const T* __restrict__ X0,
                                                          const float* __restrict__ tapsT,
                                                          const T* __restrict__ WtT,
                                                          T* __restrict__ Vt) {
  using S = Tile;
  __shared__ __attribute__((aligned(16))) char smem[S::kLdsBytes];
  const int32_t BT = (int32_t)(dm.B * dm.T);
  const int64_t d = dm.d;
  const int tiles_m = (BT + S::BM - 1) / S::BM;
  const int tiles_n = (int)((d + S::BN - 1) / S::BN);
  const TileCoord tc =
      grouped_tile(xcd_remap(blockIdx.x, tiles_m * tiles_n), tiles_m, tiles_n, 8);
  const int32_t row0 = tc.m * S::BM;
  const int64_t col0 = (int64_t)tc.n * S::BN;
  const int tr = threadIdx.x >> 3;

  ConvLoader<T, KMAX> conv;
  conv.x0 = reinterpret_cast<const char*>(X0) + (threadIdx.x & 7) * 16;
  conv.taps = tapsT;
  conv.row_bytes = d * (int64_t)sizeof(T);
  conv.d = d;
  conv.r0 = row0 + tr * 8;
  conv.BT = BT;
  conv.T_seq = (int32_t)dm.T;
  ConvLoaderRef<T, KMAX> la{conv, 0};
  RowLoader<S::BN> lb;
  lb.init([&](int q) -> const char* {
    const int64_t j = col0 + tr + 32 * q;
    return j < d ? reinterpret_cast<const char*>(WtT + j * d) : nullptr;
  });

  Accum<S> acc;
  acc.zero();
  const LanePos p = lane_pos<S>();
  const int64_t nk = d * (int64_t)sizeof(T) / kRowBytes;
  mainloop<T, S>(acc, la, lb, nk, smem, p, [](int64_t) {});

  // Epilogue: eta * V^ goes to Vt through LDS in four passes of 64 columns
  // (pass q: wave column q/2, its block columns 2(q%2) and 2(q%2)+1).
  const ChunkMap cm = chunk_map(dm);
  const float eta = dm.eta;
  const int wn = (threadIdx.x >> 6) & 1;
  using Stage = TokStage<T>;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (wn == (q >> 1)) {
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int j = 2 * (q & 1) + jj;
#pragma unroll
        for (int i = 0; i < S::MB; ++i)
#pragma unroll
          for (int rq = 0; rq < 4; ++rq) {
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = eta * acc.v[i][j][4 * rq + e];
            Stage::put4(smem, 32 * jj + (p.lane & 31), p.row(i, 4 * rq), v);
          }
      }
    }
    __syncthreads();
    const int64_t cb = col0 + 64 * q;
    Stage::flush(smem, Vt, dm.P, cb, (int)max<int64_t>(0, min<int64_t>(64, d - cb)), row0, BT, cm);
    __syncthreads();
  }
}

// ===================================================================== S4
// For each sequence b and fast-weight tile (m0.., n0..), over the chunks
// g0 .. g0+gc-1 in order:
//   slot[jj] <- W                        (the weight chunk g0+jj uses)
//   W        <- W + (eta V^_i)^T Z_i      (MFMA accumulation into the fp32 tile)
// and finally W_state <- W.  The accumulator is the fp32 state itself, so the
// result does not depend on how the chunks are grouped.
template <typename T>
__global__ __launch_bounds__(kThreads) void prefix_update_kernel(Dims dm, const T* __restrict__ Vt,
                                                                 const T* __restrict__ Zt,
                                                                 float* __restrict__ W_state,
                                                                 T* __restrict__ slots, int64_t g0,
                                                                 int64_t gc) {
  using S = Tile;
  __shared__ __attribute__((aligned(16))) char smem[S::kLdsBytes];
  const int64_t d = dm.d, f = dm.f;
  const int tiles_m = (int)((d + S::BM - 1) / S::BM);
  const int tiles_n = (int)((f + S::BN - 1) / S::BN);
  const int per_seq = tiles_m * tiles_n;
  // XCD-aware: consecutive logical tiles land on the same XCD.
  const int L = xcd_remap(blockIdx.x, per_seq * (int)dm.B);
  const int64_t b = L / per_seq;
  const TileCoord tc = grouped_tile(L - (int)b * per_seq, tiles_m, tiles_n, 4);
  const int64_t m0 = (int64_t)tc.m * S::BM, n0 = (int64_t)tc.n * S::BN;
  const int tr = threadIdx.x >> 3;
  const int64_t col_start = (b * dm.N + g0) * dm.Cp;

  RowLoader<S::BM> la;
  la.init([&](int q) -> const char* {
    const int64_t m = m0 + tr + 32 * q;
    return m < d ? reinterpret_cast<const char*>(Vt + m * dm.P + col_start) : nullptr;
  });
  RowLoader<S::BN> lb;
  lb.init([&](int q) -> const char* {
    const int64_t n = n0 + tr + 32 * q;
    return n < f ? reinterpret_cast<const char*>(Zt + n * dm.P + col_start) : nullptr;
  });

  const LanePos p = lane_pos<S>();
  // Lane base: row m0 + wave_m0 + 4 (lane / 32), column n0 + wave_n0 + lane % 32.
  // d and f are multiples of 32, so each 32x32 block is wholly inside or
  // wholly outside the weight.
  const int64_t lane_off = (m0 + p.wave_m0 + 4 * (p.lane >> 5)) * f + n0 + p.wave_n0 + (p.lane & 31);
  bool blk_ok[S::MB][S::NB];
#pragma unroll
  for (int i = 0; i < S::MB; ++i)
#pragma unroll
    for (int j = 0; j < S::NB; ++j)
      blk_ok[i][j] = (m0 + p.wave_m0 + 32 * i < d) && (n0 + p.wave_n0 + 32 * j < f);
  auto elem_off = [&](int i, int j, int r) -> int64_t {
    return (int64_t)(32 * i + 8 * (r >> 2) + (r & 3)) * f + 32 * j;
  };

  float* Wb = W_state + b * d * f + lane_off;
  Accum<S> acc;
#pragma unroll
  for (int i = 0; i < S::MB; ++i)
#pragma unroll
    for (int j = 0; j < S::NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc.v[i][j][r] = blk_ok[i][j] ? Wb[elem_off(i, j, r)] : 0.0f;

  const int64_t slot_stride = dm.B * d * f;
  T* slot_b = slots + b * d * f + lane_off;
  auto write_slot = [&](int64_t jj) {
    T* dst = slot_b + jj * slot_stride;
#pragma unroll
    for (int i = 0; i < S::MB; ++i)
#pragma unroll
      for (int j = 0; j < S::NB; ++j)
        if (blk_ok[i][j]) {
#pragma unroll
          for (int r = 0; r < 16; ++r) Elem<T>::store(dst + elem_off(i, j, r), acc.v[i][j][r]);
        }
  };

  write_slot(0);
  const int64_t kt_per_chunk = dm.Cp * (int64_t)sizeof(T) / kRowBytes;
  const int64_t nk = gc * kt_per_chunk;
  mainloop<T, S>(acc, la, lb, nk, smem, p, [&](int64_t kt) {
    const int64_t done = kt + 1;
    if (done % kt_per_chunk == 0 && done < nk) write_slot(done / kt_per_chunk);
  });

#pragma unroll
  for (int i = 0; i < S::MB; ++i)
#pragma unroll
    for (int j = 0; j < S::NB; ++j)
      if (blk_ok[i][j]) {
#pragma unroll
        for (int r = 0; r < 16; ++r) Wb[elem_off(i, j, r)] = acc.v[i][j][r];
      }
}

// ===================================================================== S3
// O_i = Z_i slot_i^T for every chunk of the group and every sequence.
template <typename T>
__global__ __launch_bounds__(kThreads) void down_proj_kernel(Dims dm, const T* __restrict__ Z,
                                                             const T* __restrict__ slots,
                                                             T* __restrict__ O, int64_t g0,
                                                             int64_t gc) {
  using S = Tile;
  __shared__ __attribute__((aligned(16))) char smem[S::kLdsBytes];
  const int64_t d = dm.d, f = dm.f, C = dm.C, T_seq = dm.T;
  const int tiles_m = (int)((C + S::BM - 1) / S::BM);
  const int tiles_n = (int)((d + S::BN - 1) / S::BN);
  const int per_chunk = tiles_m * tiles_n;
  const int L = xcd_remap(blockIdx.x, per_chunk * (int)(gc * dm.B));
  const int64_t cb = L / per_chunk;  // = b * gc + jj
  const int64_t b = cb / gc, jj = cb - b * gc;
  const int64_t chunk = g0 + jj;
  const TileCoord tc = grouped_tile(L - (int)cb * per_chunk, tiles_m, tiles_n, tiles_m);
  const int64_t c_begin = chunk * C;
  const int64_t c_len = min(C, T_seq - c_begin);
  const int64_t m0 = (int64_t)tc.m * S::BM, n0 = (int64_t)tc.n * S::BN;
  const int64_t tok0 = b * T_seq + c_begin;  // first token row of the chunk
  const int tr = threadIdx.x >> 3;
  const T* slot = slots + (jj * dm.B + b) * d * f;

  RowLoader<S::BM> la;
  la.init([&](int q) -> const char* {
    const int64_t r = m0 + tr + 32 * q;
    return r < c_len ? reinterpret_cast<const char*>(Z + (tok0 + r) * f) : nullptr;
  });
  RowLoader<S::BN> lb;
  lb.init([&](int q) -> const char* {
    const int64_t n = n0 + tr + 32 * q;
    return n < d ? reinterpret_cast<const char*>(slot + n * f) : nullptr;
  });

  Accum<S> acc;
  acc.zero();
  const LanePos p = lane_pos<S>();
  const int64_t nk = f * (int64_t)sizeof(T) / kRowBytes;
  mainloop<T, S>(acc, la, lb, nk, smem, p, [](int64_t) {});

  // Epilogue through LDS, four passes of 64 columns (pass q: wave column
  // q/2, block columns 2(q%2), 2(q%2)+1), written row-major; rows beyond the
  // chunk are skipped.
  const int wn = (threadIdx.x >> 6) & 1;
  using Stage = TokStage<T>;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (wn == (q >> 1)) {
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int i = 0; i < S::MB; ++i)
#pragma unroll
          for (int rq = 0; rq < 4; ++rq) {
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = acc.v[i][2 * (q & 1) + jj][4 * rq + e];
            Stage::put4(smem, 32 * jj + (p.lane & 31), p.row(i, 4 * rq), v);
          }
    }
    __syncthreads();
    const int64_t cb = n0 + 64 * q;
    const int ncols = (int)max<int64_t>(0, min<int64_t>(64, d - cb));
    Stage::flush_rows(smem, O + (tok0 + m0) * d, d, cb, ncols, 0,
                      (int32_t)min<int64_t>(S::BM, c_len - m0));
    __syncthreads();
  }
}

// ============================================================ small kernels
template <typename T>
__global__ void state_reset_kernel(float* __restrict__ W, const T* __restrict__ W0, int64_t B,
                                   int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += stride) {
    const float v = Elem<T>::to_f32(W0[e]);
    for (int64_t b = 0; b < B; ++b) W[b * n + e] = v;
  }
}

// dst[j][i] = src[i][j] for an n x n matrix, through a 64x64 LDS tile.
template <typename T>
__global__ void transpose_kernel(T* __restrict__ dst, const T* __restrict__ src, int64_t n) {
  __shared__ T tile[64][65];
  const int64_t i0 = (int64_t)blockIdx.y * 64, j0 = (int64_t)blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;  // 256 threads: 4 rows per pass
  for (int r = ty; r < 64; r += 4) {
    const int64_t i = i0 + r, j = j0 + tx;
    if (i < n && j < n) tile[r][tx] = src[i * n + j];
  }
  __syncthreads();
  for (int r = ty; r < 64; r += 4) {
    const int64_t j = j0 + r, i = i0 + tx;
    if (i < n && j < n) dst[j * n + i] = tile[tx][r];
  }
}

// tapsT[k][c] = taps[c][k] as fp32 for k < K, 0 for K <= k < 8.
template <typename T>
__global__ void taps_kernel(float* __restrict__ tapsT, const T* __restrict__ taps, int64_t d,
                            int32_t K) {
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= d) return;
  for (int k = 0; k < 8; ++k) tapsT[k * d + c] = k < K ? Elem<T>::to_f32(taps[c * K + k]) : 0.0f;
}

// Zero the padding columns (token index inside the chunk >= chunk length) of
// Zt ([f][P]) and Vt ([d][P]).
template <typename T>
__global__ void pad_fill_kernel(T* __restrict__ zt, T* __restrict__ vt, Dims dm) {
  const int64_t rows = dm.f + dm.d;
  const int64_t total = rows * dm.P;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += stride) {
    const int64_t row = e / dm.P, col = e - row * dm.P;
    const int64_t q = col / dm.Cp, j = col - q * dm.Cp;
    const int64_t i = q % dm.N;
    const int64_t len = min(dm.C, dm.T - i * dm.C);
    if (j < len) continue;
    T* dst = row < dm.f ? zt + row * dm.P + col : vt + (row - dm.f) * dm.P + col;
    Elem<T>::store(dst, 0.0f);
  }
}

// ================================================================ launchers
static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

WorkspacePlan plan_workspace(const Dims& dm, int64_t group) {
  const size_t es = dtype_bytes(dm.dt);
  WorkspacePlan w;
  size_t off = 0;
  w.z_off = off;
  off = align256(off + (size_t)(dm.B * dm.T) * dm.f * es);
  w.zt_off = off;
  off = align256(off + (size_t)dm.f * dm.P * es);
  w.vt_off = off;
  off = align256(off + (size_t)dm.d * dm.P * es);
  w.wtt_off = off;
  off = align256(off + (size_t)dm.d * dm.d * es);
  w.taps_off = off;
  off = align256(off + (size_t)8 * dm.d * sizeof(float));
  w.slots_off = off;
  w.fixed_bytes = off;
  w.slot_bytes = align256((size_t)dm.B * dm.d * dm.f * es);
  w.group = group;
  w.total_bytes = off + (size_t)group * w.slot_bytes;
  return w;
}

hipError_t launch_state_reset(float* W_state, const void* W0, Dtype w0_dt, int64_t B, int64_t d,
                              int64_t f, hipStream_t s) {
  const int64_t n = d * f;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 8192);
  if (w0_dt == Dtype::BF16)
    hipLaunchKernelGGL(state_reset_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, s,
                       W_state, static_cast<const uint16_t*>(W0), B, n);
  else
    hipLaunchKernelGGL(state_reset_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, s,
                       W_state, static_cast<const float*>(W0), B, n);
  return hipGetLastError();
}

hipError_t launch_transpose(void* dst, const void* src, int64_t n, Dtype dt, hipStream_t s) {
  const dim3 grid((unsigned)((n + 63) / 64), (unsigned)((n + 63) / 64));
  if (dt == Dtype::BF16)
    hipLaunchKernelGGL(transpose_kernel<uint16_t>, grid, dim3(256), 0, s,
                       static_cast<uint16_t*>(dst), static_cast<const uint16_t*>(src), n);
  else
    hipLaunchKernelGGL(transpose_kernel<float>, grid, dim3(256), 0, s, static_cast<float*>(dst),
                       static_cast<const float*>(src), n);
  return hipGetLastError();
}

hipError_t launch_taps(float* tapsT, const void* taps, const Dims& dm, hipStream_t s) {
  const unsigned blocks = (unsigned)((dm.d + 255) / 256);
  if (dm.dt == Dtype::BF16)
    hipLaunchKernelGGL(taps_kernel<uint16_t>, dim3(blocks), dim3(256), 0, s, tapsT,
                       static_cast<const uint16_t*>(taps), dm.d, dm.K);
  else
    hipLaunchKernelGGL(taps_kernel<float>, dim3(blocks), dim3(256), 0, s, tapsT,
                       static_cast<const float*>(taps), dm.d, dm.K);
  return hipGetLastError();
}

hipError_t launch_pad_fill(void* zt, void* vt, const Dims& dm, hipStream_t s) {
  const int64_t total = (dm.f + dm.d) * dm.P;
  const int64_t blocks = std::min<int64_t>((total + 255) / 256, 65536);
  if (dm.dt == Dtype::BF16)
    hipLaunchKernelGGL(pad_fill_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, s,
                       static_cast<uint16_t*>(zt), static_cast<uint16_t*>(vt), dm);
  else
    hipLaunchKernelGGL(pad_fill_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, s,
                       static_cast<float*>(zt), static_cast<float*>(vt), dm);
  return hipGetLastError();
}

hipError_t launch_swiglu(const Dims& dm, const void* H, const void* Wg, const void* Wu, void* Z,
                         void* Zt, hipStream_t s) {
  const int64_t BT = dm.B * dm.T;
  const int64_t tiles = ((BT + Tile::BM - 1) / Tile::BM) * ((dm.f + Tile::BN / 2 - 1) / (Tile::BN / 2));
  if (dm.dt == Dtype::BF16)
    hipLaunchKernelGGL(swiglu_kernel<uint16_t>, dim3((unsigned)tiles), dim3(kThreads), 0, s, dm,
                       static_cast<const uint16_t*>(H), static_cast<const uint16_t*>(Wg),
                       static_cast<const uint16_t*>(Wu), static_cast<uint16_t*>(Z),
                       static_cast<uint16_t*>(Zt));
  else
    hipLaunchKernelGGL(swiglu_kernel<float>, dim3((unsigned)tiles), dim3(kThreads), 0, s, dm,
                       static_cast<const float*>(H), static_cast<const float*>(Wg),
                       static_cast<const float*>(Wu), static_cast<float*>(Z),
                       static_cast<float*>(Zt));
  return hipGetLastError();
}

template <typename T>
static void launch_target_t(const Dims& dm, const T* X0, const float* tapsT, const T* WtT, T* Vt,
                            hipStream_t s) {
  const int64_t BT = dm.B * dm.T;
  const int64_t tiles = ((BT + Tile::BM - 1) / Tile::BM) * ((dm.d + Tile::BN - 1) / Tile::BN);
  if (dm.K <= 4)
    hipLaunchKernelGGL((target_kernel<T, 4>), dim3((unsigned)tiles), dim3(kThreads), 0, s, dm, X0,
                       tapsT, WtT, Vt);
  else
    hipLaunchKernelGGL((target_kernel<T, 8>), dim3((unsigned)tiles), dim3(kThreads), 0, s, dm, X0,
                       tapsT, WtT, Vt);
}

hipError_t launch_target(const Dims& dm, const void* X0, const void* tapsT, const void* WtT,
                         void* Vt, hipStream_t s) {
  if (dm.dt == Dtype::BF16)
    launch_target_t<uint16_t>(dm, static_cast<const uint16_t*>(X0),
                              static_cast<const float*>(tapsT),
                              static_cast<const uint16_t*>(WtT), static_cast<uint16_t*>(Vt), s);
  else
    launch_target_t<float>(dm, static_cast<const float*>(X0), static_cast<const float*>(tapsT),
                           static_cast<const float*>(WtT), static_cast<float*>(Vt), s);
  return hipGetLastError();
}

hipError_t launch_prefix_update(const Dims& dm, const void* Vt, const void* Zt, float* W_state,
                                void* slots, int64_t g0, int64_t gc, hipStream_t s) {
  const int64_t tiles =
      ((dm.d + Tile::BM - 1) / Tile::BM) * ((dm.f + Tile::BN - 1) / Tile::BN) * dm.B;
  if (dm.dt == Dtype::BF16)
    hipLaunchKernelGGL(prefix_update_kernel<uint16_t>, dim3((unsigned)tiles), dim3(kThreads), 0,
                       s, dm, static_cast<const uint16_t*>(Vt), static_cast<const uint16_t*>(Zt),
                       W_state, static_cast<uint16_t*>(slots), g0, gc);
  else
    hipLaunchKernelGGL(prefix_update_kernel<float>, dim3((unsigned)tiles), dim3(kThreads), 0, s,
                       dm, static_cast<const float*>(Vt), static_cast<const float*>(Zt), W_state,
                       static_cast<float*>(slots), g0, gc);
  return hipGetLastError();
}

hipError_t launch_down_proj(const Dims& dm, const void* Z, const void* slots, void* O, int64_t g0,
                            int64_t gc, hipStream_t s) {
  const int64_t tiles = ((dm.C + Tile::BM - 1) / Tile::BM) * ((dm.d + Tile::BN - 1) / Tile::BN) *
                        gc * dm.B;
  if (dm.dt == Dtype::BF16)
    hipLaunchKernelGGL(down_proj_kernel<uint16_t>, dim3((unsigned)tiles), dim3(kThreads), 0, s,
                       dm, static_cast<const uint16_t*>(Z), static_cast<const uint16_t*>(slots),
                       static_cast<uint16_t*>(O), g0, gc);
  else
    hipLaunchKernelGGL(down_proj_kernel<float>, dim3((unsigned)tiles), dim3(kThreads), 0, s, dm,
                       static_cast<const float*>(Z), static_cast<const float*>(slots),
                       static_cast<float*>(O), g0, gc);
  return hipGetLastError();
}

}  // namespace ttt
