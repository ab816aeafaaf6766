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
// Layouts the kernels agree on (es = element bytes, TB = 128 / es tokens):
//   H, X0, O   [B*T][d]            activations (T = bf16 bits or fp32)
//   Z          [B*T][f]            gated activations, row-major (S3's A operand)
//   Zt         [P/TB][f][TB]       Z token-major, k-blocked (S4's B operand)
//   Vt         [P/TB][d][TB]       eta * V^ token-major, k-blocked (S4's A operand)
//   WgU        [f/32][2][32][d]    W_gate / W_up rows interleaved in blocks of 32
//                                  (in TB x TB tiles when wgu_tiled(d, es))
//   WtT        [d][d]              W_target transposed ([j_out][c_in])
//   tapsT      [8][d] fp32         taps transposed, zero for k >= K
//   W_state    [B][d][f] fp32      fast weight
//   slots      [G][B][d/TB][f/TB][TB][TB]  weight used by each chunk of the group,
//                                  in TB x TB tiles (TB = 128 bytes of T)
// Token t of sequence b has token column p = (b N + i) Cp + j (i = t / C,
// j = t % C, Cp = C rounded up to 64); columns with j >= chunk length hold
// zeros.  In the k-blocked layouts one k-tile of a GEMM (TB tokens of R rows)
// is one contiguous R x 128-byte block.
#include <math.h>

#include <algorithm>

#include "epilogue.h"
#include "gemm_core.h"
#include "layer.h"

namespace ttt {

// Workgroup shape of the GEMM kernels: 256 x 256 output tile, WAVES_M x
// WAVES_N waves (wave tile 128 x 64 with 2 x 4 waves: two waves per SIMD, so
// one wave's MFMAs cover the other's LDS and barrier waits).
#ifndef TTT_WAVES_M
#define TTT_WAVES_M 2
#endif
#ifndef TTT_WAVES_N
#define TTT_WAVES_N 4
#endif
#define TTT_GEMM_THREADS (64 * TTT_WAVES_M * TTT_WAVES_N)
#define TTT_GEMM_WPE (TTT_WAVES_M * TTT_WAVES_N / 4)
using Tile = TileShape<256, 256, TTT_WAVES_M, TTT_WAVES_N>;
using PrefixTile = Tile;
// Output tiles: waves 4 x 2 (64 token rows x 128 columns each), so that each
// wave reads two transposed Z fragments per step (two 8-byte transposing LDS
// reads each) against four with the 2 x 4 arrangement: the transposing reads
// cost LDS instructions, the row-form weight fragments half as many.
using OutTile = TileShape<256, 256, 4, 2>;
static_assert(OutTile::kThreads == Tile::kThreads && OutTile::kLdsBytes == Tile::kLdsBytes,
              "output and scan tiles share a launch");
using OneChunkTile = TileShape<128, 128, 2, 2>;  // single-chunk updates
// The forward's weight slots are stored in TB x TB tiles (layout 4 of
// prefix_update_tile): an output tile reads each k-tile of its slot rows as
// four contiguous 8 KB tiles, and a scan tile writes its slot as 4 KB runs
// (against 128-byte row segments one slot row apart in the row-major layout,
// which measured 0.7-0.8% slower per step).
constexpr int kFwdSlots = 4;
// LDS for the staged slot rows: 4 KB per wave of the 256 x 256 scan tile.
constexpr int kSlotStageBytes = 8 * 4096;
// bf16 slots are staged through LDS (a quarter of the store instructions);
// fp32 slots keep the direct stores.
template <typename T>
bool staged_slots(const Dims&) {
  return sizeof(T) == 2;
}
#define TTT_GEMM_KERNEL                                  \
  __global__ __launch_bounds__(TTT_GEMM_THREADS)          \
  __attribute__((amdgpu_waves_per_eu(TTT_GEMM_WPE, TTT_GEMM_WPE)))

// Lanes hold 4 consecutive rows (e = 0..3) of one column; an even/odd lane
// pair (adjacent columns c, c+1) swaps two values (DPP) so that each lane
// holds two 32-bit bf16 pairs of adjacent columns: the even lane rows 0 and 1,
// the odd lane rows 2 and 3.  w[r] is row (odd ? 2 : 0) + r, columns
// (c & ~1, (c & ~1) + 1).
__device__ __forceinline__ void pair_pack(const float z[4], bool odd, uint32_t w[2]) {
  const float s0 = odd ? z[0] : z[2], s1 = odd ? z[1] : z[3];
  const float r0 = __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, s0), 0xB1, 0xF, 0xF, false));
  const float r1 = __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, s1), 0xB1, 0xF, 0xF, false));
  w[0] = odd ? pack_bf16x2(r0, z[2]) : pack_bf16x2(z[0], r0);
  w[1] = odd ? pack_bf16x2(r1, z[3]) : pack_bf16x2(z[1], r1);
}

// Put tile columns [W q, W q + W) into the stage (values transformed by
// `fn`); only the waves owning those columns write.
template <typename T, class S, int W = 64, class F>
__device__ __forceinline__ void stage_cols(lds_char* lds, const Accum<S>& acc, const LanePos& p,
                                           int q, F&& fn) {
  static_assert(W % 32 == 0, "whole 32-column blocks per pass");
#pragma unroll
  for (int j = 0; j < S::NB; ++j) {
    const int col = p.wave_n0 + 32 * j;  // first tile column of block j
    if (col < W * q || col >= W * q + W) continue;
#pragma unroll
    for (int i = 0; i < S::MB; ++i)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = fn(acc.v[i][j][4 * rq + e]);
        Stage<T, S::kThreads, W>::put4(lds, col - W * q + (p.lane & 31), p.row(i, 4 * rq), v);
      }
  }
}

// ===================================================================== S1
// Z = SiLU(H W_gate^T) (.) (H W_up^T) over all B*T token rows.  The B operand
// is WgU, whose 32-row blocks alternate gate and up rows of the same 32
// features, so each wave holds the gate and up sums of the same (token,
// feature) in the same lane and register (block columns 2q and 2q+1).
// Output: Zt (token-major, k-blocked), which both the scan and (bf16, with
// transposed reads) the outputs read; fp32 also writes the row-major Z its
// outputs read.
template <typename T>
TTT_GEMM_KERNEL void swiglu_kernel(Dims dm, const T* __restrict__ H, const T* __restrict__ WgU,
                                   T* __restrict__ Z, T* __restrict__ Zt) {
  using S = Tile;
  static_assert(S::NB % 2 == 0, "gate/up block pairs");
  constexpr int kLds = S::kLdsBytes;
  __shared__ __attribute__((aligned(16))) char smem_raw[kLds];
  lds_char* smem = (lds_char*)smem_raw;
  const int32_t BT = (int32_t)(dm.B * dm.T);
  const int64_t d = dm.d, f = dm.f;
  const int64_t ld = d * (int64_t)sizeof(T);
  constexpr int kFeat = S::BN / 2;
  const int tiles_m = (BT + S::BM - 1) / S::BM;
  const int tiles_n = (int)((f + kFeat - 1) / kFeat);
  const TileCoord tc =
      grouped_tile(xcd_remap(blockIdx.x, tiles_m * tiles_n), tiles_m, tiles_n, 8);
  const int32_t row0 = tc.m * S::BM;
  const int64_t feat0 = (int64_t)tc.n * kFeat;

  DirectLoader<S::BM, S::kWaves> la;
  la.init(reinterpret_cast<const char*>(H) + row0 * ld, ld, kRowBytes, (BT - row0) * ld,
          kRowBytes);
  DirectLoader<S::BN, S::kWaves> lb;
  if (wgu_tiled(d, (int64_t)sizeof(T))) {
    constexpr int TB = kRowBytes / (int)sizeof(T);
    lb.init_blocked(reinterpret_cast<const char*>(WgU) + (2 * feat0 / TB) * d * kRowBytes, TB,
                    d * kRowBytes, TB * kRowBytes, ((2 * f - 2 * feat0) / TB) * d * kRowBytes,
                    TB * kRowBytes);
  } else {
    lb.init(reinterpret_cast<const char*>(WgU) + 2 * feat0 * ld, ld, kRowBytes,
            (2 * f - 2 * feat0) * ld, kRowBytes);
  }

  Accum<S> acc;
  acc.zero();
  const LanePos p = lane_pos<S>();
  mainloop<T, S>(acc, la, lb, ld / kRowBytes, smem, p, [](int64_t) {});

  // z = silu(gate) * up, staged through LDS and written to Zt (and for fp32
  // to Z).  bf16: all 128 features in one pass; fp32: two passes of 64
  // features through the token-run stage, read back as column runs for Z.
  const ChunkMap cm = chunk_map(dm);
  constexpr int kPass = sizeof(T) == 2 ? kFeat : 64;  // features per pass
  using St = Stage<T, S::kThreads, kPass>;
  static_assert(St::kBytes <= kLds, "staging fits the kernel's LDS");
#pragma unroll
  for (int h = 0; h < kFeat / kPass; ++h) {
#pragma unroll
    for (int jp = 0; jp < S::NB / 2; ++jp) {
      const int brow = p.wave_n0 + 64 * jp;  // B-tile row of the gate block of this pair
      if (brow < 2 * kPass * h || brow >= 2 * kPass * (h + 1)) continue;
      const int fcol = brow / 2 - kPass * h;   // feature column inside the pass
#pragma unroll
      for (int i = 0; i < S::MB; ++i)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          float z[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            z[e] = silu(acc.v[i][2 * jp][4 * rq + e]) * acc.v[i][2 * jp + 1][4 * rq + e];
          St::put4(smem, fcol + (p.lane & 31), p.row(i, 4 * rq), z);
        }
    }
    __syncthreads();
    const int64_t cb = feat0 + kPass * h;
    const int ncols = (int)max<int64_t>(0, min<int64_t>(kPass, f - cb));
    St::flush_tokens(smem, Zt, f, cb, ncols, row0, BT, cm);
    if constexpr (sizeof(T) == 4) St::flush_rows(smem, Z, row0, f, cb, ncols, 0, min(BT - row0, S::BM));
    if (h + 1 < kFeat / kPass) __syncthreads();
  }
}

// ===================================================================== S2
// U[t][c] = sum_{k<K} taps[c][k] X0[t+1-k][c] (zero outside the token's own
// sequence), accumulated in fp32 over k = 0..K-1 and rounded once to T.
// Thread work item: one 16-byte channel chunk of kConvRows consecutive token
// rows, with the X0 window of those rows (kConvRows + KMAX - 1 rows) in
// registers; consecutive threads take consecutive chunks of a row group, so
// every access is a coalesced 16-byte load or store.
constexpr int kConvRows = 8;
template <typename T, int KMAX>
__global__ __launch_bounds__(256) void conv_kernel(Dims dm, const T* __restrict__ X0,
                                                   const float* __restrict__ tapsT,
                                                   T* __restrict__ U) {
  constexpr int EPC = Elem<T>::kPerChunk;
  constexpr int kWin = kConvRows + KMAX - 1;
  const int64_t d = dm.d, BT = dm.B * dm.T, T_seq = dm.T;
  const int K = dm.K;
  const int64_t chunks = d / EPC;
  const int64_t total = (BT + kConvRows - 1) / kConvRows * chunks;
  for (int64_t it = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; it < total;
       it += (int64_t)gridDim.x * blockDim.x) {
    const int64_t c = it % chunks, r0 = it / chunks * kConvRows;
    float tp[KMAX][EPC];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
      const float4* src = reinterpret_cast<const float4*>(tapsT + k * d + c * EPC);
#pragma unroll
      for (int v = 0; v < EPC / 4; ++v) {
        const float4 t = src[v];
        tp[k][4 * v] = t.x;
        tp[k][4 * v + 1] = t.y;
        tp[k][4 * v + 2] = t.z;
        tp[k][4 * v + 3] = t.w;
      }
    }
    uint4 win[kWin];  // X0 rows r0 + shift - (KMAX - 1) + w
#pragma unroll
    for (int w = 0; w < kWin; ++w) {
      const int64_t row = r0 + dm.shift - (KMAX - 1) + w;
      win[w] = row >= 0 && row < BT
                   ? *reinterpret_cast<const uint4*>(X0 + row * d + c * EPC)
                   : make_uint4(0, 0, 0, 0);
    }
    // Interior items: all kConvRows rows in one sequence and every tap's row
    // inside it -- the same sums in the same order without the per-row and
    // per-tap position checks.
    const int64_t sq0 = r0 % T_seq;
    if (r0 + kConvRows <= BT && sq0 + dm.shift >= K - 1 && sq0 + kConvRows + dm.shift <= T_seq) {
#pragma unroll
      for (int jj = 0; jj < kConvRows; ++jj) {
        float u[EPC];
#pragma unroll
        for (int e = 0; e < EPC; ++e) u[e] = 0.0f;
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
          if (k >= K) break;
#pragma unroll
          for (int e = 0; e < EPC; ++e)
            u[e] = fmaf(tp[k][e], chunk_value<T>(win[jj + KMAX - 1 - k], e), u[e]);
        }
        uint4 out;
        if constexpr (sizeof(T) == 2)
          out = make_uint4(pack_bf16x2(u[0], u[1]), pack_bf16x2(u[2], u[3]),
                           pack_bf16x2(u[4], u[5]), pack_bf16x2(u[6], u[7]));
        else
          out = make_uint4(__float_as_uint(u[0]), __float_as_uint(u[1]), __float_as_uint(u[2]),
                           __float_as_uint(u[3]));
        *reinterpret_cast<uint4*>(U + (r0 + jj) * d + c * EPC) = out;
      }
      continue;
    }
#pragma unroll
    for (int jj = 0; jj < kConvRows; ++jj) {
      const int64_t o = r0 + jj;
      if (o >= BT) break;
      const int64_t sq = o % T_seq;  // position inside its sequence
      float u[EPC];
#pragma unroll
      for (int e = 0; e < EPC; ++e) u[e] = 0.0f;
#pragma unroll
      for (int k = 0; k < KMAX; ++k) {
        const int64_t src = sq + dm.shift - k;  // X0 row of tap k, inside the sequence
        if (k >= K) continue;
        if (src >= T_seq) {  // after the sequence: zero, or the share's right halo row
          if (dm.halo_r == nullptr || src > T_seq) continue;
          const uint4 hv = *reinterpret_cast<const uint4*>(
              static_cast<const T*>(dm.halo_r) + (o / T_seq) * dm.halo_r_stride + c * EPC);
#pragma unroll
          for (int e = 0; e < EPC; ++e) u[e] = fmaf(tp[k][e], chunk_value<T>(hv, e), u[e]);
          continue;
        }
        if (src < 0) {  // before the sequence: zero, or the streaming halo
          if (dm.halo == nullptr || src < -kHaloRows) continue;
          const uint4 hv = *reinterpret_cast<const uint4*>(
              static_cast<const T*>(dm.halo) + (o / T_seq) * dm.halo_stride +
              (kHaloRows + src) * d + c * EPC);
#pragma unroll
          for (int e = 0; e < EPC; ++e) u[e] = fmaf(tp[k][e], chunk_value<T>(hv, e), u[e]);
          continue;
        }
#pragma unroll
        for (int e = 0; e < EPC; ++e)
          u[e] = fmaf(tp[k][e], chunk_value<T>(win[jj + KMAX - 1 - k], e), u[e]);
      }
      uint4 out;
      if constexpr (sizeof(T) == 2)
        out = make_uint4(pack_bf16x2(u[0], u[1]), pack_bf16x2(u[2], u[3]), pack_bf16x2(u[4], u[5]),
                         pack_bf16x2(u[6], u[7]));
      else
        out = make_uint4(__float_as_uint(u[0]), __float_as_uint(u[1]), __float_as_uint(u[2]),
                         __float_as_uint(u[3]));
      *reinterpret_cast<uint4*>(U + o * d + c * EPC) = out;
    }
  }
}

// eta * V^ = eta * U W_target over all token rows, written token-major to Vt.
// LDS of the projection tile: the pipeline's stages, or the epilogue stage
// (all 256 columns at once for bf16, 128 for fp32), whichever is larger.
template <typename T>
struct TargetLds {
  static constexpr int kPass = sizeof(T) == 2 ? Tile::BN : Tile::BN / 2;
  using St = Stage<T, Tile::kThreads, kPass>;
  static constexpr int kBytes = St::kBytes > Tile::kLdsBytes ? St::kBytes : Tile::kLdsBytes;
};

// Tile `blk` of `nblk` of the projection of token rows [t_lo, t_hi) of every
// sequence (tiles do not straddle sequences): eta V^ into Vt and, with kV,
// V^ itself (unscaled, row-major [B*T][d]) into V.
template <typename T, bool kV = false>
__device__ __forceinline__ void target_tile(const Dims& dm, const T* __restrict__ U,
                                            const T* __restrict__ WtT, T* __restrict__ Vt,
                                            int64_t t_lo, int64_t t_hi, int blk, int nblk,
                                            lds_char* smem, T* __restrict__ V = nullptr) {
  using S = Tile;
  constexpr int kPass = TargetLds<T>::kPass;
  using St = typename TargetLds<T>::St;
  const int64_t d = dm.d;
  const int64_t ld = d * (int64_t)sizeof(T);
  const int tiles_seq = (int)((t_hi - t_lo + S::BM - 1) / S::BM);
  const int tiles_m = tiles_seq * (int)dm.B;
  const int tiles_n = (int)((d + S::BN - 1) / S::BN);
  const TileCoord tc = grouped_tile(xcd_remap(blk, nblk), tiles_m, tiles_n, 8);
  const int64_t b = tc.m / tiles_seq;
  const int32_t row0 = (int32_t)(b * dm.T + t_lo + (int64_t)(tc.m - b * tiles_seq) * S::BM);
  const int32_t row_end = (int32_t)(b * dm.T + t_hi);  // rows of this sequence end here
  const int64_t col0 = (int64_t)tc.n * S::BN;

  DirectLoader<S::BM, S::kWaves> la;
  la.init(reinterpret_cast<const char*>(U) + (int64_t)row0 * ld, ld, kRowBytes,
          (int64_t)(row_end - row0) * ld, kRowBytes);
  DirectLoader<S::BN, S::kWaves> lb;
  lb.init(reinterpret_cast<const char*>(WtT) + col0 * ld, ld, kRowBytes, (d - col0) * ld,
          kRowBytes);

  Accum<S> acc;
  acc.zero();
  const LanePos p = lane_pos<S>();
  mainloop<T, S>(acc, la, lb, ld / kRowBytes, smem, p, [](int64_t) {});

  // eta * acc to Vt through the stage, kPass columns per pass.
  const ChunkMap cm = chunk_map(dm);
  const float eta = dm.eta;
#pragma unroll
  for (int q = 0; q < S::BN / kPass; ++q) {
    if (q > 0) __syncthreads();  // the previous pass's flush has read the stage
    stage_cols<T, S, kPass>(smem, acc, p, q, [&](float x) { return eta * x; });
    __syncthreads();
    const int64_t cb = col0 + kPass * q;
    const int ncols = (int)max<int64_t>(0, min<int64_t>(kPass, d - cb));
    St::flush_tokens(smem, Vt, d, cb, ncols, row0, row_end, cm);
    if constexpr (kV) {
      __syncthreads();
      stage_cols<T, S, kPass>(smem, acc, p, q, [](float x) { return x; });
      __syncthreads();
      St::flush_rows(smem, V, row0, d, cb, ncols, 0, min(S::BM, row_end - row0));
    }
  }
}

template <typename T, bool kV = false>
TTT_GEMM_KERNEL void target_kernel(Dims dm, const T* __restrict__ U, const T* __restrict__ WtT,
                                   T* __restrict__ Vt, int64_t t_lo, int64_t t_hi,
                                   T* __restrict__ V) {
  __shared__ __attribute__((aligned(16))) char smem_raw[TargetLds<T>::kBytes];
  target_tile<T, kV>(dm, U, WtT, Vt, t_lo, t_hi, blockIdx.x, gridDim.x, (lds_char*)smem_raw, V);
}

// eta * R (R [B*T][d] row-major: X0 or U) into Vt, for the targets without a
// projection.  A workgroup stages 256 token rows x 64 channels through LDS and
// leaves through the token-major flush.
template <typename T>
__global__ __launch_bounds__(256) void rows_to_vt_kernel(Dims dm, const T* __restrict__ R,
                                                         T* __restrict__ Vt) {
  using St = Stage<T, 256, 64>;
  __shared__ __attribute__((aligned(16))) char smem_raw[St::kBytes];
  lds_char* smem = (lds_char*)smem_raw;
  constexpr int EPC = Elem<T>::kPerChunk;
  const int32_t BT = (int32_t)(dm.B * dm.T);
  const int32_t row0 = (int32_t)blockIdx.x * St::kToks;
  const int64_t c0 = (int64_t)blockIdx.y * St::kCols;
  const int ncols = (int)min<int64_t>(St::kCols, dm.d - c0);
  for (int it = threadIdx.x; it < St::kToks * (St::kCols / EPC); it += 256) {
    const int t = it / (St::kCols / EPC), c = (it % (St::kCols / EPC)) * EPC;
    if (row0 + t >= BT || c >= ncols) continue;
    const uint4 v = *reinterpret_cast<const uint4*>(R + (int64_t)(row0 + t) * dm.d + c0 + c);
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      T x;
      Elem<T>::store(&x, dm.eta * chunk_value<T>(v, e));
      lds_store<T>(smem + (c + e) * St::kStride + t * (int)sizeof(T), x);
    }
  }
  __syncthreads();
  St::flush_tokens(smem, Vt, dm.d, c0, ncols, row0, BT, chunk_map(dm));
}

// ===================================================================== S4
// For each sequence b and fast-weight tile (m0.., n0..), over the chunks
// g0 .. g0+gc-1 in order:
//   slot[jj] <- W                        (the weight chunk g0+jj uses)
//   W        <- W + (eta V^_i)^T Z_i      (MFMA accumulation into the fp32 tile)
// and finally W_state <- W.  The accumulator is the fp32 state itself, so the
// result does not depend on how the chunks are grouped.  The tile shape S
// divides d and f exactly (the host picks it), so every tile is full.
// Tile `blk` of `nblk` (workgroups [0, nblk) of the launch are these tiles).
// kSlots: the slot layout, one of bits 0-2 -- 1: `slots` [G][B][d][f] (what
// the outputs read); 2: `slots_t` [G][B][f][d], the weights transposed (the
// backward's products that contract over d read them with K contiguous); 4:
// `slots` in TB x TB tiles, element (m, n) of a slot at
// ((m / TB) (f / TB) + n / TB) TB^2 + (m % TB) TB + n % TB with TB = 128
// bytes of T -- every k-tile of a product that contracts over d (k-major) or
// over f (rows of 128 bytes) is then whole 128-row blocks of TB rows each,
// contiguous in memory.  Bit 3 (bf16 and waves of 128 x 64 only): the same
// layout, each wave's 32-row block rows staged through a 4 KB region of LDS
// past the k-tile stages (the caller's `smem` holds S::kLdsBytes +
// kSlotStageBytes) and stored 16 bytes per lane as whole row segments (128
// bytes of a row, 64 of a transposed row, 4 KB runs of a tile): 16 store
// instructions per lane and slot instead of 64 (32 transposed).
template <typename T, class S, int kSlots = 1, bool kRevChunks = false>
__device__ __forceinline__ void prefix_update_tile(const Dims& dm, const T* __restrict__ Vt,
                                                   const T* __restrict__ Zt,
                                                   float* __restrict__ W_state,
                                                   T* __restrict__ slots, int64_t g0, int64_t gc,
                                                   int blk, int nblk, lds_char* smem,
                                                   T* __restrict__ slots_t = nullptr) {
  constexpr int TB = kRowBytes / (int)sizeof(T);
  const int64_t d = dm.d, f = dm.f;
  const int tiles_m = (int)(d / S::BM);
  const int tiles_n = (int)(f / S::BN);
  const int per_seq = tiles_m * tiles_n;
  const int L = xcd_remap(blk, nblk);
  const int64_t b = L / per_seq;
  const TileCoord tc = grouped_tile(L - (int)b * per_seq, tiles_m, tiles_n, 4);
  const int64_t m0 = (int64_t)tc.m * S::BM, n0 = (int64_t)tc.n * S::BN;
  const int64_t kb0 = (b * dm.N + g0) * dm.Cp / TB;  // first k-block of the group

  DirectLoader<S::BM, S::kWaves> la;
  la.init(reinterpret_cast<const char*>(Vt) + (kb0 * d + m0) * kRowBytes, kRowBytes,
          d * kRowBytes, (d - m0) * kRowBytes, 0);
  DirectLoader<S::BN, S::kWaves> lb;
  lb.init(reinterpret_cast<const char*>(Zt) + (kb0 * f + n0) * kRowBytes, kRowBytes,
          f * kRowBytes, (f - n0) * kRowBytes, 0);

  const LanePos p = lane_pos<S>();
  // Accumulator element (i, j, 4q + e) of this lane is W[m][n] with
  //   m = m0 + wave_m0 + 32 i + 8 q + 4 (lane / 32) + e,  n = n0 + wave_n0 + 32 j + lane % 32.
  // Buffer accesses: per-lane offset for each e (4 registers), the uniform
  // row part (32 i + 8 q) f as the scalar offset, 32 j as the immediate.
  uint32_t lane_e[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    lane_e[e] = (uint32_t)((p.wave_m0 + 4 * (p.lane >> 5) + e) * f + p.wave_n0 + (p.lane & 31));
  const int64_t corner = m0 * f + n0;
  const int64_t span = (d - m0) * f - n0;  // elements addressable from the corner
  const uint32_t fu = (uint32_t)f;

  const rsrc_t wr = make_rsrc(W_state + b * d * f + corner, span * 4);
  Accum<S> acc;
#pragma unroll
  for (int i = 0; i < S::MB; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t so = (uint32_t)(32 * i + 8 * q) * fu * 4u;
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int j = 0; j < S::NB; ++j)
          acc.v[i][j][4 * q + e] = __builtin_bit_cast(
              float, __builtin_amdgcn_raw_buffer_load_b32(wr, (lane_e[e] + 32 * j) * 4, so, 0));
      __builtin_amdgcn_sched_barrier(0);
    }

  const int64_t slot_stride = dm.B * d * f;
  // bf16 slots leave as 32-bit column pairs (pair_pack): half the store
  // instructions of 16-bit stores
  const bool odd = p.lane & 1;
  uint32_t lane_pair[2];
#pragma unroll
  for (int r = 0; r < 2; ++r)
    lane_pair[r] = (uint32_t)((p.wave_m0 + 4 * (p.lane >> 5) + (odd ? 2 : 0) + r) * f +
                              p.wave_n0 + ((p.lane & 31) & ~1)) * 2u;
  // store instructions per lane of one slot: row-major pairs (bf16) or
  // values (fp32); transposed, 4 consecutive rows of a column in one store
  constexpr int kLayout = kSlots & 7;
  constexpr bool kStaged = (kSlots & 8) != 0;
  static_assert(kLayout == 1 || kLayout == 2 || kLayout == 4, "one slot layout");
  static_assert(!kStaged || (sizeof(T) == 2 && S::WM == 128 && S::WN == 64),
                "staged slots: bf16, waves of 128 x 64");
  const uint32_t lane_t = (uint32_t)(((p.wave_n0 + (p.lane & 31)) * d + p.wave_m0 +
                                      4 * (p.lane >> 5)) * (int64_t)sizeof(T));
  const uint32_t du = (uint32_t)d;
  auto write_slot_t = [&](int64_t js) {
    const rsrc_t sr = make_rsrc(slots_t + js * slot_stride + b * d * f + n0 * d + m0,
                                ((f - n0) * d - m0) * (int64_t)sizeof(T));
#pragma unroll
    for (int i = 0; i < S::MB; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
#pragma unroll
        for (int j = 0; j < S::NB; ++j) {
          const uint32_t so = (uint32_t)(32 * j * du + 32 * i + 8 * q) * (uint32_t)sizeof(T);
          float z[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) z[e] = acc.v[i][j][4 * q + e];
          if constexpr (sizeof(T) == 2) {
            typedef uint32_t u2 __attribute__((ext_vector_type(2)));
            __builtin_amdgcn_raw_buffer_store_b64(u2{pack_bf16x2(z[0], z[1]), pack_bf16x2(z[2], z[3])},
                                                  sr, lane_t, so, 0);
          } else {
            __builtin_amdgcn_raw_buffer_store_b128(
                u32x4_t{__float_as_uint(z[0]), __float_as_uint(z[1]), __float_as_uint(z[2]),
                        __float_as_uint(z[3])},
                sr, lane_t, so, 0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
  };
  // Tiled slots: the lane's part of the offset (its rows and columns inside a
  // 32 x 32 block, and the wave's corner), and per block (i, q, j) a uniform
  // part.  A wave's rows (columns) stay inside one tile row (column) of TB:
  // the wave tiles start on multiples of TB, or a block of 32 is all a wave
  // holds.
  static_assert((32 * S::MB) % TB == 0 || S::MB == 1, "wave rows inside whole tiles");
  static_assert((32 * S::NB) % TB == 0 || S::NB == 1, "wave columns inside whole tiles");
  const int64_t fT = f / TB;
  const int64_t corner_t = ((m0 / TB) * fT + n0 / TB) * TB * TB;
  const uint32_t wave_t = (uint32_t)((p.wave_m0 / TB) * fT * TB * TB + (p.wave_m0 % TB) * TB +
                                     (p.wave_n0 / TB) * TB * TB + p.wave_n0 % TB);
  uint32_t lane_tl[4];  // bf16: pair rows r = 0, 1; fp32: rows e = 0..3
#pragma unroll
  for (int e = 0; e < 4; ++e)
    lane_tl[e] = sizeof(T) == 2
                     ? wave_t + (uint32_t)((4 * (p.lane >> 5) + (odd ? 2 : 0) + (e & 1)) * TB +
                                           ((p.lane & 31) & ~1))
                     : wave_t + (uint32_t)((4 * (p.lane >> 5) + e) * TB + (p.lane & 31));
  auto tiled_uniform = [&](int i, int q, int j) -> uint32_t {
    const int r = 32 * i + 8 * q, c = 32 * j;
    return (uint32_t)(((r / TB) * fT + c / TB) * TB * TB + (r % TB) * TB + c % TB);
  };
  auto write_slot_tiled = [&](int64_t js) {
    const rsrc_t sr = make_rsrc(slots + js * slot_stride + b * d * f + corner_t,
                                (d * f - corner_t) * (int64_t)sizeof(T));
#pragma unroll
    for (int i = 0; i < S::MB; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int j = 0; j < S::NB; ++j) {
            const uint32_t so = tiled_uniform(i, q, j) * 2u;
            float z[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) z[e] = acc.v[i][j][4 * q + e];
            uint32_t w[2];
            pair_pack(z, odd, w);
#pragma unroll
            for (int r = 0; r < 2; ++r)
              __builtin_amdgcn_raw_buffer_store_b32(w[r], sr, lane_tl[r] * 2u, so, 0);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int j = 0; j < S::NB; ++j)
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc.v[i][j][4 * q + e]), sr,
                                                    lane_tl[e] * 4u, tiled_uniform(i, q, j) * 4u,
                                                    0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
  };
  // Staged slots: block row i of the wave (32 rows x 64 columns, bf16) goes
  // to the wave's LDS region and back as 16-byte chunks, one row segment per
  // 2-8 lanes, then out with one 16-byte store per chunk.  Rows and tiles:
  // the LDS image is row-major (row r at r * 128 bytes, its 16-byte chunk c
  // at c ^ (r & 7)), written as column pairs; lane l reads chunk l & 7 of
  // row 8 s + l / 8.  Transposed: the image is column-major (column n at
  // n * 64 bytes, chunk c -- rows 8 c .. 8 c + 7 -- at c ^ ((n / 4) & 3)),
  // written as the lane's 4 consecutive rows of a column; lane l reads chunk
  // l & 3 of column 16 s + l / 4.  Both swizzles keep the writes at two
  // passes and the reads conflict-free.  A wave's LDS accesses run in order,
  // so each block row's reads come before the next one's writes.
  lds_char* const stage_slot = smem + S::kLdsBytes + (threadIdx.x >> 6) * 4096;
  uint32_t lane_st = 0, wave_st = 0;  // per-lane and per-wave byte offsets of the stores
  int64_t base_st = 0, span_st = 0;   // first element and extent from it
  if constexpr (kLayout == 1) {
    lane_st = (uint32_t)((p.lane >> 3) * f + 8 * (p.lane & 7)) * 2u;
    wave_st = (uint32_t)(p.wave_m0 * f + p.wave_n0) * 2u;
    base_st = b * d * f + corner;
    span_st = span;
  } else if constexpr (kLayout == 2) {
    lane_st = (uint32_t)((p.lane >> 2) * d + 8 * (p.lane & 3)) * 2u;
    wave_st = (uint32_t)(p.wave_n0 * d + p.wave_m0) * 2u;
    base_st = b * d * f + n0 * d + m0;
    span_st = (f - n0) * d - m0;
  } else {
    lane_st = (uint32_t)(8 * p.lane) * 2u;  // 8 rows of TB values: 1 KB in a row of lanes
    wave_st = (uint32_t)((p.wave_m0 / TB) * fT * TB * TB + (p.wave_n0 / TB) * TB * TB) * 2u;
    base_st = b * d * f + corner_t;
    span_st = d * f - corner_t;
  }
  auto staged_uniform = [&](int i, int s4) -> uint32_t {
    if constexpr (kLayout == 1) return (uint32_t)((32 * i + 8 * s4) * f) * 2u;
    if constexpr (kLayout == 2) return (uint32_t)(16 * s4 * d + 32 * i) * 2u;
    const int r = 32 * i + 8 * s4;  // rows of the wave; TB = 64 divides 32 * 2
    return (uint32_t)((r / TB) * fT * TB * TB + (r % TB) * TB) * 2u;
  };
  auto write_slot_staged = [&](int64_t js) {
    T* const dst = kLayout == 2 ? slots_t : slots;
    const rsrc_t sr = make_rsrc(dst + js * slot_stride + base_st, span_st * (int64_t)sizeof(T));
#pragma unroll
    for (int i = 0; i < S::MB; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int j = 0; j < S::NB; ++j) {
          float z[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) z[e] = acc.v[i][j][4 * q + e];
          if constexpr (kLayout == 2) {
            const int n = 32 * j + (p.lane & 31);
            lds_store<u32x2_t>(stage_slot + n * 64 + ((q ^ ((n >> 2) & 3)) << 4) +
                                   (p.lane >> 5) * 8,
                               u32x2_t{pack_bf16x2(z[0], z[1]), pack_bf16x2(z[2], z[3])});
          } else {
            uint32_t w[2];
            pair_pack(z, odd, w);
#pragma unroll
            for (int r = 0; r < 2; ++r) {
              const int row = 8 * q + 4 * (p.lane >> 5) + (odd ? 2 : 0) + r;
              const int col = 32 * j + ((p.lane & 31) & ~1);
              lds_store<uint32_t>(stage_slot + row * kRowBytes +
                                      ((((col >> 3) ^ (row & 7))) << 4) + (col & 7) * 2,
                                  w[r]);
            }
          }
        }
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        u32x4_t v;
        if constexpr (kLayout == 2) {
          const int n = 16 * s4 + (p.lane >> 2);
          v = lds_load<u32x4_t>(stage_slot + n * 64 + (((p.lane & 3) ^ ((n >> 2) & 3)) << 4));
        } else {
          const int row = 8 * s4 + (p.lane >> 3);
          v = lds_load<u32x4_t>(stage_slot + row * kRowBytes + ((((p.lane & 7) ^ (row & 7))) << 4));
        }
        // non-temporal (cache policy nt): the slot is read back by the next
        // launch's output tiles, long after it has left this XCD's L2
        __builtin_amdgcn_raw_buffer_store_b128(v, sr, lane_st, wave_st + staged_uniform(i, s4), 2);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto write_slot = [&](int64_t jj) {
    const int64_t js = dm.reverse_slots ? gc - 1 - jj : jj;
    if constexpr (kStaged) {
      write_slot_staged(js);
      return;
    }
    if constexpr (kLayout == 2) write_slot_t(js);
    if constexpr (kLayout == 4) write_slot_tiled(js);
    if constexpr (kLayout != 1) return;
    const rsrc_t sr = make_rsrc(slots + js * slot_stride + b * d * f + corner,
                                span * (int64_t)sizeof(T));
#pragma unroll
    for (int i = 0; i < S::MB; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t so = (uint32_t)(32 * i + 8 * q) * fu * (uint32_t)sizeof(T);
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int j = 0; j < S::NB; ++j) {
            float z[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) z[e] = acc.v[i][j][4 * q + e];
            uint32_t w[2];
            pair_pack(z, odd, w);
#pragma unroll
            for (int r = 0; r < 2; ++r)
              __builtin_amdgcn_raw_buffer_store_b32(w[r], sr, lane_pair[r] + 64 * j, so, 0);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int j = 0; j < S::NB; ++j)
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc.v[i][j][4 * q + e]), sr,
                                                    (lane_e[e] + 32 * j) * 4, so, 0);
        }
        // one row group at a time: keeps the compiler from hoisting every
        // accumulator read (and conversion) ahead of the stores
        __builtin_amdgcn_sched_barrier(0);
      }
  };

  // none: the increments' sum only
  const bool with_slots = kLayout == 2 ? slots_t != nullptr : slots != nullptr;
  if (with_slots) write_slot(0);
  const int64_t kt_per_chunk = dm.Cp / TB;
  // a streaming call leaves the sequence's last chunk out of the state (its
  // last token's target needs the next call's first token); its slot is
  // still written
  const bool skip = dm.skip_last && g0 + gc == dm.N;
  const int64_t nk = (skip ? gc - 1 : gc) * kt_per_chunk;
  // Slot jj (the weight after jj chunks) is stored before the MFMAs of the
  // chunk's first k-tile and drains while they run, ahead of the next
  // k-tile's loads (spread over the MFMAs for bf16).
  int64_t next_slot = 1, next_slot_kt = kt_per_chunk;  // counters, not a division per k-tile
  // kRevChunks: the group's chunks in reverse order (each chunk's k-tiles in
  // order) from operands stored in forward order
  mainloop_with_stores<T, S>(
      acc, la, lb, nk, smem, p,
      [&](int64_t kt) {
        if (kt != next_slot_kt || !with_slots) return;
        write_slot(next_slot);
        ++next_slot;
        next_slot_kt += kt_per_chunk;
      },
      [&](int64_t kt) -> int64_t {
        if constexpr (kRevChunks) {
          const int64_t c = kt / kt_per_chunk;
          return (gc - 1 - 2 * c) * kt_per_chunk + kt;
        } else {
          return kt;
        }
      });
  if (skip && gc > 1 && with_slots) write_slot(gc - 1);

#pragma unroll
  for (int i = 0; i < S::MB; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t so = (uint32_t)(32 * i + 8 * q) * fu * 4u;
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int j = 0; j < S::NB; ++j)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc.v[i][j][4 * q + e]), wr,
                                                (lane_e[e] + 32 * j) * 4, so, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
}

// kOcc: workgroups meant to share a CU (the register budget follows).
template <typename T, class S, int kSlots = 1, int kOcc = 1, bool kRevChunks = false>
__global__ __launch_bounds__(S::kThreads) __attribute__((amdgpu_waves_per_eu(
    kOcc * S::kWaves / 4, kOcc * S::kWaves / 4))) void prefix_update_kernel(
    Dims dm, const T* __restrict__ Vt, const T* __restrict__ Zt, float* __restrict__ W_state,
    T* __restrict__ slots, int64_t g0, int64_t gc, T* __restrict__ slots_t) {
  __shared__ __attribute__((aligned(16))) char smem_raw[S::kLdsBytes];
  prefix_update_tile<T, S, kSlots, kRevChunks>(dm, Vt, Zt, W_state, slots, g0, gc, blockIdx.x,
                                               gridDim.x, (lds_char*)smem_raw, slots_t);
}

// ===================================================================== S3
// O_i = Z_i slot_i^T for every chunk of the group and every sequence.
// Tile `blk` of `nblk` (the launch's workgroups [first, first + nblk), first a
// multiple of 8 so that the XCD of workgroup first + blk is blk % 8).
// Zs: bf16 -- the token-major Zt the scan reads, taken as a k-major A tile
// (a tile's 256 token rows are 4 consecutive 64-token blocks) and read with
// transposed fragment loads, so S1 writes Z in this one layout; fp32 -- the
// row-major Z.
template <typename T>
__device__ __forceinline__ void down_proj_tile(const Dims& dm, const T* __restrict__ Zs,
                                               const T* __restrict__ slots, T* __restrict__ O,
                                               int64_t g0, int64_t gc, int blk, int nblk,
                                               lds_char* smem) {
  using S = OutTile;
  const int64_t d = dm.d, f = dm.f, C = dm.C, T_seq = dm.T;
  const int64_t ld = f * (int64_t)sizeof(T);
  const int tiles_m = (int)((C + S::BM - 1) / S::BM);
  const int tiles_n = (int)((d + S::BN - 1) / S::BN);
  const int per_chunk = tiles_m * tiles_n;
  const int L = xcd_remap(blk, nblk);
  const int64_t cb = L / per_chunk;  // = b * gc + jj
  const int64_t b = cb / gc, jj = cb - b * gc;
  const int64_t chunk = g0 + jj;
  const TileCoord tc = grouped_tile(L - (int)cb * per_chunk, tiles_m, tiles_n, tiles_m);
  const int64_t c_begin = chunk * C;
  const int64_t c_len = min(C, T_seq - c_begin);
  const int64_t m0 = (int64_t)tc.m * S::BM, n0 = (int64_t)tc.n * S::BN;
  const int64_t row0 = b * T_seq + c_begin + m0;  // first token row of the tile
  const T* slot = slots + (jj * dm.B + b) * d * f;

  // the slot in TB x TB tiles: k-tile kt of slot rows n0.. is tile column kt
  // of each TB-row block (block rows f * 128 bytes apart)
  static_assert(kFwdSlots == 4, "tiled forward slots");
  constexpr int TB = kRowBytes / (int)sizeof(T);
  DirectLoader<S::BN, S::kWaves> lb;
  lb.init_blocked(reinterpret_cast<const char*>(slot) + (n0 / TB) * f * kRowBytes, TB,
                  f * kRowBytes, TB * kRowBytes, ((d - n0) / TB) * f * kRowBytes, TB * kRowBytes);

  Accum<S> acc;
  acc.zero();
  const LanePos p = lane_pos<S>();
  if constexpr (sizeof(T) == 2) {
    static_assert(S::BM == 256, "four 64-token blocks per tile");
    // token column of tile row 0; rows past the chunk read the next chunk's
    // columns (or zeros past the end), which only reach output rows that are
    // not stored
    const int64_t col0 = (b * dm.N + chunk) * dm.Cp + m0;
    const int64_t block_bytes = f * kRowBytes;
    KMajorLoader<T, S::kWaves> la;
    la.init(reinterpret_cast<const char*>(Zs) + (col0 / kTokenAlign) * block_bytes, block_bytes,
            kRowBytes, kTokenAlign * kRowBytes, (dm.P - col0) / kTokenAlign * block_bytes);
    // one load per MFMA: the output tiles' operands come from HBM (slots of the
    // previous launch, Z of the previous group), so they are issued early
    mainloop<T, S, true, true, false, 1>(acc, la, lb, ld / kRowBytes, smem, p, [](int64_t) {});
  } else {
    DirectLoader<S::BM, S::kWaves> la;
    la.init(reinterpret_cast<const char*>(Zs) + row0 * ld, ld, kRowBytes, (c_len - m0) * ld,
            kRowBytes);
    mainloop<T, S>(acc, la, lb, ld / kRowBytes, smem, p, [](int64_t) {});
  }

  // O through the stage, four passes of 64 columns, written row-major; rows
  // beyond the chunk are skipped, and so are the first out_skip rows of each
  // session (tokens a previous streaming call has already output).
  const int32_t rows_valid = (int32_t)min<int64_t>(S::BM, c_len - m0);
  const int64_t srow = c_begin + m0;  // session row of tile row 0
  const int32_t rows_lo = (int32_t)max<int64_t>(0, min<int64_t>(S::BM, dm.out_skip - srow));
  const int64_t out_T = dm.out_T > 0 ? dm.out_T : T_seq;
#pragma unroll
  for (int q = 0; q < S::BN / 64; ++q) {
    stage_cols<T, S>(smem, acc, p, q, [](float x) { return x; });
    __syncthreads();
    const int64_t cbase = n0 + 64 * q;
    Stage<T, S::kThreads>::flush_rows(smem, O, b * out_T + srow - dm.out_skip, d, cbase,
                                      (int)max<int64_t>(0, min<int64_t>(64, d - cbase)),
                                      rows_lo, rows_valid);
    __syncthreads();
  }
}

template <typename T>
TTT_GEMM_KERNEL void down_proj_kernel(Dims dm, const T* __restrict__ Z,
                                      const T* __restrict__ slots, T* __restrict__ O, int64_t g0,
                                      int64_t gc) {
  __shared__ __attribute__((aligned(16))) char smem_raw[Tile::kLdsBytes];
  down_proj_tile<T>(dm, Z, slots, O, g0, gc, blockIdx.x, gridDim.x, (lds_char*)smem_raw);
}

// ============================================================== S4 + S3
// One launch of the group pipeline: the scan tiles of chunks g0.. and the
// outputs of chunks a0.. of the previous group, whose slots the previous
// launch completed.  The longer kind of tile is dispatched first (the scan's
// k-loop is the group's tokens, the outputs' is f): workgroups [0, n1) run
// it, [n1, pad) exit at once (pad rounds n1 up to a multiple of 8, so the
// second kind starts on XCD 0), the rest run the other kind.
template <typename T, int kScanSlots = 1>
TTT_GEMM_KERNEL void scan_apply_kernel(Dims dm, const T* __restrict__ Vt, const T* __restrict__ Zt,
                                       float* __restrict__ W_state, T* __restrict__ scan_slots,
                                       int64_t g0, int64_t gc, int n1, int pad, int outputs_first,
                                       const T* __restrict__ Z, const T* __restrict__ apply_slots,
                                       T* __restrict__ O, int64_t a0, int64_t ac) {
  static_assert(Tile::kThreads == PrefixTile::kThreads && Tile::kLdsBytes == PrefixTile::kLdsBytes,
                "both parts share the launch shape");
  __shared__ __attribute__((aligned(16)))
  char smem_raw[Tile::kLdsBytes + ((kScanSlots & 8) ? kSlotStageBytes : 0)];
  const int b = blockIdx.x;
  const int n2 = (int)gridDim.x - pad;
  const bool first = b < pad;
  if (first && b >= n1) return;
  const int blk = first ? b : b - pad, nblk = first ? n1 : n2;
  if (first != (outputs_first != 0))
    prefix_update_tile<T, PrefixTile, kScanSlots>(dm, Vt, Zt, W_state, scan_slots, g0, gc, blk,
                                                  nblk, (lds_char*)smem_raw);
  else
    down_proj_tile<T>(dm, Z, apply_slots, O, a0, ac, blk, nblk, (lds_char*)smem_raw);
}

// The first launch of the group pipeline when the projection of later
// chunks is still to do: workgroups [0, scan_blocks) scan chunks g0.. (as in
// scan_apply_kernel), the rest project token rows [t_lo, T) of every
// sequence.  The scan tiles alone fill about 1.5 waves of the chip; the
// projection tiles fill the rest.  The scan reads the target columns of
// chunks g0 .. g0 + gc - 1, the projection writes those of chunks from t_lo
// on: disjoint 64-token blocks.
template <typename T, int kScanSlots = 1>
TTT_GEMM_KERNEL void scan_target_kernel(Dims dm, const T* __restrict__ Vt,
                                        const T* __restrict__ Zt, float* __restrict__ W_state,
                                        T* __restrict__ scan_slots, int64_t g0, int64_t gc,
                                        int scan_blocks, int scan_pad, const T* __restrict__ rows,
                                        const T* __restrict__ WtT, T* __restrict__ Vt_out,
                                        int64_t t_lo) {
  constexpr int kScanLds = PrefixTile::kLdsBytes + ((kScanSlots & 8) ? kSlotStageBytes : 0);
  constexpr int kLds = TargetLds<T>::kBytes > kScanLds ? TargetLds<T>::kBytes : kScanLds;
  __shared__ __attribute__((aligned(16))) char smem_raw[kLds];
  const int b = blockIdx.x;
  if (b < scan_pad) {
    if (b < scan_blocks)
      prefix_update_tile<T, PrefixTile, kScanSlots>(dm, Vt, Zt, W_state, scan_slots, g0, gc, b,
                                                    scan_blocks, (lds_char*)smem_raw);
    return;
  }
  target_tile<T>(dm, rows, WtT, Vt_out, t_lo, dm.T, b - scan_pad, (int)gridDim.x - scan_pad,
                 (lds_char*)smem_raw);
}

// Two independent scans of all N chunks (the backward's forward weights and
// its chunk-reversed gradient sums) in one launch: one group of all chunks
// gives ~1.5 waves of tiles per scan, two together fill the chip better.  The
// first writes its slots transposed (slots1t), the second in TB x TB tiles
// (slots2; see prefix_update_tile).
template <typename T>
TTT_GEMM_KERNEL void dual_scan_kernel(Dims d1, const T* __restrict__ Vt1, const T* __restrict__ Zt1,
                                      float* __restrict__ W1, T* __restrict__ slots1t, Dims d2,
                                      const T* __restrict__ Vt2, const T* __restrict__ Zt2,
                                      float* __restrict__ W2, T* __restrict__ slots2, int blocks,
                                      int pad) {
  constexpr int kStage = sizeof(T) == 2 ? 8 : 0;  // bf16 slots staged through LDS
  __shared__ __attribute__((aligned(16)))
  char smem_raw[Tile::kLdsBytes + (kStage ? kSlotStageBytes : 0)];
  const int b = blockIdx.x;
  if (b < pad) {
    if (b < blocks)
      prefix_update_tile<T, PrefixTile, 2 | kStage>(d1, Vt1, Zt1, W1, nullptr, 0, d1.N, b, blocks,
                                                    (lds_char*)smem_raw, slots1t);
  } else if (b - pad < blocks) {
    prefix_update_tile<T, PrefixTile, 4 | kStage, true>(d2, Vt2, Zt2, W2, slots2, 0, d2.N,
                                                        b - pad, blocks, (lds_char*)smem_raw);
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

// WgU[(n/32)*64 + (n%32)] = W_gate[n], WgU[(n/32)*64 + 32 + (n%32)] = W_up[n]
// (rows of d elements), 16 bytes per thread; tb > 0: in tb x tb tiles.
__global__ void interleave_kernel(uint4* __restrict__ dst, const uint4* __restrict__ wg,
                                  const uint4* __restrict__ wu, int64_t f, int64_t row_vecs,
                                  int32_t tb) {
  const int64_t total = 2 * f * row_vecs;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += stride) {
    const int64_t r = e / row_vecs, v = e - r * row_vecs;
    const int64_t blk = r / 64, w = r % 64;
    const int64_t n = blk * 32 + (w & 31);
    // tb > 0: row r, vector v in TB x TB tiles (8 vectors of 16 bytes per tile row)
    const int64_t at = tb > 0 ? ((r / tb) * (row_vecs / 8) + v / 8) * (tb * 8) + (r % tb) * 8 + v % 8
                              : e;
    dst[at] = (w < 32 ? wg : wu)[n * row_vecs + v];
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

// Zero the padding token columns (index inside the chunk >= chunk length) of
// Zt and Vt (k-blocked, f and d rows).
template <typename T>
__global__ void pad_fill_kernel(T* __restrict__ a, int64_t Ra, T* __restrict__ b, int64_t Rb,
                                Dims dm) {
  const int64_t rows = Ra + Rb;
  const int64_t total = rows * dm.P;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += stride) {
    const int64_t row = e / dm.P, col = e - row * dm.P;
    const int64_t q = col / dm.Cp, j = col - q * dm.Cp;
    const int64_t i = q % dm.N;
    const int64_t len = min(dm.C, dm.T - i * dm.C);
    if (j < len) continue;
    if (row < Ra)
      Elem<T>::store(a + kblock_index<T>(row, col, Ra), 0.0f);
    else
      Elem<T>::store(b + kblock_index<T>(row - Ra, col, Rb), 0.0f);
  }
}

// ========================================================= streaming calls
// A streaming call runs the layer on a virtual sequence per session: the
// carried rows of the pending chunk (n_pend tokens that an earlier call has
// seen but whose chunk update is still open) followed by the call's L new
// tokens.  Carry of a session (element offsets, e = element type):
//   H rows   [C][d]            at 0
//   X0 rows  [kHaloRows + C][d] at C * d: the kHaloRows rows before the
//            pending chunk, then its rows
// All copies move 16-byte chunks of rows.
template <typename T>
__global__ void stream_build_kernel(const T* __restrict__ H, const T* __restrict__ X0,
                                    const T* __restrict__ carry, T* __restrict__ Hv,
                                    T* __restrict__ X0v, int64_t B, int64_t L, int64_t n_pend,
                                    int64_t C, int64_t d) {
  constexpr int EPC = Elem<T>::kPerChunk;
  const int64_t Tv = n_pend + L, cpr = d / EPC, per_seq = Tv * cpr;
  const int64_t carry_seq = (C + kHaloRows + C) * d;
  for (int64_t it = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; it < 2 * B * per_seq;
       it += (int64_t)gridDim.x * blockDim.x) {
    const bool x = it >= B * per_seq;  // second half: X0
    const int64_t j = x ? it - B * per_seq : it;
    const int64_t b = j / per_seq, r = j % per_seq / cpr, c = j % cpr * EPC;
    const T* src;
    if (r < n_pend)
      src = carry + b * carry_seq + (x ? (C + kHaloRows + r) * d : r * d) + c;
    else
      src = (x ? X0 : H) + (b * L + r - n_pend) * d + c;
    T* dst = (x ? X0v : Hv) + (b * Tv + r) * d + c;
    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
  }
}

// The carry after a call, into `out` (a separate buffer: the halo of the new
// pending chunk may come from the old carry).  Pending chunk = virtual rows
// [c_new, Tv); its halo = virtual rows [c_new - kHaloRows, c_new), read from
// X0v, or before the virtual start from the old carry's halo (zeros at the
// stream's start: `old` is null there).
template <typename T>
__global__ void stream_save_kernel(const T* __restrict__ Hv, const T* __restrict__ X0v,
                                   const T* __restrict__ old, T* __restrict__ out, int64_t B,
                                   int64_t Tv, int64_t c_new, int64_t C, int64_t d) {
  constexpr int EPC = Elem<T>::kPerChunk;
  const int64_t cpr = d / EPC, n_new = Tv - c_new;
  const int64_t rows = n_new + kHaloRows + n_new;  // H rows, then halo + X0 rows
  const int64_t carry_seq = (C + kHaloRows + C) * d;
  for (int64_t it = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; it < B * rows * cpr;
       it += (int64_t)gridDim.x * blockDim.x) {
    const int64_t b = it / (rows * cpr), r = it % (rows * cpr) / cpr, c = it % cpr * EPC;
    uint4 v = make_uint4(0, 0, 0, 0);
    T* dst;
    if (r < n_new) {  // H row c_new + r
      v = *reinterpret_cast<const uint4*>(Hv + (b * Tv + c_new + r) * d + c);
      dst = out + b * carry_seq + r * d + c;
    } else {  // X0 row j of the halo + pending block = virtual row c_new - kHaloRows + j
      const int64_t j = r - n_new, vr = c_new - kHaloRows + j;
      if (vr >= 0)
        v = *reinterpret_cast<const uint4*>(X0v + (b * Tv + vr) * d + c);
      else if (old != nullptr)
        v = *reinterpret_cast<const uint4*>(old + b * carry_seq + (C + kHaloRows + vr) * d + c);
      dst = out + b * carry_seq + (C + j) * d + c;
    }
    *reinterpret_cast<uint4*>(dst) = v;
  }
}

// ================================================================ launchers
static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

WorkspacePlan plan_workspace(const Dims& dm, int64_t group, bool row_z) {
  const size_t es = dtype_bytes(dm.dt);
  WorkspacePlan w;
  size_t off = 0;
  w.z_off = off;  // Z row-major (fp32 outputs and the backward read it)
  if (row_z || dm.dt == Dtype::F32) off = align256(off + (size_t)(dm.B * dm.T) * dm.f * es);
  w.u_off = off;  // U of S2 (the conv output the projection reads)
  off = align256(off + (size_t)(dm.B * dm.T) * dm.d * es);
  w.zt_off = off;
  off = align256(off + (size_t)dm.f * dm.P * es);
  w.vt_off = off;
  off = align256(off + (size_t)dm.d * dm.P * es);
  w.wgu_off = off;
  off = align256(off + (size_t)2 * dm.f * dm.d * es);
  w.wtt_off = off;
  off = align256(off + (size_t)dm.d * dm.d * es);
  w.taps_off = off;
  off = align256(off + (size_t)8 * dm.d * sizeof(float));
  w.slots_off = off;
  w.fixed_bytes = off;
  w.slot_bytes = align256((size_t)dm.B * dm.d * dm.f * es);
  w.group = group;
  w.slot_sets = group < dm.N ? 2 : 1;
  w.total_bytes = off + (size_t)(w.slot_sets * group) * w.slot_bytes;
  return w;
}

static inline unsigned grid_for(int64_t n, int64_t per_block, int64_t cap) {
  return (unsigned)std::max<int64_t>(1, std::min<int64_t>((n + per_block - 1) / per_block, cap));
}

hipError_t launch_state_reset(float* W_state, const void* W0, Dtype w0_dt, int64_t B, int64_t d,
                              int64_t f, hipStream_t s) {
  const int64_t n = d * f;
  if (w0_dt == Dtype::BF16)
    hipLaunchKernelGGL(state_reset_kernel<uint16_t>, dim3(grid_for(n, 256, 8192)), dim3(256), 0, s,
                       W_state, static_cast<const uint16_t*>(W0), B, n);
  else
    hipLaunchKernelGGL(state_reset_kernel<float>, dim3(grid_for(n, 256, 8192)), dim3(256), 0, s,
                       W_state, static_cast<const float*>(W0), B, n);
  return hipGetLastError();
}

hipError_t launch_weight_prep(const Dims& dm, const void* Wg, const void* Wu, const void* Wt,
                              const void* taps, void* WgU, void* WtT, float* tapsT,
                              hipStream_t s) {
  const int64_t row_vecs = dm.d * (int64_t)dtype_bytes(dm.dt) / 16;
  hipLaunchKernelGGL(interleave_kernel, dim3(grid_for(2 * dm.f * row_vecs, 256, 16384)), dim3(256),
                     0, s, static_cast<uint4*>(WgU), static_cast<const uint4*>(Wg),
                     static_cast<const uint4*>(Wu), dm.f, row_vecs,
                     wgu_tiled(dm.d, (int64_t)dtype_bytes(dm.dt))
                         ? (int32_t)(kRowBytes / dtype_bytes(dm.dt))
                         : 0);
  const dim3 tgrid((unsigned)((dm.d + 63) / 64), (unsigned)((dm.d + 63) / 64));
  const unsigned tblocks = (unsigned)((dm.d + 255) / 256);
  if (dm.dt == Dtype::BF16) {
    if (dm.proj)
      hipLaunchKernelGGL(transpose_kernel<uint16_t>, tgrid, dim3(256), 0, s,
                         static_cast<uint16_t*>(WtT), static_cast<const uint16_t*>(Wt), dm.d);
    if (dm.conv)
      hipLaunchKernelGGL(taps_kernel<uint16_t>, dim3(tblocks), dim3(256), 0, s, tapsT,
                         static_cast<const uint16_t*>(taps), dm.d, dm.K);
  } else {
    if (dm.proj)
      hipLaunchKernelGGL(transpose_kernel<float>, tgrid, dim3(256), 0, s, static_cast<float*>(WtT),
                         static_cast<const float*>(Wt), dm.d);
    if (dm.conv)
      hipLaunchKernelGGL(taps_kernel<float>, dim3(tblocks), dim3(256), 0, s, tapsT,
                         static_cast<const float*>(taps), dm.d, dm.K);
  }
  return hipGetLastError();
}

hipError_t launch_pad_fill(void* a, int64_t Ra, void* b, int64_t Rb, const Dims& dm,
                          hipStream_t s) {
  const int64_t total = (Ra + Rb) * dm.P;
  if (total == 0) return hipSuccess;
  if (dm.dt == Dtype::BF16)
    hipLaunchKernelGGL(pad_fill_kernel<uint16_t>, dim3(grid_for(total, 256, 65536)), dim3(256), 0,
                       s, static_cast<uint16_t*>(a), Ra, static_cast<uint16_t*>(b), Rb, dm);
  else
    hipLaunchKernelGGL(pad_fill_kernel<float>, dim3(grid_for(total, 256, 65536)), dim3(256), 0, s,
                       static_cast<float*>(a), Ra, static_cast<float*>(b), Rb, dm);
  return hipGetLastError();
}

hipError_t launch_swiglu(const Dims& dm, const void* H, const void* WgU, void* Z, void* Zt,
                         hipStream_t s) {
  const int64_t BT = dm.B * dm.T;
  const int64_t tiles =
      ((BT + Tile::BM - 1) / Tile::BM) * ((dm.f + Tile::BN / 2 - 1) / (Tile::BN / 2));
  if (dm.dt == Dtype::BF16)
    hipLaunchKernelGGL(swiglu_kernel<uint16_t>, dim3((unsigned)tiles), dim3(Tile::kThreads), 0, s, dm,
                       static_cast<const uint16_t*>(H), static_cast<const uint16_t*>(WgU),
                       static_cast<uint16_t*>(Z), static_cast<uint16_t*>(Zt));
  else
    hipLaunchKernelGGL(swiglu_kernel<float>, dim3((unsigned)tiles), dim3(Tile::kThreads), 0, s, dm,
                       static_cast<const float*>(H), static_cast<const float*>(WgU),
                       static_cast<float*>(Z), static_cast<float*>(Zt));
  return hipGetLastError();
}

template <typename T>
static void launch_target_t(const Dims& dm, const T* X0, const float* tapsT, const T* WtT, T* U,
                            T* Vt, int64_t t_hi, T* V, hipStream_t s) {
  const int64_t BT = dm.B * dm.T;
  const T* rows = X0;  // the rows the projection (or the copy into Vt) reads
  if (dm.conv) {
    const int64_t items = (BT + kConvRows - 1) / kConvRows * (dm.d / Elem<T>::kPerChunk);
    const dim3 cgrid(grid_for(items, 256, 65536));
    if (dm.K <= 4)
      hipLaunchKernelGGL((conv_kernel<T, 4>), cgrid, dim3(256), 0, s, dm, X0, tapsT, U);
    else
      hipLaunchKernelGGL((conv_kernel<T, 8>), cgrid, dim3(256), 0, s, dm, X0, tapsT, U);
    rows = U;
  }
  if (dm.proj) {
    if (t_hi <= 0) return;
    const int64_t tiles = ((t_hi + Tile::BM - 1) / Tile::BM) * dm.B * ((dm.d + Tile::BN - 1) / Tile::BN);
    if (V != nullptr)
      hipLaunchKernelGGL((target_kernel<T, true>), dim3((unsigned)tiles), dim3(Tile::kThreads), 0,
                         s, dm, rows, WtT, Vt, (int64_t)0, t_hi, V);
    else
      hipLaunchKernelGGL((target_kernel<T, false>), dim3((unsigned)tiles), dim3(Tile::kThreads), 0,
                         s, dm, rows, WtT, Vt, (int64_t)0, t_hi, V);
  } else {
    hipLaunchKernelGGL(rows_to_vt_kernel<T>, dim3((unsigned)((BT + 255) / 256), (unsigned)((dm.d + 63) / 64)),
                       dim3(256), 0, s, dm, rows, Vt);
  }
}

hipError_t launch_target(const Dims& dm, const void* X0, const void* tapsT, const void* WtT,
                         void* U, void* Vt, hipStream_t s, int64_t t_hi, void* V) {
  if (t_hi < 0) t_hi = dm.T;
  if (V != nullptr && (!dm.proj || t_hi != dm.T)) return hipErrorInvalidValue;
  if (dm.dt == Dtype::BF16)
    launch_target_t<uint16_t>(dm, static_cast<const uint16_t*>(X0),
                              static_cast<const float*>(tapsT), static_cast<const uint16_t*>(WtT),
                              static_cast<uint16_t*>(U), static_cast<uint16_t*>(Vt), t_hi,
                              static_cast<uint16_t*>(V), s);
  else
    launch_target_t<float>(dm, static_cast<const float*>(X0), static_cast<const float*>(tapsT),
                           static_cast<const float*>(WtT), static_cast<float*>(U),
                           static_cast<float*>(Vt), t_hi, static_cast<float*>(V), s);
  return hipGetLastError();
}

template <typename T>
static void launch_scan_target_t(const Dims& dm, const T* Vt, const T* Zt, float* W_state,
                                 T* scan_slots, int64_t gc, const T* rows, const T* WtT,
                                 int64_t t_lo, hipStream_t s) {
  const int64_t scan = (dm.d / PrefixTile::BM) * (dm.f / PrefixTile::BN) * dm.B;
  const int64_t pad = (scan + 7) / 8 * 8;
  const int64_t tiles =
      ((dm.T - t_lo + Tile::BM - 1) / Tile::BM) * dm.B * ((dm.d + Tile::BN - 1) / Tile::BN);
  if constexpr (sizeof(T) == 2) {
    if (staged_slots<T>(dm)) {
      hipLaunchKernelGGL((scan_target_kernel<T, kFwdSlots | 8>), dim3((unsigned)(pad + tiles)),
                         dim3(Tile::kThreads), 0, s, dm, Vt, Zt, W_state, scan_slots, (int64_t)0,
                         gc, (int)scan, (int)pad, rows, WtT, const_cast<T*>(Vt), t_lo);
      return;
    }
  }
  hipLaunchKernelGGL((scan_target_kernel<T, kFwdSlots>), dim3((unsigned)(pad + tiles)),
                     dim3(Tile::kThreads), 0, s, dm, Vt, Zt, W_state, scan_slots, (int64_t)0, gc,
                     (int)scan, (int)pad, rows, WtT, const_cast<T*>(Vt), t_lo);
}

bool scan_target_fits(const Dims& dm) {
  return dm.proj && dm.d % PrefixTile::BM == 0 && dm.f % PrefixTile::BN == 0;
}

hipError_t launch_scan_target(const Dims& dm, void* Vt, const void* Zt, float* W_state,
                              void* scan_slots, int64_t gc, const void* rows, const void* WtT,
                              int64_t t_lo, hipStream_t s) {
  if (!scan_target_fits(dm) || t_lo <= 0 || t_lo >= dm.T) return hipErrorInvalidValue;
  if (dm.dt == Dtype::BF16)
    launch_scan_target_t<uint16_t>(dm, static_cast<const uint16_t*>(Vt),
                                   static_cast<const uint16_t*>(Zt), W_state,
                                   static_cast<uint16_t*>(scan_slots), gc,
                                   static_cast<const uint16_t*>(rows),
                                   static_cast<const uint16_t*>(WtT), t_lo, s);
  else
    launch_scan_target_t<float>(dm, static_cast<const float*>(Vt), static_cast<const float*>(Zt),
                                W_state, static_cast<float*>(scan_slots), gc,
                                static_cast<const float*>(rows), static_cast<const float*>(WtT),
                                t_lo, s);
  return hipGetLastError();
}

template <typename T>
static void launch_scan_apply_t(const Dims& dm, const T* Vt, const T* Zt, float* W_state,
                                T* scan_slots, int64_t g0, int64_t gc, const T* Z,
                                const T* apply_slots, T* O, int64_t a0, int64_t ac, hipStream_t s) {
  if (sizeof(T) == 2) Z = Zt;  // bf16 outputs read the token-major Z (down_proj_tile)
  const int64_t down_tiles = ac > 0 ? ((dm.C + Tile::BM - 1) / Tile::BM) *
                                          ((dm.d + Tile::BN - 1) / Tile::BN) * ac * dm.B
                                    : 0;
  if (gc == 1 && ac == 0 && dm.d % OneChunkTile::BM == 0 && dm.f % OneChunkTile::BN == 0) {
    // one chunk's update alone (sequential mode): 128 x 128 tiles, two
    // workgroups per CU, so that one's state load and store overlap the
    // other's MFMAs, and four times the tiles to spread over the CUs
    hipLaunchKernelGGL((prefix_update_kernel<T, OneChunkTile, kFwdSlots, 2>),
                       dim3((unsigned)((dm.d / OneChunkTile::BM) * (dm.f / OneChunkTile::BN) * dm.B)),
                       dim3(OneChunkTile::kThreads), 0, s, dm, Vt, Zt, W_state, scan_slots, g0, gc,
                       static_cast<T*>(nullptr));
    return;
  }
  if (dm.d % PrefixTile::BM == 0 && dm.f % PrefixTile::BN == 0) {
    const int64_t scan = gc > 0 ? (dm.d / PrefixTile::BM) * (dm.f / PrefixTile::BN) * dm.B : 0;
    if (scan + down_tiles == 0) return;
    // longest first: a scan tile runs over the group's gc * Cp tokens, an
    // output tile over the f features
    const bool outputs_first = down_tiles > 0 && scan > 0 && gc * dm.Cp < dm.f;
    const int64_t n1 = outputs_first ? down_tiles : scan, n2 = outputs_first ? scan : down_tiles;
    const int64_t pad = (n1 + 7) / 8 * 8;
    if constexpr (sizeof(T) == 2) {
      if (staged_slots<T>(dm)) {
        hipLaunchKernelGGL((scan_apply_kernel<T, kFwdSlots | 8>), dim3((unsigned)(pad + n2)),
                           dim3(Tile::kThreads), 0, s, dm, Vt, Zt, W_state, scan_slots, g0, gc,
                           (int)n1, (int)pad, outputs_first ? 1 : 0, Z, apply_slots, O, a0, ac);
        return;
      }
    }
    hipLaunchKernelGGL((scan_apply_kernel<T, kFwdSlots>), dim3((unsigned)(pad + n2)),
                       dim3(Tile::kThreads), 0, s, dm, Vt, Zt, W_state, scan_slots, g0, gc,
                       (int)n1, (int)pad, outputs_first ? 1 : 0, Z, apply_slots, O, a0, ac);
    return;
  }
  // 64 x 64 scan tiles when 256 does not divide the weight (d and f are
  // multiples of 64): two launches in the same order.
  using Small = TileShape<64, 64, 2, 2>;
  if (gc > 0)
    hipLaunchKernelGGL((prefix_update_kernel<T, Small, kFwdSlots>),
                       dim3((unsigned)((dm.d / Small::BM) * (dm.f / Small::BN) * dm.B)),
                       dim3(Small::kThreads), 0, s, dm, Vt, Zt, W_state, scan_slots, g0, gc,
                       static_cast<T*>(nullptr));
  if (down_tiles > 0)
    hipLaunchKernelGGL(down_proj_kernel<T>, dim3((unsigned)down_tiles), dim3(Tile::kThreads), 0, s,
                       dm, Z, apply_slots, O, a0, ac);
}

hipError_t launch_scan_apply(const Dims& dm, const void* Vt, const void* Zt, float* W_state,
                             void* scan_slots, int64_t g0, int64_t gc, const void* Z,
                             const void* apply_slots, void* O, int64_t a0, int64_t ac,
                             hipStream_t s) {
  if (dm.dt == Dtype::BF16)
    launch_scan_apply_t<uint16_t>(dm, static_cast<const uint16_t*>(Vt),
                                  static_cast<const uint16_t*>(Zt), W_state,
                                  static_cast<uint16_t*>(scan_slots), g0, gc,
                                  static_cast<const uint16_t*>(Z),
                                  static_cast<const uint16_t*>(apply_slots),
                                  static_cast<uint16_t*>(O), a0, ac, s);
  else
    launch_scan_apply_t<float>(dm, static_cast<const float*>(Vt), static_cast<const float*>(Zt),
                               W_state, static_cast<float*>(scan_slots), g0, gc,
                               static_cast<const float*>(Z), static_cast<const float*>(apply_slots),
                               static_cast<float*>(O), a0, ac, s);
  return hipGetLastError();
}

template <typename T>
static void launch_dual_scan_t(const Dims& d1, const T* Vt1, const T* Zt1, float* W1, T* slots1t,
                               const Dims& d2, const T* Vt2, const T* Zt2, float* W2, T* slots2,
                               hipStream_t s) {
  if (d1.d % PrefixTile::BM != 0 || d1.f % PrefixTile::BN != 0) {
    // 64 x 64 tiles when 256 does not divide the weight: two launches
    using Small = TileShape<64, 64, 2, 2>;
    const dim3 grid((unsigned)((d1.d / Small::BM) * (d1.f / Small::BN) * d1.B));
    hipLaunchKernelGGL((prefix_update_kernel<T, Small, 2>), grid, dim3(Small::kThreads), 0, s, d1,
                       Vt1, Zt1, W1, static_cast<T*>(nullptr), (int64_t)0, d1.N, slots1t);
    hipLaunchKernelGGL((prefix_update_kernel<T, Small, 4, 1, true>), grid, dim3(Small::kThreads),
                       0, s, d2, Vt2, Zt2, W2, slots2, (int64_t)0, d2.N, static_cast<T*>(nullptr));
    return;
  }
  const int blocks = (int)((d1.d / PrefixTile::BM) * (d1.f / PrefixTile::BN) * d1.B);
  const int pad = (blocks + 7) / 8 * 8;  // the second scan starts on XCD 0
  hipLaunchKernelGGL(dual_scan_kernel<T>, dim3((unsigned)(pad + blocks)), dim3(Tile::kThreads), 0,
                     s, d1, Vt1, Zt1, W1, slots1t, d2, Vt2, Zt2, W2, slots2, blocks, pad);
}

hipError_t launch_dual_scan(const Dims& d1, const void* Vt1, const void* Zt1, float* W1,
                            void* slots1t, const Dims& d2, const void* Vt2, const void* Zt2,
                            float* W2, void* slots2, hipStream_t s) {
  if (d1.dt == Dtype::BF16)
    launch_dual_scan_t<uint16_t>(d1, static_cast<const uint16_t*>(Vt1),
                                 static_cast<const uint16_t*>(Zt1), W1,
                                 static_cast<uint16_t*>(slots1t), d2,
                                 static_cast<const uint16_t*>(Vt2),
                                 static_cast<const uint16_t*>(Zt2), W2,
                                 static_cast<uint16_t*>(slots2), s);
  else
    launch_dual_scan_t<float>(d1, static_cast<const float*>(Vt1), static_cast<const float*>(Zt1),
                              W1, static_cast<float*>(slots1t), d2,
                              static_cast<const float*>(Vt2), static_cast<const float*>(Zt2), W2,
                              static_cast<float*>(slots2), s);
  return hipGetLastError();
}

hipError_t launch_stream_build(const Dims& dv, const void* H, const void* X0, const void* carry,
                               void* Hv, void* X0v, int64_t L, int64_t n_pend, int64_t C,
                               hipStream_t s) {
  const int64_t n = 2 * dv.B * dv.T * (dv.d / (16 / (int64_t)dtype_bytes(dv.dt)));
  const dim3 g(grid_for(n, 256, 65536));
  if (dv.dt == Dtype::BF16)
    hipLaunchKernelGGL(stream_build_kernel<uint16_t>, g, dim3(256), 0, s,
                       static_cast<const uint16_t*>(H), static_cast<const uint16_t*>(X0),
                       static_cast<const uint16_t*>(carry), static_cast<uint16_t*>(Hv),
                       static_cast<uint16_t*>(X0v), dv.B, L, n_pend, C, dv.d);
  else
    hipLaunchKernelGGL(stream_build_kernel<float>, g, dim3(256), 0, s,
                       static_cast<const float*>(H), static_cast<const float*>(X0),
                       static_cast<const float*>(carry), static_cast<float*>(Hv),
                       static_cast<float*>(X0v), dv.B, L, n_pend, C, dv.d);
  return hipGetLastError();
}

hipError_t launch_stream_save(const Dims& dv, const void* Hv, const void* X0v, const void* old,
                              void* out, int64_t c_new, int64_t C, hipStream_t s) {
  const int64_t rows = 2 * (dv.T - c_new) + kHaloRows;
  const int64_t n = dv.B * rows * (dv.d / (16 / (int64_t)dtype_bytes(dv.dt)));
  const dim3 g(grid_for(n, 256, 65536));
  if (dv.dt == Dtype::BF16)
    hipLaunchKernelGGL(stream_save_kernel<uint16_t>, g, dim3(256), 0, s,
                       static_cast<const uint16_t*>(Hv), static_cast<const uint16_t*>(X0v),
                       static_cast<const uint16_t*>(old), static_cast<uint16_t*>(out), dv.B,
                       dv.T, c_new, C, dv.d);
  else
    hipLaunchKernelGGL(stream_save_kernel<float>, g, dim3(256), 0, s,
                       static_cast<const float*>(Hv), static_cast<const float*>(X0v),
                       static_cast<const float*>(old), static_cast<float*>(out), dv.B, dv.T,
                       c_new, C, dv.d);
  return hipGetLastError();
}

}  // namespace ttt
