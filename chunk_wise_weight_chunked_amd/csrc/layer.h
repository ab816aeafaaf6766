// layer.h -- internal interface between the C ABI (api.cpp) and the HIP
// kernels (kernels.hip) of the TTT-MLP layer.  Not part of the public header.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ttt {

enum class Dtype : int { F32 = 0, BF16 = 1 };

inline size_t dtype_bytes(Dtype t) { return t == Dtype::F32 ? 4 : 2; }

// Shapes of one call, with the derived chunk geometry.
//   N  = ceil(T / C) chunks per sequence;
//   Cp = C rounded up to 64 tokens: the chunk stride of the token-major
//        layouts Zt and Vt, whose extra columns hold zeros;
//   P  = B * N * Cp columns of Zt and Vt.
// X0 rows a streaming call keeps before each session's first row (the conv
// reaches back K - 2 <= 6 tokens, K - 1 <= 7 with the reconstruction alignment).
constexpr int kHaloRows = 7;

struct Dims {
  int64_t B, T, d, f, C, N, Cp, P;
  int32_t K;
  float eta;
  Dtype dt;
  bool conv, proj;  // the target's conv and projection (both: the method)
  int32_t shift = 1;  // conv tap k reads X0 row t + shift - k (1: next-token alignment)
  // Streaming continuation (defaults give the one-shot layer):
  const void* halo = nullptr;  // [B][halo_stride]: kHaloRows X0 rows before each session's row 0
  int64_t halo_stride = 0;     // elements between sessions in `halo`
  // A share of a longer sequence (context parallelism): the X0 row after each
  // session's last row (null: the sequence ends there, zero padding).
  const void* halo_r = nullptr;  // [B][halo_r_stride]
  int64_t halo_r_stride = 0;
  bool skip_last = false;      // leave the last chunk's update out of the state
  bool reverse_slots = false;  // the scan writes chunk jj's slot at gc - 1 - jj
  int64_t out_skip = 0;        // rows [0, out_skip) of each session are not output ...
  int64_t out_T = 0;           // ... and output row t goes to O row b * out_T + t - out_skip
};

// Token row t's column in the chunk-padded token-major layouts is t itself:
// whole chunks (T a multiple of C) and no padding (Cp = C).
__host__ __device__ inline bool chunk_map_is_identity(const Dims& dm) {
  return dm.Cp == dm.C && dm.N * dm.C == dm.T;
}

// WgU (the interleaved gate/up weight, d elements of es bytes per row) is
// stored in TB x TB tiles of 128-byte rows when a row is longer than 4 KB: a
// k-tile of 256 WgU rows is then four contiguous 8 KB tiles instead of 256
// segments a row apart.  Shorter rows stay row-major (a 256-row block is
// contiguous there already, and tiles measured slower).
__host__ __device__ inline bool wgu_tiled(int64_t d, int64_t es) { return d * es > 4096; }

// Workspace regions (byte offsets from the workspace base, 256-byte aligned).
// The slots are one set of G per group, two sets when there are several
// groups: the scan of group g+1 writes one set while the outputs of group g
// read the other.
struct WorkspacePlan {
  size_t z_off, u_off, zt_off, vt_off, wgu_off, wtt_off, taps_off, slots_off;
  size_t slot_bytes;   // one chunk slot for all B sequences: B * d * f * es
  size_t fixed_bytes;  // everything except the slots
  int64_t group;       // chunks per group G
  int64_t slot_sets;   // 1 if G covers all chunks, else 2
  size_t total_bytes;  // fixed_bytes + slot_sets * group * slot_bytes
};

// row_z: keep a row-major Z region even for bf16 (the backward builds Z there;
// the bf16 forward writes Z only token-major).
WorkspacePlan plan_workspace(const Dims& dm, int64_t group, bool row_z = false);

// Kernel launchers (asynchronous on `s`; return hipGetLastError()).
hipError_t launch_state_reset(float* W_state, const void* W0, Dtype w0_dt, int64_t B, int64_t d,
                              int64_t f, hipStream_t s);
// W_gate/W_up interleaved into WgU, W_target transposed into WtT, taps to fp32 tapsT.
hipError_t launch_weight_prep(const Dims& dm, const void* Wg, const void* Wu, const void* Wt,
                              const void* taps, void* WgU, void* WtT, float* tapsT, hipStream_t s);
// Zeros at the padding token columns (j >= chunk length) of two k-blocked
// token-major matrices: a with Ra rows, b with Rb rows (Rb = 0: a only).
hipError_t launch_pad_fill(void* a, int64_t Ra, void* b, int64_t Rb, const Dims& dm,
                           hipStream_t s);
hipError_t launch_swiglu(const Dims& dm, const void* H, const void* WgU, void* Z, void* Zt,
                         hipStream_t s);
// eta * V^ into Vt: the conv of X0 into U (scratch of B*T x d elements) if
// dm.conv, then the projection by W_target if dm.proj (each part left out is
// the identity).  With a projection, t_hi >= 0 projects only token rows
// [0, t_hi) of each sequence (the conv always covers all rows); V (not null:
// a projection of all rows only) also receives V^ unscaled, row-major
// [B*T][d].
hipError_t launch_target(const Dims& dm, const void* X0, const void* taps, const void* WtT,
                         void* U, void* Vt, hipStream_t s, int64_t t_hi = -1, void* V = nullptr);
// Whether launch_scan_target serves these dims (a projection, and the scan
// tiles divide the weight).
bool scan_target_fits(const Dims& dm);
// The first pipeline launch together with the rest of the projection: scan of
// chunks [0, gc) (slots into scan_slots, state in W_state) and projection of
// token rows [t_lo, T) of every sequence from `rows` (U, or X0 without a
// conv) into Vt.  0 < t_lo < T, and the chunks [0, gc) end at or before t_lo.
hipError_t launch_scan_target(const Dims& dm, void* Vt, const void* Zt, float* W_state,
                              void* scan_slots, int64_t gc, const void* rows, const void* WtT,
                              int64_t t_lo, hipStream_t s);
// One step of the group pipeline: the scan (S4) of chunks [g0, g0 + gc) into
// scan_slots, and the outputs (S3) of chunks [a0, a0 + ac) from apply_slots;
// gc == 0 or ac == 0 leaves that part out.  Both parts run in one launch
// where the tile shapes allow, so the outputs fill the CUs the scan's last
// partial wave of tiles leaves idle.
hipError_t launch_scan_apply(const Dims& dm, const void* Vt, const void* Zt, float* W_state,
                             void* scan_slots, int64_t g0, int64_t gc, const void* Z,
                             const void* apply_slots, void* O, int64_t a0, int64_t ac,
                             hipStream_t s);

// Streaming calls: the virtual sequences (carried pending rows + the call's L
// new rows) into Hv / X0v, and the carry after the call (pending chunk from
// virtual row c_new on, with its halo) into `out`.
hipError_t launch_stream_build(const Dims& dv, const void* H, const void* X0, const void* carry,
                               void* Hv, void* X0v, int64_t L, int64_t n_pend, int64_t C,
                               hipStream_t s);
hipError_t launch_stream_save(const Dims& dv, const void* Hv, const void* X0v, const void* old,
                              void* out, int64_t c_new, int64_t C, hipStream_t s);

// Decode kernels (bf16 only).  Z[M][f] = SiLU(H W_gateᵀ) ⊙ (H W_upᵀ) for M <= 64
// rows, with the new H and X0 rows of the sessions in `mask` appended to their
// carries' pending chunks (at n_pend[b]; a zero halo for those in zero_halo)
// in the same launch; O[b][L][d] = Z[b][L] W_cur[b]ᵀ for L <= 16 rows of each
// session in `mask`; W_cur = bf16(W_state).  At most kDecodeMaxSessions sessions.
constexpr int kDecodeMaxSessions = 64;
hipError_t launch_decode_swiglu(const void* H, int64_t M, const void* Wg, const void* Wu, void* Z,
                                int64_t d, int64_t f, const void* X0, void* carry, int64_t B,
                                int64_t L, const int64_t* n_pend, int64_t C, uint64_t mask,
                                uint64_t zero_halo, hipStream_t s);
hipError_t launch_decode_down(const void* Z, const void* Wc, void* O, int64_t B, int64_t L,
                              int64_t d, int64_t f, uint64_t mask, hipStream_t s);
hipError_t launch_state_to_bf16(const float* W, void* out, int64_t n, hipStream_t s);
// The allocation-free decode call's scratch for its gated activations (at
// most kDecodeMaxSessions rows of d_ff bf16 values in all: 64 rows of up to
// 32768 features): the calling thread's current device's address of a static
// device array, looked up once per device.
constexpr size_t kDecodeScratchBytes = (size_t)4 << 20;
hipError_t decode_scratch_ptr(void** out);

// Batched GEMM on the library's mainloop (gemm.hip):
//   C[b] = alpha * A[b] B[b]ᵀ   (accumulate: C[b] += ...)
// over b < batch, A [M][K] and B [N][K] of element type dt; C [M][ldc] fp32
// (c_f32) or of type dt.  Operand layouts (X = A or B, rows = M or N, ld = lda
// or ldb, TB = 128 / element bytes):
//   kRowK     X[r][k] at r * ld + k                  (K contiguous)
//   kKMajor   X[r][k] at k * ld + r                  ([K][ld] row-major)
//   kKBlocked X[r][k] at ((k / TB) * ld + r) * TB + k % TB  (ld = rows per
//             block: the k-blocked token-major layouts, K = token columns)
//   kTiledRowK   X[r][k] at ((r / TB) (ld / TB) + k / TB) TB^2 + (r % TB) TB
//             + k % TB  (TB x TB tiles, K contiguous inside; ld = K)
//   kTiledKMajor X[r][k] at ((k / TB) (ld / TB) + r / TB) TB^2 + (k % TB) TB
//             + r % TB  (the same tiles of a [K][ld] matrix; ld = row count)
// (a weight slot in tiles, [d/TB][f/TB][TB][TB], is kTiledRowK with r = d,
// k = f and kTiledKMajor with k = d, r = f).  Tiled operands need their row
// count and ld to be multiples of TB and whole matrices between batches.
// Element offsets between batches sa, sb, sc (for kKBlocked, a row offset
// r0 * TB or whole blocks); the last batch contracts K_last values (split
// products: batch = K slice).  kRowK, kKBlocked and the tiled layouts need K
// and K_last to be multiples of TB; N a multiple of 8.
enum GemmLayout : int32_t {
  kRowK = 0,
  kKMajor = 1,
  kKBlocked = 2,
  kTiledRowK = 3,
  kTiledKMajor = 4
};
struct GemmArgs {
  Dtype dt;
  const void* A;
  int64_t lda, sa;
  int32_t a_layout;
  const void* B;
  int64_t ldb, sb;
  int32_t b_layout;
  void* C;
  int64_t ldc, sc;
  int32_t c_f32, accumulate;
  int64_t M, N, K, K_last, batch;
  float alpha;
};
hipError_t launch_gemm(const GemmArgs& g, hipStream_t s);
// The backward's dZ and SwiGLU derivative in one launch.  Per batch b,
// dZ[b] = g.alpha (A[b] B[b]ᵀ + g2.alpha A2[b] B2[b]ᵀ) (g's operands (kRowK,
// kRowK), g2's (kRowK, kTiledKMajor); g's M, N = f and batch; the second
// product runs first on the same accumulators) stays in the tile; with
// s = sigmoid(A_g), the epilogue writes dA_g = dZ A_u s (1 + A_g (1 - s)) and
// dA_u = dZ A_g s for the tile's tokens, row t of batch b being token row
// row0 + b * row_stride + t of the whole batch of sequences: row-major into
// dA [BT][2f] (dA_g at [0, f), dA_u at [f, 2f)) and k-blocked token-major into
// dAk ([P/TB][2f][TB], the chunk-padded token columns of dm; padding columns
// are not written).  Ag [BT][2f] fp32 holds A_g and A_u the same way.
hipError_t launch_dz_swiglu(const GemmArgs& g, const GemmArgs& g2, const Dims& dm, int64_t row0,
                            int64_t row_stride, const float* Ag, void* dA, void* dAk,
                            hipStream_t s);
// The backward's pre-activations and gated activations in one launch:
// Ag [BT][2f] fp32 (A_g at columns [0, f), A_u at [f, 2f)) = H WgUᵀ with the
// interleaved gate/up weight WgU of launch_weight_prep, and Z [BT][f] =
// SiLU(A_g) * A_u in type dt.  d and f multiples of 64.
hipError_t launch_preact_swiglu(Dtype dt, const void* H, const void* WgU, int64_t BT, int64_t d,
                                int64_t f, float* Ag, void* Z, hipStream_t s);
// dst [cols][ld_dst] = srcᵀ into columns [col0, col0 + rows) of each dst row,
// for src [rows][cols] of element type dt; ld_dst < 0: rows.  tiled: dst in
// TB x TB tiles of 128-byte rows (ld_dst and cols multiples of TB).
hipError_t launch_transpose(const void* src, void* dst, int64_t rows, int64_t cols, Dtype dt,
                            hipStream_t s, int64_t ld_dst = -1, int64_t col0 = 0,
                            bool tiled = false);

// Backward-pass kernels (backward.hip).
constexpr int kTargetBackwardRows = 256;  // token rows per partial sum of the taps' gradient
constexpr int kDotPartials = 1024;        // partial sums of the learning rate's gradient
// dst = rows of src [B][T][R] in the k-blocked token-major layout, zeros in
// the padding columns.
hipError_t launch_to_kblocked(const void* src, void* dst, const Dims& dm, int64_t R,
                              hipStream_t s);
// The scans of two independent problems (same shapes) in one launch: the
// first writes its slots transposed ([N][B][f][d], slots1t), the second in
// tiles of TB x TB (slots2: [N][B][d/TB][f/TB][TB][TB], TB = 128 bytes of the
// type) and walks its chunks last to first (operands in forward order).
hipError_t launch_dual_scan(const Dims& d1, const void* Vt1, const void* Zt1, float* W1,
                            void* slots1t, const Dims& d2, const void* Vt2, const void* Zt2,
                            float* W2, void* slots2, hipStream_t s);
// dX0 and dtaps from dU = scale * src (fp32 [B*T][d]); `part` holds
// target_backward_ranges(dm) * 8 * d floats.
int64_t target_backward_ranges(const Dims& dm);
hipError_t launch_target_backward(const float* src, float scale, const void* X0,
                                  const float* tapsT, void* dX0, float* part, float* dtaps,
                                  const Dims& dm, hipStream_t s);
// *out = scale * sum_i a[i] b[i] (a: activation type, b: fp32); `part` holds
// kDotPartials floats.
hipError_t launch_dot(const void* a, const float* b, int64_t n, Dtype dt, float scale, float* part,
                      float* out, hipStream_t s);
hipError_t launch_from_f32(const float* in, void* out, int64_t n, Dtype dt, hipStream_t s);
hipError_t launch_fill_f32(float* out, int64_t n, float v, hipStream_t s);
// out[i] = sum over s < slices (in order) of part[s * n + i].
hipError_t launch_sum_slices(const float* part, float* out, int64_t n, int slices,
                             hipStream_t s);

}  // namespace ttt
