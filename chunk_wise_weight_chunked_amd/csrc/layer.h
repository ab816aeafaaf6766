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
  bool skip_last = false;      // leave the last chunk's update out of the state
  bool reverse_slots = false;  // the scan writes chunk jj's slot at gc - 1 - jj
  int64_t out_skip = 0;        // rows [0, out_skip) of each session are not output ...
  int64_t out_T = 0;           // ... and output row t goes to O row b * out_T + t - out_skip
};

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

WorkspacePlan plan_workspace(const Dims& dm, int64_t group);

// Kernel launchers (asynchronous on `s`; return hipGetLastError()).
hipError_t launch_state_reset(float* W_state, const void* W0, Dtype w0_dt, int64_t B, int64_t d,
                              int64_t f, hipStream_t s);
// W_gate/W_up interleaved into WgU, W_target transposed into WtT, taps to fp32 tapsT.
hipError_t launch_weight_prep(const Dims& dm, const void* Wg, const void* Wu, const void* Wt,
                              const void* taps, void* WgU, void* WtT, float* tapsT, hipStream_t s);
hipError_t launch_pad_fill(void* zt, void* vt, const Dims& dm, hipStream_t s);
hipError_t launch_swiglu(const Dims& dm, const void* H, const void* WgU, void* Z, void* Zt,
                         hipStream_t s);
// eta * V^ into Vt: the conv of X0 into U (scratch of B*T x d elements) if
// dm.conv, then the projection by W_target if dm.proj (each part left out is
// the identity).  With a projection, t_hi >= 0 projects only token rows
// [0, t_hi) of each sequence (the conv always covers all rows).
hipError_t launch_target(const Dims& dm, const void* X0, const void* taps, const void* WtT,
                         void* U, void* Vt, hipStream_t s, int64_t t_hi = -1);
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

// Backward-pass kernels (backward.hip).
constexpr int kTargetBackwardRows = 256;  // token rows per partial sum of the taps' gradient
constexpr int kDotPartials = 1024;        // partial sums of the learning rate's gradient
// dst = rows of src [B][T][R] in the k-blocked token-major layout (chunks
// reversed if `reverse`), zeros in the padding columns.
hipError_t launch_to_kblocked(const void* src, void* dst, const Dims& dm, int64_t R, bool reverse,
                              hipStream_t s);
// Z [B*T][f] = SiLU(A_g) * A_u (activation type) from fp32 pre-activations
// (row t of A_g and A_u at t * ld).
hipError_t launch_swiglu_rows(const float* Ag, const float* Au, int64_t ld, void* Z,
                              const Dims& dm, hipStream_t s);
// The scans of two independent problems (same shapes) in one launch.
hipError_t launch_dual_scan(const Dims& d1, const void* Vt1, const void* Zt1, float* W1,
                            void* slots1, const Dims& d2, const void* Vt2, const void* Zt2,
                            float* W2, void* slots2, hipStream_t s);
// dA [B*T][2f] = [dA_g | dA_u] from dZ (fp32 [B*T][f]) and A_g, A_u (fp32,
// row t at t * ld).
hipError_t launch_swiglu_backward(const float* dZ, const float* Ag, const float* Au, int64_t ld,
                                  void* dA, const Dims& dm, hipStream_t s);
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
