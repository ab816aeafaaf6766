// backward_api.cpp -- C ABI of the layer's backward pass: validation,
// workspace planning and the launch sequence (own kernels and rocBLAS GEMMs)
// on the caller's stream.  Semantics in include/ttt_mlp.h.
#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>

#include <algorithm>
#include <string>

#include "../../include/ttt_mlp.h"
#include "api_common.h"
#include "layer.h"

using namespace ttt::api;

namespace {

// Workspace of the backward pass: the forward's regions with one group of all
// N chunks (its slots hold every chunk's weight W^(j-1)), then the backward's
// own regions, 256-byte aligned.
struct BackwardPlan {
  ttt::WorkspacePlan fwd;
  size_t wst, u, v, agu, ztr, dotr, sslots, dz, da, wgu, g, gf, du, tpart, dpart, wtpart,
      blas, total;
  int64_t wt_slices;  // token slices of the dW_target product (split over K = B*T)
};

constexpr size_t kBlasWorkspace = (size_t)32 << 20;

BackwardPlan plan_backward(const ttt::Dims& dm) {
  BackwardPlan p;
  p.fwd = ttt::plan_workspace(dm, dm.N);
  const size_t es = ttt::dtype_bytes(dm.dt), BT = (size_t)(dm.B * dm.T);
  const size_t d = dm.d, f = dm.f;
  size_t off = p.fwd.total_bytes;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = (off + bytes + 255) & ~(size_t)255;
    return at;
  };
  p.wst = take((size_t)dm.B * d * f * 4);                 // fp32 state of the forward scan
  p.u = take(dm.conv ? BT * d * es : 0);                  // conv output U
  p.v = take(dm.proj ? BT * d * es : 0);                  // V^ = U W_target, row-major
  p.agu = take(BT * 2 * f * 4);                           // [A_g | A_u] per row (fp32)
  p.ztr = take(f * (size_t)dm.P * es);                    // Zt, chunks reversed
  p.dotr = take(d * (size_t)dm.P * es);                   // dOᵀ k-blocked, chunks reversed
  p.sslots = take((size_t)dm.N * dm.B * d * f * es);      // S_j, reversed chunk order
  p.dz = take(BT * f * 4);                                // dZ (fp32)
  p.da = take(BT * 2 * f * es);                           // [dA_g | dA_u]
  p.wgu = take(2 * f * d * es);                           // [W_gate; W_up]
  p.gf = take(BT * d * 4);                                // G = Z_j S_jᵀ (dV^ = eta G), fp32
  p.g = take(dm.proj ? BT * d * es : 0);                  // G rounded: the GEMMs' operand
  p.du = take(dm.proj ? BT * d * 4 : 0);                  // dU (fp32)
  p.tpart = take((size_t)ttt::target_backward_ranges(dm) * 8 * d * 4);
  p.dpart = take((size_t)ttt::kDotPartials * 4);
  // dW_target = Uᵀ dV^ is d x d with K = B*T: one product per slice of about
  // 2048 tokens keeps the GPU busy, the slices are then added in order
  p.wt_slices = dm.proj ? std::max<int64_t>(1, std::min<int64_t>(16, (int64_t)BT / 2048)) : 0;
  p.wtpart = take((size_t)p.wt_slices * d * d * 4);
  p.blas = take(kBlasWorkspace);
  p.total = off;
  return p;
}

// One rocBLAS handle per host thread, kept for the life of the process.
rocblas_handle blas_handle() {
  thread_local rocblas_handle h = nullptr;
  if (!h && rocblas_create_handle(&h) != rocblas_status_success) h = nullptr;
  return h;
}

// Row-major C[M][N] (ldc) = alpha op(A) op(B) + beta C, op(A) [M][K], op(B)
// [K][N]: A is stored [M][K] (lda), or [K][M] when ta; B is [K][N] (ldb), or
// [N][K] when tb.  rocBLAS is column-major, so it computes Cᵀ = op(B)ᵀ op(A)ᵀ.
// `batch` products at the given element strides.
struct Gemm {
  rocblas_handle h;
  rocblas_datatype ab;  // type of A and B
  rocblas_status st = rocblas_status_success;
  void operator()(bool ta, bool tb, int64_t M, int64_t N, int64_t K, float alpha, const void* A,
                  int64_t lda, int64_t sa, const void* B, int64_t ldb, int64_t sb, float beta,
                  void* C, int64_t ldc, int64_t sc, int64_t batch, rocblas_datatype ctype) {
    if (st != rocblas_status_success || M == 0 || N == 0) return;
    st = rocblas_gemm_strided_batched_ex_64(
        h, tb ? rocblas_operation_transpose : rocblas_operation_none,
        ta ? rocblas_operation_transpose : rocblas_operation_none, N, M, K, &alpha, B, ab, ldb, sb,
        A, ab, lda, sa, &beta, C, ctype, ldc, sc, C, ctype, ldc, sc, batch, rocblas_datatype_f32_r,
        rocblas_gemm_algo_standard, 0, 0);
  }
};

}  // namespace

extern "C" {

size_t ttt_mlp_backward_workspace_size(const ttt_mlp_desc_t* desc) {
  ttt::Dims dm;
  if (make_dims(desc, &dm)) return 0;
  ok();
  return plan_backward(dm).total;
}

ttt_status_t ttt_mlp_backward_batched(
    const ttt_mlp_desc_t* desc, const void* H, const void* X0, const void* W_gate,
    const void* W_up, const void* W_down0, const float* W_start, const void* conv_taps,
    const void* W_target, const void* dO, const float* dW_final, void* dH, void* dX0,
    float* dW_gate, float* dW_up, float* dW_start, float* dtaps, float* dW_target, float* d_eta,
    void* ws, size_t ws_bytes, void* stream) {
  ttt::Dims dm;
  ttt_status_t st = make_dims(desc, &dm);
  if (st) return st;
  const bool init = desc->init_from_w0 == 1;
  const size_t es = ttt::dtype_bytes(dm.dt), BT = (size_t)(dm.B * dm.T);
  const size_t d = dm.d, f = dm.f, act = BT * d * es, state = (size_t)dm.B * d * f * 4;
  struct P {
    const char* name;
    const void* p;
    bool needed;
    size_t bytes;
    bool out;
  } ptrs[] = {{"H", H, true, act, false},
              {"X0", X0, true, act, false},
              {"W_gate", W_gate, true, f * d * es, false},
              {"W_up", W_up, true, f * d * es, false},
              {"W_down0", W_down0, init, d * f * es, false},
              {"W_start", W_start, !init, state, false},
              {"conv_taps", conv_taps, dm.conv, d * dm.K * es, false},
              {"W_target", W_target, dm.proj, d * d * es, false},
              {"dO", dO, true, act, false},
              {"dW_final", dW_final, false, state, false},
              {"dH", dH, true, act, true},
              {"dX0", dX0, true, act, true},
              {"dW_gate", dW_gate, true, f * d * 4, true},
              {"dW_up", dW_up, true, f * d * 4, true},
              {"dW_start", dW_start, true, state, true},
              {"dtaps", dtaps, dm.conv, d * dm.K * 4, true},
              {"dW_target", dW_target, dm.proj, d * d * 4, true},
              {"d_eta", d_eta, true, 4, true},
              {"ws", ws, true, ws_bytes, true}};
  for (const P& q : ptrs) {
    if (q.needed && !q.p) return fail(TTT_ERR_INVALID_ARGUMENT, "%s is NULL", q.name);
    const size_t a = q.bytes == 4 ? 4 : 16;
    if (q.p && !aligned(q.p, a))
      return fail(TTT_ERR_INVALID_ARGUMENT, "%s is not %zu-byte aligned", q.name, a);
  }
  if (!aligned(ws, 256)) return fail(TTT_ERR_INVALID_ARGUMENT, "ws is not 256-byte aligned");
  // every output (and the workspace) apart from every buffer in use
  for (const P& o : ptrs) {
    if (!o.out || !o.needed) continue;
    for (const P& i : ptrs) {
      if (&i == &o || !i.p || (!i.needed && i.p != dW_final)) continue;
      if (i.out && &i < &o) continue;  // each pair of outputs once
      if (overlaps(range(o.name, o.p, o.bytes), range(i.name, i.p, i.bytes)))
        return fail(TTT_ERR_INVALID_ARGUMENT, "%s overlaps %s", o.name, i.name);
    }
  }
  const BackwardPlan bp = plan_backward(dm);
  if (ws_bytes < bp.total)
    return fail(TTT_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes is below the minimum %zu",
                ws_bytes, bp.total);
  const rocblas_handle h = blas_handle();
  if (!h) return fail(TTT_ERR_HIP, "rocblas_create_handle failed");

  const hipStream_t s = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(ws);
  const ttt::WorkspacePlan& wp = bp.fwd;
  void* Z = base + wp.z_off;
  void* Zt = base + wp.zt_off;
  void* Vt = base + wp.vt_off;
  void* WgU = base + wp.wgu_off;
  void* WtT = base + wp.wtt_off;
  float* tapsT = reinterpret_cast<float*>(base + wp.taps_off);
  char* Wslots = base + wp.slots_off;
  float* Wst = reinterpret_cast<float*>(base + bp.wst);
  void* U = dm.conv ? static_cast<void*>(base + bp.u) : const_cast<void*>(X0);
  void* V = dm.proj ? static_cast<void*>(base + bp.v) : U;
  float* Ag = reinterpret_cast<float*>(base + bp.agu);  // row t at t * 2f
  float* Au = Ag + f;
  void* Ztr = base + bp.ztr;
  void* dOtr = base + bp.dotr;
  char* Sslots = base + bp.sslots;
  float* dZ = reinterpret_cast<float*>(base + bp.dz);
  char* dA = base + bp.da;
  char* Wgu = base + bp.wgu;
  float* Gf = reinterpret_cast<float*>(base + bp.gf);
  void* G = base + bp.g;
  float* dU = reinterpret_cast<float*>(base + bp.du);
  float* tpart = reinterpret_cast<float*>(base + bp.tpart);
  float* dpart = reinterpret_cast<float*>(base + bp.dpart);

  // 1. The forward again: the starting state, U and eta V^ (Vt).
  hipError_t e = init ? ttt::launch_state_reset(Wst, W_down0, dm.dt, dm.B, dm.d, dm.f, s)
                      : hipMemcpyAsync(Wst, W_start, state, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess) e = ttt::launch_weight_prep(dm, W_gate, W_up, W_target, conv_taps, WgU, WtT, tapsT, s);
  if (e == hipSuccess && (dm.Cp != dm.C || dm.T % dm.C != 0)) e = ttt::launch_pad_fill(Zt, Vt, dm, s);
  if (e == hipSuccess) e = ttt::launch_target(dm, X0, tapsT, WtT, dm.conv ? U : Z, Vt, s);
  if (e == hipSuccess) e = hipMemcpyAsync(Wgu, W_gate, f * d * es, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess) e = hipMemcpyAsync(Wgu + f * d * es, W_up, f * d * es, hipMemcpyDeviceToDevice, s);
  if (e != hipSuccess) return hip_fail(e, "backward");

  // 2. The plain GEMMs run in rocBLAS (fp32 accumulation): first the fp32
  //    pre-activations [A_g | A_u] = H [W_gate; W_up]ᵀ in one GEMM (row t
  //    holds both, 2f wide) and V^ = U W_target.
  if (rocblas_set_stream(h, s) != rocblas_status_success ||
      rocblas_set_workspace(h, base + bp.blas, kBlasWorkspace) != rocblas_status_success)
    return fail(TTT_ERR_HIP, "rocblas set-up failed");
  const rocblas_datatype ab = dm.dt == ttt::Dtype::BF16 ? rocblas_datatype_bf16_r : rocblas_datatype_f32_r;
  const rocblas_datatype f32 = rocblas_datatype_f32_r;
  Gemm gemm{h, ab};
  const int64_t B = dm.B, T = dm.T, C = dm.C, N = dm.N, sl = (int64_t)(B * d * f);
  const int64_t Di = (int64_t)d, Fi = (int64_t)f, BTi = (int64_t)BT;
  gemm(false, true, BTi, 2 * Fi, Di, 1.f, H, Di, 0, Wgu, Di, 0, 0.f, Ag, 2 * Fi, 0, 1, f32);
  if (dm.proj)
    gemm(false, false, BTi, Di, Di, 1.f, U, Di, 0, W_target, Di, 0, 0.f, V, Di, 0, 1, ab);
  if (gemm.st != rocblas_status_success) return fail(TTT_ERR_HIP, "rocblas gemm failed (%d)", (int)gemm.st);

  // 3. Z from them, in row-major and in the scans' k-blocked layout (chunks in
  //    order and reversed); dOᵀ k-blocked with the chunks reversed.  Then, in
  //    one launch, the forward's scan (slot j = W^(j-1)) and the same scan
  //    over dOᵀ and Z in reverse chunk order from dW_final (slot j = S_j; its
  //    final state is the gradient of the starting weight).
  e = ttt::launch_swiglu_rows(Ag, Au, 2 * Fi, Z, dm, s);
  if (e == hipSuccess) e = ttt::launch_to_kblocked(Z, Zt, dm, dm.f, false, s);
  if (e == hipSuccess) e = ttt::launch_to_kblocked(Z, Ztr, dm, dm.f, true, s);
  if (e == hipSuccess) e = ttt::launch_to_kblocked(dO, dOtr, dm, dm.d, true, s);
  if (e == hipSuccess)
    e = dW_final ? hipMemcpyAsync(dW_start, dW_final, state, hipMemcpyDeviceToDevice, s)
                 : ttt::launch_fill_f32(dW_start, (int64_t)(state / 4), 0.0f, s);
  ttt::Dims dr = dm;
  dr.reverse_slots = true;  // S_j lands in slot j
  if (e == hipSuccess)
    e = ttt::launch_dual_scan(dm, Vt, Zt, Wst, Wslots, dr, dOtr, Ztr, dW_start, Sslots, s);
  if (e != hipSuccess) return hip_fail(e, "backward");

  // per chunk j: dZ_j = dO_j W^(j-1) + eta V^_j S_j and G_j = Z_j S_jᵀ, with
  // W^(j-1) and S_j in slot j.  The full chunks of a sequence are one batch
  // (rows C apart, slots B*d*f apart); a ragged last chunk is one batch over
  // the sequences.
  const char* Zc = static_cast<const char*>(Z);
  const char* dOc = static_cast<const char*>(dO);
  const char* Vc = static_cast<const char*>(V);
  auto chunk_gemms = [&](int64_t j, int64_t rows, int64_t b0, int64_t count, int64_t row_stride,
                         int64_t slot_stride) {
    const int64_t r = b0 * T + j * C;  // first row
    const char* Wj = Wslots + (size_t)(j * sl + b0 * Di * Fi) * es;
    const char* Sj = Sslots + (size_t)(j * sl + b0 * Di * Fi) * es;
    gemm(false, false, rows, Fi, Di, 1.f, dOc + r * d * es, Di, row_stride * Di, Wj, Fi,
         slot_stride, 0.f, dZ + r * f, Fi, row_stride * Fi, count, f32);
    gemm(false, false, rows, Fi, Di, dm.eta, Vc + r * d * es, Di, row_stride * Di, Sj, Fi,
         slot_stride, 1.f, dZ + r * f, Fi, row_stride * Fi, count, f32);
    gemm(false, true, rows, Di, Fi, 1.f, Zc + r * f * es, Fi, row_stride * Fi, Sj, Fi,
         slot_stride, 0.f, Gf + r * d, Di, row_stride * Di, count, f32);
  };
  const int64_t full = T / C;
  if (full > 0)
    for (int64_t b = 0; b < B; ++b) chunk_gemms(0, C, b, full, C, sl);
  if (full < N) chunk_gemms(full, T - full * C, 0, B, T, Di * Fi);
  if (gemm.st != rocblas_status_success) return fail(TTT_ERR_HIP, "rocblas gemm failed (%d)", (int)gemm.st);
  // 4. eta's gradient sum_t <V^[t], G[t]>; the SwiGLU derivative; dH and the
  //    gated MLP's weight gradients
  e = ttt::launch_dot(V, Gf, BTi * Di, dm.dt, 1.0f, dpart, d_eta, s);
  if (e == hipSuccess) e = ttt::launch_swiglu_backward(dZ, Ag, Au, 2 * Fi, dA, dm, s);
  if (e == hipSuccess && dm.proj) e = ttt::launch_from_f32(Gf, G, BTi * Di, dm.dt, s);
  if (e != hipSuccess) return hip_fail(e, "backward");
  gemm(false, false, BTi, Di, 2 * Fi, 1.f, dA, 2 * Fi, 0, Wgu, Di, 0, 0.f, dH, Di, 0, 1, ab);
  gemm(true, false, Fi, Di, BTi, 1.f, dA, 2 * Fi, 0, H, Di, 0, 0.f, dW_gate, Di, 0, 1, f32);
  gemm(true, false, Fi, Di, BTi, 1.f, dA + f * es, 2 * Fi, 0, H, Di, 0, 0.f, dW_up, Di, 0, 1, f32);
  // 5. the target: dV^ = eta G; dU = dV^ W_targetᵀ, dW_target = Uᵀ dV^; then
  //    the conv's transpose (or dX0 = dU without the conv)
  if (dm.proj) {
    gemm(false, true, BTi, Di, Di, dm.eta, G, Di, 0, W_target, Di, 0, 0.f, dU, Di, 0, 1, f32);
    // split over token slices: slices - 1 of `rows` tokens, the last the rest
    const int64_t S = bp.wt_slices, rows = BTi / S, rest = BTi - (S - 1) * rows;
    float* wtp = reinterpret_cast<float*>(base + bp.wtpart);
    if (S > 1)
      gemm(true, false, Di, Di, rows, dm.eta, U, Di, rows * Di, G, Di, rows * Di, 0.f, wtp, Di,
           Di * Di, S - 1, f32);
    gemm(true, false, Di, Di, rest, dm.eta, static_cast<const char*>(U) + (S - 1) * rows * Di * es,
         Di, 0, static_cast<const char*>(G) + (S - 1) * rows * Di * es, Di, 0, 0.f,
         wtp + (S - 1) * Di * Di, Di, 0, 1, f32);
  }
  if (gemm.st != rocblas_status_success) return fail(TTT_ERR_HIP, "rocblas gemm failed (%d)", (int)gemm.st);
  if (dm.proj) {
    e = ttt::launch_sum_slices(reinterpret_cast<float*>(base + bp.wtpart), dW_target, Di * Di,
                               (int)bp.wt_slices, s);
    if (e != hipSuccess) return hip_fail(e, "backward");
  }
  e = dm.proj ? ttt::launch_target_backward(dU, 1.0f, X0, tapsT, dX0, tpart, dtaps, dm, s)
              : ttt::launch_target_backward(Gf, dm.eta, X0, tapsT, dX0, tpart, dtaps, dm, s);
  if (e != hipSuccess) return hip_fail(e, "backward");
  return ok();
}

}  // extern "C"
