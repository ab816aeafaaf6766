// backward_api.cpp -- C ABI of the layer's backward pass: validation,
// workspace planning and the launch sequence (the library's own kernels and
// its batched MFMA GEMM) on the caller's stream.  Semantics in
// include/ttt_mlp.h.
#include <hip/hip_runtime.h>

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
  size_t wst, u, v, agu, dot, sslots, da, g, gf, du, tpart, dpart, wtpart, dak,
      hk, uk, gk, wgut, total;
  int64_t wt_slices;  // token slices of the dW_target product (split over K = B*T)
};

BackwardPlan plan_backward(const ttt::Dims& dm) {
  BackwardPlan p;
  p.fwd = ttt::plan_workspace(dm, dm.N, true);
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
  p.dot = take(d * (size_t)dm.P * es);                    // dOᵀ k-blocked
  p.sslots = take((size_t)dm.N * dm.B * d * f * es);      // S_j in slot j
  p.da = take(BT * 2 * f * es);                           // [dA_g | dA_u]
  p.gf = take(BT * d * 4);                                // G = Z_j S_jᵀ (dV^ = eta G), fp32
  p.g = take(dm.proj ? BT * d * es : 0);                  // G rounded: the GEMMs' operand
  p.du = take(dm.proj ? BT * d * 4 : 0);                  // dU (fp32)
  p.tpart = take((size_t)ttt::target_backward_ranges(dm) * 8 * d * 4);
  p.dpart = take((size_t)ttt::kDotPartials * 4);
  // dW_target = Uᵀ dV^ is d x d with K = B*T: one product per slice of about
  // 2048 tokens keeps the GPU busy, the slices are then added in order
  p.wt_slices = dm.proj ? std::max<int64_t>(1, std::min<int64_t>(16, (int64_t)BT / 2048)) : 0;
  p.wtpart = take((size_t)p.wt_slices * d * d * 4);
  // k-blocked token-major copies of the operands of the products over all
  // tokens (dW_gate, dW_up, dW_target), and [W_gate; W_up]ᵀ for dH
  p.dak = take(2 * f * (size_t)dm.P * es);
  p.hk = take(d * (size_t)dm.P * es);
  p.uk = take(dm.proj ? d * (size_t)dm.P * es : 0);
  p.gk = take(dm.proj ? d * (size_t)dm.P * es : 0);
  p.wgut = take(2 * f * d * es);
  p.total = off;
  return p;
}

// The arguments of one product C = alpha A' B'ᵀ (+ C when accumulate) of the
// library's batched GEMM, with each operand's layout (ttt::GemmLayout, see
// layer.h).
ttt::GemmArgs product(ttt::Dtype dt, int32_t la, int32_t lb, int64_t M, int64_t N, int64_t K,
                      float alpha, const void* A, int64_t lda, int64_t sa, const void* B,
                      int64_t ldb, int64_t sb, bool accumulate, void* C, int64_t ldc, int64_t sc,
                      int64_t batch, bool c_f32, int64_t K_last = -1) {
  ttt::GemmArgs g{};
  g.dt = dt;
  g.A = A;
  g.lda = lda;
  g.sa = sa;
  g.a_layout = la;
  g.B = B;
  g.ldb = ldb;
  g.sb = sb;
  g.b_layout = lb;
  g.C = C;
  g.ldc = ldc;
  g.sc = sc;
  g.c_f32 = c_f32 ? 1 : 0;
  g.accumulate = accumulate ? 1 : 0;
  g.M = M;
  g.N = N;
  g.K = K;
  g.K_last = K_last < 0 ? K : K_last;
  g.batch = batch;
  g.alpha = alpha;
  return g;
}

// Launches products on one stream, keeping the first failure.
struct Gemm {
  ttt::Dtype dt;
  hipStream_t s;
  hipError_t err = hipSuccess;
  template <class... A>
  void operator()(A... a) {
    if (err == hipSuccess) err = ttt::launch_gemm(product(dt, a...), s);
  }
};

using ttt::kKBlocked;
using ttt::kTiledKMajor;
using ttt::kTiledRowK;
using ttt::kRowK;

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
  float* Ag = reinterpret_cast<float*>(base + bp.agu);  // row t: [A_g | A_u], 2f wide
  void* dOt = base + bp.dot;
  char* Sslots = base + bp.sslots;
  char* dA = base + bp.da;
  float* Gf = reinterpret_cast<float*>(base + bp.gf);
  void* G = base + bp.g;
  float* dU = reinterpret_cast<float*>(base + bp.du);
  float* tpart = reinterpret_cast<float*>(base + bp.tpart);
  float* dpart = reinterpret_cast<float*>(base + bp.dpart);

  // 1. The forward again: the starting state, U and eta V^ (Vt).
  hipError_t e = init ? ttt::launch_state_reset(Wst, W_down0, dm.dt, dm.B, dm.d, dm.f, s)
                      : hipMemcpyAsync(Wst, W_start, state, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess) e = ttt::launch_weight_prep(dm, W_gate, W_up, W_target, conv_taps, WgU, WtT, tapsT, s);
  if (e == hipSuccess && !ttt::chunk_map_is_identity(dm))
    e = ttt::launch_pad_fill(Zt, dm.f, Vt, dm.d, dm, s);
  // eta V^ token-major into Vt and, with a projection, V^ row-major into V
  if (e == hipSuccess)
    e = ttt::launch_target(dm, X0, tapsT, WtT, dm.conv ? U : Z, Vt, s, -1, dm.proj ? V : nullptr);
  if (e != hipSuccess) return hip_fail(e, "backward");

  // 2. The plain GEMMs (the library's batched MFMA GEMM, fp32 accumulation):
  //    first the fp32 pre-activations [A_g | A_u] = H [W_gate; W_up]ᵀ (row t
  //    holds both, 2f wide) with Z = SiLU(A_g) A_u from the same launch.
  Gemm gemm{dm.dt, s};
  const bool f32 = true, act_f32 = dm.dt == ttt::Dtype::F32;  // output types
  const int64_t B = dm.B, T = dm.T, C = dm.C, N = dm.N, sl = (int64_t)(B * d * f);
  const int64_t Di = (int64_t)d, Fi = (int64_t)f, BTi = (int64_t)BT;
  e = ttt::launch_preact_swiglu(dm.dt, H, WgU, BTi, Di, Fi, Ag, Z, s);
  if (e != hipSuccess) return hip_fail(e, "backward");
  // operands of the later products in the layouts they are read in
  void* Hk = base + bp.hk;
  void* Uk = base + bp.uk;
  void* Gk = base + bp.gk;
  void* WguT = base + bp.wgut;
  e = ttt::launch_to_kblocked(H, Hk, dm, dm.d, s);
  // [W_gate; W_up]ᵀ in TB x TB tiles (dH's B operand): row c holds
  // W_gate[:, c] then W_up[:, c]
  if (e == hipSuccess) e = ttt::launch_transpose(W_gate, WguT, Fi, Di, dm.dt, s, 2 * Fi, 0, true);
  if (e == hipSuccess) e = ttt::launch_transpose(W_up, WguT, Fi, Di, dm.dt, s, 2 * Fi, Fi, true);
  if (e == hipSuccess && dm.proj) e = ttt::launch_to_kblocked(U, Uk, dm, dm.d, s);
  if (e != hipSuccess) return hip_fail(e, "backward");

  // 3. Z and dOᵀ in the scans' k-blocked layout.  Then, in one launch, the
  //    forward's scan (slot j = W^(j-1), written transposed) and the same
  //    scan over dOᵀ and Z walking the chunks last to first from dW_final
  //    (slot j = S_j; its final state is the gradient of the starting
  //    weight).
  e = ttt::launch_to_kblocked(Z, Zt, dm, dm.f, s);
  if (e == hipSuccess) e = ttt::launch_to_kblocked(dO, dOt, dm, dm.d, s);
  if (e == hipSuccess)
    e = dW_final ? hipMemcpyAsync(dW_start, dW_final, state, hipMemcpyDeviceToDevice, s)
                 : ttt::launch_fill_f32(dW_start, (int64_t)(state / 4), 0.0f, s);
  ttt::Dims dr = dm;
  dr.reverse_slots = true;  // S_j lands in slot j
  if (e == hipSuccess)
    e = ttt::launch_dual_scan(dm, Vt, Zt, Wst, Wslots, dr, dOt, Zt, dW_start, Sslots, s);
  if (e != hipSuccess) return hip_fail(e, "backward");

  // per chunk j: dZ_j = dO_j W^(j-1) + eta V^_j S_j (one launch: both
  // products on the same accumulators) with the SwiGLU derivative in its
  // epilogue, which writes dA = [dA_g | dA_u] row-major and k-blocked; and
  // G_j = Z_j S_jᵀ.  W^(j-1) (transposed: K = d contiguous) and S_j (in
  // TB x TB tiles: k-major tiles for dZ, K-contiguous tiles for G) are in
  // slot j.  The full chunks of a sequence are one batch (rows C apart, slots
  // B*d*f apart); a ragged last chunk is one batch over the sequences.
  void* dAk = base + bp.dak;
  if (!ttt::chunk_map_is_identity(dm)) {
    e = ttt::launch_pad_fill(dAk, 2 * Fi, nullptr, 0, dm, s);  // padding token columns of dAk
    if (e != hipSuccess) return hip_fail(e, "backward");
  }
  const char* Zc = static_cast<const char*>(Z);
  const char* dOc = static_cast<const char*>(dO);
  const char* Vc = static_cast<const char*>(V);
  auto chunk_gemms = [&](int64_t j, int64_t rows, int64_t b0, int64_t count, int64_t row_stride,
                         int64_t slot_stride) {
    const int64_t r = b0 * T + j * C;  // first row
    const char* WjT = Wslots + (size_t)(j * sl + b0 * Di * Fi) * es;
    const char* Sj = Sslots + (size_t)(j * sl + b0 * Di * Fi) * es;
    if (gemm.err == hipSuccess)
      gemm.err = ttt::launch_dz_swiglu(
          product(dm.dt, kRowK, kRowK, rows, Fi, Di, 1.f, dOc + r * d * es, Di, row_stride * Di,
                  WjT, Di, slot_stride, false, nullptr, Fi, 0, count, f32),
          product(dm.dt, kRowK, kTiledKMajor, rows, Fi, Di, dm.eta, Vc + r * d * es, Di,
                  row_stride * Di, Sj, Fi, slot_stride, false, nullptr, Fi, 0, count, f32),
          dm, r, row_stride, Ag, dA, dAk, s);
    gemm(kRowK, kTiledRowK, rows, Di, Fi, 1.f, Zc + r * f * es, Fi, row_stride * Fi, Sj, Fi,
         slot_stride, false, Gf + r * d, Di, row_stride * Di, count, f32);
  };
  const int64_t full = T / C;
  if (full > 0)
    for (int64_t b = 0; b < B; ++b) chunk_gemms(0, C, b, full, C, sl);
  if (full < N) chunk_gemms(full, T - full * C, 0, B, T, Di * Fi);
  if (gemm.err != hipSuccess) return hip_fail(gemm.err, "backward gemm");
  // 4. eta's gradient sum_t <V^[t], G[t]>; dH and the gated MLP's weight
  //    gradients
  e = ttt::launch_dot(V, Gf, BTi * Di, dm.dt, 1.0f, dpart, d_eta, s);
  if (e == hipSuccess && dm.proj) e = ttt::launch_from_f32(Gf, G, BTi * Di, dm.dt, s);
  if (e == hipSuccess && dm.proj) e = ttt::launch_to_kblocked(G, Gk, dm, dm.d, s);
  if (e != hipSuccess) return hip_fail(e, "backward");
  const int64_t tb = 128 / (int64_t)es, P = dm.P;  // tokens per 128-byte block row
  gemm(kRowK, kTiledRowK, BTi, Di, 2 * Fi, 1.f, dA, 2 * Fi, 0, WguT, 2 * Fi, 0, false, dH, Di, 0, 1,
       act_f32);
  // dW_gate and dW_up (dA_gᵀ H, dA_uᵀ H over every token column) as one
  // launch of two products: the second's A starts f rows into each block and
  // its C is the other output buffer (element distance as the batch stride)
  const int64_t gu = (int64_t)(reinterpret_cast<intptr_t>(dW_up) -
                               reinterpret_cast<intptr_t>(dW_gate)) / (int64_t)sizeof(float);
  gemm(kKBlocked, kKBlocked, Fi, Di, P, 1.f, dAk, 2 * Fi, Fi * tb, Hk, Di, 0, false, dW_gate, Di,
       gu, 2, f32);
  // 5. the target: dV^ = eta G; dU = dV^ W_targetᵀ, dW_target = Uᵀ dV^; then
  //    the conv's transpose (or dX0 = dU without the conv)
  int64_t slices = 0;
  if (dm.proj) {
    gemm(kRowK, kRowK, BTi, Di, Di, dm.eta, G, Di, 0, W_target, Di, 0, false, dU, Di, 0, 1, f32);
    // split over token slices of whole 64-token blocks, summed in order below
    const int64_t nb = P / tb, per = (nb + bp.wt_slices - 1) / bp.wt_slices;
    slices = (nb + per - 1) / per;
    float* wtp = reinterpret_cast<float*>(base + bp.wtpart);
    gemm(kKBlocked, kKBlocked, Di, Di, per * tb, dm.eta, Uk, Di, per * Di * tb, Gk, Di,
         per * Di * tb, false, wtp, Di, Di * Di, slices, f32, (nb - (slices - 1) * per) * tb);
  }
  if (gemm.err != hipSuccess) return hip_fail(gemm.err, "backward gemm");
  if (dm.proj) {
    e = ttt::launch_sum_slices(reinterpret_cast<float*>(base + bp.wtpart), dW_target, Di * Di,
                               (int)slices, s);
    if (e != hipSuccess) return hip_fail(e, "backward");
  }
  e = dm.proj ? ttt::launch_target_backward(dU, 1.0f, X0, tapsT, dX0, tpart, dtaps, dm, s)
              : ttt::launch_target_backward(Gf, dm.eta, X0, tapsT, dX0, tpart, dtaps, dm, s);
  if (e != hipSuccess) return hip_fail(e, "backward");
  return ok();
}

}  // extern "C"
