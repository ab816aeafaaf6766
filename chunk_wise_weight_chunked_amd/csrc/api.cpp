// api.cpp -- C ABI of the TTT-MLP layer's forward and streaming calls:
// validation, workspace planning and the launch sequence on the caller's
// stream (the backward's entry points are in backward_api.cpp).  The
// semantics of every entry point are documented in include/ttt_mlp.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/ttt_mlp.h"
#include "api_common.h"
#include "layer.h"

namespace ttt {
namespace api {

thread_local std::string g_err;

ttt_status_t fail(ttt_status_t code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

ttt_status_t ok() {
  g_err.clear();
  return TTT_OK;
}

}  // namespace api
}  // namespace ttt

using namespace ttt::api;

namespace {

// ---------------------------------------------------------------- profiling
const char* const kStageNames[TTT_NUM_STAGES] = {
    "state_reset", "weight_prep", "pad_fill", "swiglu", "target", "prefix_update", "down_proj",
    "scan_apply", "scan_target"};
enum Stage { kReset = 0, kPrep, kPad, kSwiglu, kTarget, kPrefix, kDown, kScanApply, kScanTarget };

struct Profiler {
  std::mutex mu;
  bool enabled = false;
  struct Rec {
    int stage;
    hipEvent_t a, b;
  };
  std::vector<Rec> recs;
  std::vector<hipEvent_t> pool;

  hipEvent_t get() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
};
Profiler g_prof;

// Enqueue one launch, bracketed by events when profiling is on.
template <class F>
hipError_t staged(int stage, hipStream_t s, F&& launch) {
  hipEvent_t a = nullptr, b = nullptr;
  bool prof;
  {
    std::lock_guard<std::mutex> lk(g_prof.mu);
    prof = g_prof.enabled;
    if (prof) {
      a = g_prof.get();
      b = g_prof.get();
    }
  }
  if (prof && a) (void)hipEventRecord(a, s);
  const hipError_t err = launch();
  if (prof && b) (void)hipEventRecord(b, s);
  if (prof) {
    std::lock_guard<std::mutex> lk(g_prof.mu);
    if (a && b)
      g_prof.recs.push_back({stage, a, b});
    else {
      if (a) g_prof.pool.push_back(a);
      if (b) g_prof.pool.push_back(b);
    }
  }
  return err;
}

}  // namespace

// ----------------------------------------------------------------- checking
namespace ttt {
namespace api {

bool overlaps(const Range& x, const Range& y) {
  return x.lo < y.hi && y.lo < x.hi && x.hi > x.lo && y.hi > y.lo;
}

Range range(const char* name, const void* p, size_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{name, lo, lo + bytes};
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr int64_t kMaxInt32 = 2147483647;

ttt_status_t make_dims(const ttt_mlp_desc_t* desc, ttt::Dims* dm) {
  if (!desc) return fail(TTT_ERR_INVALID_ARGUMENT, "desc is NULL");
  const ttt_mlp_desc_t& q = *desc;
  if (q.batch < 1) return fail(TTT_ERR_INVALID_ARGUMENT, "batch must be >= 1 (got %lld)", (long long)q.batch);
  if (q.seq_len < 1) return fail(TTT_ERR_INVALID_ARGUMENT, "seq_len must be >= 1 (got %lld)", (long long)q.seq_len);
  if (q.d_model < 64 || q.d_model % 64)
    return fail(TTT_ERR_UNSUPPORTED, "d_model must be a positive multiple of 64 (got %lld)", (long long)q.d_model);
  if (q.d_ff < 64 || q.d_ff % 64)
    return fail(TTT_ERR_UNSUPPORTED, "d_ff must be a positive multiple of 64 (got %lld)", (long long)q.d_ff);
  if (q.chunk < 1) return fail(TTT_ERR_INVALID_ARGUMENT, "chunk must be >= 1 (got %d)", q.chunk);
  if (q.conv_k < 1) return fail(TTT_ERR_INVALID_ARGUMENT, "conv_k must be >= 1 (got %d)", q.conv_k);
  if (q.conv_k > 8) return fail(TTT_ERR_UNSUPPORTED, "conv_k must be <= 8 (got %d)", q.conv_k);
  if (!std::isfinite(q.eta)) return fail(TTT_ERR_INVALID_ARGUMENT, "eta must be finite");
  if (q.dtype != TTT_F32 && q.dtype != TTT_BF16)
    return fail(TTT_ERR_INVALID_ARGUMENT, "dtype must be TTT_F32 or TTT_BF16 (got %d)", (int)q.dtype);
  if (q.mode != TTT_MODE_AUTO && q.mode != TTT_MODE_SEQUENTIAL && q.mode != TTT_MODE_CHUNK_PARALLEL)
    return fail(TTT_ERR_INVALID_ARGUMENT, "unknown mode %d", (int)q.mode);
  if (q.init_from_w0 != 0 && q.init_from_w0 != 1)
    return fail(TTT_ERR_INVALID_ARGUMENT, "init_from_w0 must be 0 or 1");
  if (q.target < TTT_TARGET_CONV_PROJ || q.target > TTT_TARGET_EMBED)
    return fail(TTT_ERR_INVALID_ARGUMENT, "unknown target %d", (int)q.target);
  if (q.align != TTT_ALIGN_NEXT && q.align != TTT_ALIGN_SELF)
    return fail(TTT_ERR_INVALID_ARGUMENT, "unknown align %d", (int)q.align);
  ttt::Dims d{};
  d.B = q.batch;
  d.T = q.seq_len;
  d.d = q.d_model;
  d.f = q.d_ff;
  d.C = std::min<int64_t>(q.chunk, q.seq_len);  // C >= T is one chunk of T tokens
  d.N = (d.T + d.C - 1) / d.C;
  d.Cp = (d.C + 63) / 64 * 64;
  d.K = q.conv_k;
  d.eta = q.eta;
  d.dt = q.dtype == TTT_BF16 ? ttt::Dtype::BF16 : ttt::Dtype::F32;
  d.conv = q.target == TTT_TARGET_CONV_PROJ || q.target == TTT_TARGET_CONV;
  d.proj = q.target == TTT_TARGET_CONV_PROJ || q.target == TTT_TARGET_PROJ;
  d.shift = q.align == TTT_ALIGN_SELF ? 0 : 1;
  if (d.B > kMaxInt32 / d.T) return fail(TTT_ERR_UNSUPPORTED, "batch * seq_len must be < 2^31");
  if (d.d * d.f > kMaxInt32) return fail(TTT_ERR_UNSUPPORTED, "d_model * d_ff must be < 2^31");
  if (d.B * d.N > kMaxInt32 / d.Cp) return fail(TTT_ERR_UNSUPPORTED, "padded token count must be < 2^31");
  d.P = d.B * d.N * d.Cp;
  // the GEMM tiles address 256 rows of d or f values (up to 4 bytes each)
  // with 32-bit byte offsets from the tile's corner
  if (d.f > (int64_t)1 << 20) return fail(TTT_ERR_UNSUPPORTED, "d_ff must be <= 2^20");
  if (d.d > (int64_t)1 << 20) return fail(TTT_ERR_UNSUPPORTED, "d_model must be <= 2^20");
  *dm = d;
  return TTT_OK;
}

ttt_status_t hip_fail(hipError_t e, const char* what) {
  return fail(TTT_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace api
}  // namespace ttt

namespace {

// Groups the default (AUTO) plan splits a sequence's chunks into: with
// several groups every launch runs one group's scan next to the previous
// group's outputs, and four keep the scan's last partial wave of tiles busy
// while the state is read and written only four times.
constexpr int64_t kAutoGroups = 4;

// The largest group the mode allows (before looking at the workspace).
// Auto mode: four groups, so that each group's scan shares its launch with
// the previous group's outputs -- unless the scan of one group is already
// kAutoOneGroupTiles tiles or more (many sequences: four waves of tiles on
// 256 CUs), where the launches are full anyway and one group reads and
// writes the fp32 states once instead of four times (measured 5.6% faster on
// 16 sequences of 8192 tokens).  A fixed count, so that the workspace a
// descriptor needs does not depend on the device.
constexpr int64_t kAutoOneGroupTiles = 1024;

// Sequential mode takes auto's groups for its slots (the state itself still
// goes through memory after every chunk; see run_layer).
int64_t mode_group(const ttt::Dims& dm, ttt_mode_t mode) {
  if (mode == TTT_MODE_CHUNK_PARALLEL) return dm.N;
  const int64_t scan_tiles = dm.B * ((dm.d + 255) / 256) * ((dm.f + 255) / 256);
  if (scan_tiles >= kAutoOneGroupTiles) return dm.N;
  return (dm.N + kAutoGroups - 1) / kAutoGroups;
}

ttt_status_t plan_group(const ttt::Dims& dm, ttt_mode_t mode, size_t ws_bytes, int64_t* group) {
  const ttt::WorkspacePlan p1 = ttt::plan_workspace(dm, 1);
  if (ws_bytes < p1.total_bytes)
    return fail(TTT_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes is below the minimum %zu",
                ws_bytes, p1.total_bytes);
  const int64_t room = (int64_t)((ws_bytes - p1.fixed_bytes) / p1.slot_bytes);  // slots
  int64_t g = mode_group(dm, mode);
  if (g == dm.N && room < dm.N) g = dm.N - 1;  // one set of N slots does not fit
  if (g < dm.N) g = std::min<int64_t>(g, room / 2);  // two sets of g
  *group = std::max<int64_t>(g, 1);
  return TTT_OK;
}

// Compute units of the current device (cached per device; 256 if the query
// fails).
int64_t compute_units() {
  static std::mutex mu;
  static std::map<int, int64_t> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(dev);
  if (it != cache.end()) return it->second;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  cache[dev] = n;
  return n;
}

// The fast-weight-independent part of the layer: the prepared weights, S2
// (the conv into U, the projection into Vt: token rows [0, t_split) of each
// sequence when t_split < T, the rest left to the first scan launch) and S1
// (Z and Zt), in the workspace regions of `wp`.
ttt_status_t run_activations(const ttt::Dims& dm, const ttt::WorkspacePlan& wp, const void* H,
                             const void* X0, const void* Wg, const void* Wu, const void* taps,
                             const void* Wt, void* ws, int64_t t_split, hipStream_t s) {
  char* base = static_cast<char*>(ws);
  void* Z = base + wp.z_off;
  void* U = base + wp.u_off;
  void* Zt = base + wp.zt_off;
  void* Vt = base + wp.vt_off;
  void* WgU = base + wp.wgu_off;
  void* WtT = base + wp.wtt_off;
  float* tapsT = reinterpret_cast<float*>(base + wp.taps_off);
  hipError_t e = staged(kPrep, s, [&] {
    return ttt::launch_weight_prep(dm, Wg, Wu, Wt, taps, WgU, WtT, tapsT, s);
  });
  if (e != hipSuccess) return hip_fail(e, "weight_prep");
  const bool padded = !ttt::chunk_map_is_identity(dm);
  if (padded) {
    e = staged(kPad, s, [&] { return ttt::launch_pad_fill(Zt, dm.f, Vt, dm.d, dm, s); });
    if (e != hipSuccess) return hip_fail(e, "pad_fill");
  }
  e = staged(kTarget, s, [&] {
    return ttt::launch_target(dm, X0, tapsT, WtT, U, Vt, s, t_split < dm.T ? t_split : -1);
  });
  if (e != hipSuccess) return hip_fail(e, "target");
  e = staged(kSwiglu, s, [&] { return ttt::launch_swiglu(dm, H, WgU, Z, Zt, s); });
  if (e != hipSuccess) return hip_fail(e, "swiglu");
  return TTT_OK;
}

// The whole layer for B sequences whose starting weights are in W_state.
// acts_ready: the workspace already holds S1's and S2's results for these
// inputs (a share's increment call made them), so only the scans and outputs
// run.
ttt_status_t run_layer(const ttt::Dims& dm, ttt_mode_t mode, bool reset, const void* H,
                       const void* X0, const void* Wg, const void* Wu, const void* W0,
                       const void* taps, const void* Wt, void* O, float* W_state, void* ws,
                       size_t ws_bytes, hipStream_t s, bool acts_ready = false) {
  int64_t G = 1;
  ttt_status_t st = plan_group(dm, mode, ws_bytes, &G);
  if (st) return st;
  const ttt::WorkspacePlan wp = ttt::plan_workspace(dm, G);
  char* base = static_cast<char*>(ws);
  void* Z = base + wp.z_off;
  void* U = base + wp.u_off;
  void* Zt = base + wp.zt_off;
  void* Vt = base + wp.vt_off;
  void* WtT = base + wp.wtt_off;
  void* slots = base + wp.slots_off;

  hipError_t e;
  if (reset) {
    e = staged(kReset, s, [&] { return ttt::launch_state_reset(W_state, W0, dm.dt, dm.B, dm.d, dm.f, s); });
    if (e != hipSuccess) return hip_fail(e, "state_reset");
  }
  // S2 (the conv into U, the projection into Vt), then S1.  With a
  // projection and more than one group, S2 may project only the first
  // group's token rows here and the rest next to the first group's scan: when
  // the scan's tiles leave CUs idle (at most two waves of them, a quarter of
  // the CUs or more idle in the last) and are long enough (G·C >= 2 d tokens:
  // twice a projection tile's k-loop) for projection tiles to fit beside them.
  const int64_t groups = (dm.N + G - 1) / G;
  const int64_t scan_tiles = dm.B * (dm.d / 256) * (dm.f / 256);
  const int64_t cus = compute_units();
  const int64_t scan_waves = (scan_tiles + cus - 1) / cus;
  const bool split = !acts_ready && groups > 1 && ttt::scan_target_fits(dm) &&
                     G * dm.C >= 2 * dm.d && scan_waves <= 2 &&
                     scan_waves * cus - scan_tiles >= cus / 4;
  const int64_t t_split = split ? G * dm.C : dm.T;  // 0 < t_split < T when split
  if (!acts_ready) {
    const ttt_status_t st_a = run_activations(dm, wp, H, X0, Wg, Wu, taps, Wt, ws, t_split, s);
    if (st_a) return st_a;
  }
  // Group pipeline: launch g scans group g (slot set g & 1) and computes the
  // outputs of group g - 1 (the other set, completed by launch g - 1).
  // Sequential mode scans one chunk per launch instead -- the fp32 state is
  // read from and written back to W_state for every chunk, as the sequential
  // form of the recurrence has it -- and computes the outputs of group g - 1
  // in the launch of group g's first chunk; with groups of one chunk the two
  // schedules are the same.  Either way each chunk's slot holds the weight
  // its outputs use, and the state's fp32 sums run in the same order.
  const bool per_chunk = mode == TTT_MODE_SEQUENTIAL;
  const size_t set_bytes = (size_t)G * wp.slot_bytes;
  for (int64_t g = 0; g <= groups; ++g) {
    const int64_t g0 = g * G, gc = g < groups ? std::min<int64_t>(G, dm.N - g0) : 0;
    const int64_t a0 = (g - 1) * G, ac = g > 0 ? std::min<int64_t>(G, dm.N - a0) : 0;
    char* scan_slots = static_cast<char*>(slots) + (g & 1) * (wp.slot_sets > 1 ? set_bytes : 0);
    const char* apply_slots =
        static_cast<char*>(slots) + ((g - 1) & 1) * (wp.slot_sets > 1 ? set_bytes : 0);
    if (per_chunk && gc > 1) {
      for (int64_t j = 0; j < gc; ++j) {
        char* sj = scan_slots + j * (size_t)(dm.B * dm.d * dm.f) * ttt::dtype_bytes(dm.dt);
        if (g == 0 && j == 0 && split) {
          e = staged(kScanTarget, s, [&] {
            return ttt::launch_scan_target(dm, Vt, Zt, W_state, sj, 1, dm.conv ? U : X0, WtT,
                                           t_split, s);
          });
          if (e != hipSuccess) return hip_fail(e, "scan_target");
          continue;
        }
        const int64_t jc = j == 0 ? ac : 0;  // outputs of group g - 1 with the first chunk
        e = staged(jc > 0 ? kScanApply : kPrefix, s, [&] {
          return ttt::launch_scan_apply(dm, Vt, Zt, W_state, sj, g0 + j, 1, Z, apply_slots, O, a0,
                                        jc, s);
        });
        if (e != hipSuccess) return hip_fail(e, "scan_apply");
      }
      continue;
    }
    if (g == 0 && split) {
      e = staged(kScanTarget, s, [&] {
        return ttt::launch_scan_target(dm, Vt, Zt, W_state, scan_slots, gc, dm.conv ? U : X0, WtT,
                                       t_split, s);
      });
      if (e != hipSuccess) return hip_fail(e, "scan_target");
      continue;
    }
    const int stage = gc > 0 && ac > 0 ? kScanApply : gc > 0 ? kPrefix : kDown;
    e = staged(stage, s, [&] {
      return ttt::launch_scan_apply(dm, Vt, Zt, W_state, scan_slots, g0, gc, Z, apply_slots, O, a0,
                                    ac, s);
    });
    if (e != hipSuccess) return hip_fail(e, "scan_apply");
  }
  return ok();
}

struct Buffers {
  const void *H, *X0, *Wg, *Wu, *W0, *taps, *Wt;
  void* O;
  float* W;
  void* ws;
  size_t ws_bytes;
};

// Null, alignment and overlap checks of a call's buffers.  need_o = false:
// the call writes no O (b.O is ignored).  `extra` inputs (halo rows) join the
// overlap check against every output.
ttt_status_t check_buffers(const ttt::Dims& dm, const Buffers& b, bool need_w0, bool need_o = true,
                           const std::vector<Range>& extra = {}) {
  struct P {
    const char* name;
    const void* p;
    bool needed;
  } ptrs[] = {{"H", b.H, true},       {"X0", b.X0, true},     {"W_gate", b.Wg, true},
              {"W_up", b.Wu, true},   {"W_down0", b.W0, need_w0}, {"conv_taps", b.taps, dm.conv},
              {"W_target", b.Wt, dm.proj}, {"O", b.O, need_o},   {"W_state", b.W, true},
              {"ws", b.ws, true}};
  for (const P& q : ptrs) {
    if (!q.needed) continue;
    if (!q.p) return fail(TTT_ERR_INVALID_ARGUMENT, "%s is NULL", q.name);
    if (!aligned(q.p, 16)) return fail(TTT_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", q.name);
  }
  if (!aligned(b.ws, 256)) return fail(TTT_ERR_INVALID_ARGUMENT, "ws is not 256-byte aligned");
  const size_t es = ttt::dtype_bytes(dm.dt);
  const size_t act = (size_t)(dm.B * dm.T) * dm.d * es;
  std::vector<Range> ins = {range("H", b.H, act),
                            range("X0", b.X0, act),
                            range("W_gate", b.Wg, (size_t)dm.f * dm.d * es),
                            range("W_up", b.Wu, (size_t)dm.f * dm.d * es)};
  if (dm.conv) ins.push_back(range("conv_taps", b.taps, (size_t)dm.d * dm.K * es));
  if (dm.proj) ins.push_back(range("W_target", b.Wt, (size_t)dm.d * dm.d * es));
  if (need_w0) ins.push_back(range("W_down0", b.W0, (size_t)dm.d * dm.f * es));
  ins.insert(ins.end(), extra.begin(), extra.end());
  const Range outs[] = {range("O", need_o ? b.O : nullptr, need_o ? act : 0),
                        range("W_state", b.W, (size_t)dm.B * dm.d * dm.f * sizeof(float)),
                        range("ws", b.ws, b.ws_bytes)};
  for (const Range& o : outs)
    for (const Range& i : ins)
      if (overlaps(o, i)) return fail(TTT_ERR_INVALID_ARGUMENT, "%s overlaps input %s", o.name, i.name);
  for (int i = 0; i < 3; ++i)
    for (int j = i + 1; j < 3; ++j)
      if (overlaps(outs[i], outs[j]))
        return fail(TTT_ERR_INVALID_ARGUMENT, "%s overlaps %s", outs[i].name, outs[j].name);
  return TTT_OK;
}

}  // namespace

// ---------------------------------------------------------------- streaming
namespace {

// Pending tokens a session carries into a call at stream position pos: the
// tokens of the chunk holding token pos - 1 (its update waits for the next
// token's X0, the look-ahead of the last target).
int64_t pending_tokens(int64_t pos, int64_t C) { return pos == 0 ? 0 : pos - (pos - 1) / C * C; }

// The carry of a stream: per session C rows of H, then kHaloRows + C rows of
// X0 (the halo before the pending chunk, then the chunk); for bf16 then, at a
// 256-byte boundary, the sessions' current weights in bf16 [B][d][f] (read by
// the decode kernels until the next update).
size_t carry_rows_bytes(const ttt::Dims& dm, int64_t C) {
  return (size_t)dm.B * (size_t)(2 * C + ttt::kHaloRows) * dm.d * ttt::dtype_bytes(dm.dt);
}
size_t carry_wcur_offset(const ttt::Dims& dm, int64_t C) {
  return (carry_rows_bytes(dm, C) + 255) & ~(size_t)255;
}
size_t carry_bytes(const ttt::Dims& dm, int64_t C) {
  if (dm.dt != ttt::Dtype::BF16) return carry_rows_bytes(dm, C);
  return carry_wcur_offset(dm, C) + (size_t)dm.B * dm.d * dm.f * 2;
}

// Sessions the decode kernels serve: in a bf16 call of at most 16 new rows
// per session and 64 in all, a session that does not close its stream and
// whose new rows stay in its pending chunk (no update due: the chunk is not
// complete before the call).
constexpr int64_t kDecodeMaxRows = 16, kDecodeMaxTotal = 64;
bool decode_shape(const ttt::Dims& du) {
  return du.dt == ttt::Dtype::BF16 && du.T <= kDecodeMaxRows && du.B * du.T <= kDecodeMaxTotal;
}
bool decode_session(int64_t L, int64_t C, int64_t n_pend, int32_t last) {
  return last == 0 && n_pend + L <= C;
}

// A streaming call's workspace: the layer's workspace for the virtual
// sequences (sized for the longest, L + C rows), then Hv and X0v
// [B][L + C][d], then the carry being built.
struct StreamPlan {
  size_t layer_bytes, hv_off, x0v_off, tmp_off, total;
};

ttt_status_t plan_stream(const ttt_mlp_desc_t* desc, int64_t max_group, size_t ws_bytes,
                         StreamPlan* sp) {
  ttt_mlp_desc_t q = *desc;
  q.seq_len = desc->seq_len + desc->chunk;
  ttt::Dims dmax;
  ttt_status_t st = make_dims(&q, &dmax);
  if (st) return st;
  const size_t es = ttt::dtype_bytes(dmax.dt);
  auto a256 = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t rows = a256((size_t)(dmax.B * dmax.T) * dmax.d * es);
  // bytes after the layer's part (which is a multiple of 256)
  const size_t extra = 2 * rows + carry_rows_bytes(dmax, desc->chunk);
  if (ws_bytes == 0) {  // size for groups of up to max_group chunks
    const int64_t g =
        max_group == 0 ? mode_group(dmax, desc->mode) : std::min<int64_t>(max_group, dmax.N);
    sp->layer_bytes = ttt::plan_workspace(dmax, g).total_bytes;
  } else {  // what a given workspace leaves for the layer
    const size_t minimum = ttt::plan_workspace(dmax, 1).total_bytes + extra;
    if (ws_bytes < minimum)
      return fail(TTT_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes is below the minimum %zu",
                  ws_bytes, minimum);
    sp->layer_bytes = (ws_bytes - extra) / 256 * 256;
  }
  sp->hv_off = sp->layer_bytes;
  sp->x0v_off = sp->hv_off + rows;
  sp->tmp_off = sp->x0v_off + rows;
  sp->total = sp->tmp_off + carry_rows_bytes(dmax, desc->chunk);
  return TTT_OK;
}

}  // namespace

extern "C" {

size_t ttt_mlp_workspace_size(const ttt_mlp_desc_t* desc, int64_t max_group) {
  ttt::Dims dm;
  if (make_dims(desc, &dm)) return 0;
  if (max_group < 0) {
    fail(TTT_ERR_INVALID_ARGUMENT, "max_group must be >= 0");
    return 0;
  }
  const int64_t g = max_group == 0 ? mode_group(dm, desc->mode) : std::min<int64_t>(max_group, dm.N);
  ok();
  return ttt::plan_workspace(dm, g).total_bytes;
}

int64_t ttt_mlp_group_size(const ttt_mlp_desc_t* desc, size_t ws_bytes) {
  ttt::Dims dm;
  ttt_status_t st = make_dims(desc, &dm);
  if (st) return st;
  int64_t g = 0;
  st = plan_group(dm, desc->mode, ws_bytes, &g);
  if (st) return st;
  ok();
  return g;
}

ttt_status_t ttt_mlp_forward(const ttt_mlp_desc_t* desc, const void* H, const void* X0,
                             const void* W_gate, const void* W_up, const void* W_down0,
                             const void* conv_taps, const void* W_target, void* O,
                             float* W_down_final, void* ws, size_t ws_bytes, void* stream) {
  ttt::Dims dm;
  ttt_status_t st = make_dims(desc, &dm);
  if (st) return st;
  if (dm.B != 1) return fail(TTT_ERR_INVALID_ARGUMENT, "ttt_mlp_forward takes one sequence (batch == 1)");
  const Buffers b{H, X0, W_gate, W_up, W_down0, conv_taps, W_target, O, W_down_final, ws, ws_bytes};
  st = check_buffers(dm, b, true);
  if (st) return st;
  int64_t g;
  st = plan_group(dm, desc->mode, ws_bytes, &g);
  if (st) return st;
  return run_layer(dm, desc->mode, true, H, X0, W_gate, W_up, W_down0, conv_taps, W_target, O,
                   W_down_final, ws, ws_bytes, static_cast<hipStream_t>(stream));
}

ttt_status_t ttt_mlp_forward_batched(const ttt_mlp_desc_t* desc, const void* H, const void* X0,
                                     const void* W_gate, const void* W_up, const void* W_down0,
                                     const void* conv_taps, const void* W_target, void* O,
                                     float* W_state, void* ws, size_t ws_bytes, void* stream) {
  ttt::Dims dm;
  ttt_status_t st = make_dims(desc, &dm);
  if (st) return st;
  const bool init = desc->init_from_w0 == 1;
  const Buffers b{H, X0, W_gate, W_up, W_down0, conv_taps, W_target, O, W_state, ws, ws_bytes};
  st = check_buffers(dm, b, init);
  if (st) return st;
  int64_t g;
  st = plan_group(dm, desc->mode, ws_bytes, &g);
  if (st) return st;
  return run_layer(dm, desc->mode, init, H, X0, W_gate, W_up, W_down0, conv_taps, W_target, O,
                   W_state, ws, ws_bytes, static_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace {

// A share's descriptor and halo rows: validates them and sets the conv's
// halo pointers in dm (the left halo is read as the streaming halo of
// kHaloRows rows before each session's first row).
ttt_status_t share_dims(const ttt_mlp_desc_t* desc, const ttt_share_t* share, ttt::Dims* dm,
                        std::vector<Range>* halos) {
  ttt_status_t st = make_dims(desc, dm);
  if (st) return st;
  if (!share) return fail(TTT_ERR_INVALID_ARGUMENT, "share is NULL");
  const size_t row = (size_t)dm->d * ttt::dtype_bytes(dm->dt);
  if (share->X0_left) {
    if (!aligned(share->X0_left, 16))
      return fail(TTT_ERR_INVALID_ARGUMENT, "X0_left is not 16-byte aligned");
    dm->halo = share->X0_left;
    dm->halo_stride = ttt::kHaloRows * dm->d;
    halos->push_back(range("X0_left", share->X0_left, (size_t)dm->B * ttt::kHaloRows * row));
  }
  if (share->X0_right) {
    if (!aligned(share->X0_right, 16))
      return fail(TTT_ERR_INVALID_ARGUMENT, "X0_right is not 16-byte aligned");
    if (dm->T % dm->C != 0)
      return fail(TTT_ERR_INVALID_ARGUMENT,
                  "a share followed by more tokens (X0_right given) must hold whole chunks "
                  "(seq_len %lld, chunk %lld)", (long long)dm->T, (long long)dm->C);
    dm->halo_r = share->X0_right;
    dm->halo_r_stride = dm->d;
    halos->push_back(range("X0_right", share->X0_right, (size_t)dm->B * row));
  }
  return TTT_OK;
}

}  // namespace

extern "C" {

ttt_status_t ttt_mlp_share_increment(const ttt_mlp_desc_t* desc, const ttt_share_t* share,
                                     const void* H, const void* X0, const void* W_gate,
                                     const void* W_up, const void* conv_taps,
                                     const void* W_target, float* S, void* ws, size_t ws_bytes,
                                     void* stream) {
  ttt::Dims dm;
  std::vector<Range> halos;
  ttt_status_t st = share_dims(desc, share, &dm, &halos);
  if (st) return st;
  const Buffers b{H, X0, W_gate, W_up, nullptr, conv_taps, W_target, nullptr, S, ws, ws_bytes};
  st = check_buffers(dm, b, false, false, halos);
  if (st) return st;
  const ttt::WorkspacePlan wp = ttt::plan_workspace(dm, 1);
  if (ws_bytes < wp.total_bytes)
    return fail(TTT_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes is below the minimum %zu",
                ws_bytes, wp.total_bytes);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  st = run_activations(dm, wp, H, X0, W_gate, W_up, conv_taps, W_target, ws, dm.T, s);
  if (st) return st;
  // the scan of every chunk from a zero state, without weight slots: the
  // accumulator ends as the sum of the share's increments
  char* base = static_cast<char*>(ws);
  hipError_t e = ttt::launch_fill_f32(S, dm.B * dm.d * dm.f, 0.0f, s);
  if (e == hipSuccess)
    e = staged(kPrefix, s, [&] {
      return ttt::launch_scan_apply(dm, base + wp.vt_off, base + wp.zt_off, S, nullptr, 0, dm.N,
                                    nullptr, nullptr, nullptr, 0, 0, s);
    });
  if (e != hipSuccess) return hip_fail(e, "share increment");
  return ok();
}

ttt_status_t ttt_mlp_share_forward(const ttt_mlp_desc_t* desc, const ttt_share_t* share,
                                   int32_t reuse, const void* H, const void* X0,
                                   const void* W_gate, const void* W_up, const void* conv_taps,
                                   const void* W_target, void* O, float* W_state, void* ws,
                                   size_t ws_bytes, void* stream) {
  ttt::Dims dm;
  std::vector<Range> halos;
  ttt_status_t st = share_dims(desc, share, &dm, &halos);
  if (st) return st;
  if (reuse != 0 && reuse != 1) return fail(TTT_ERR_INVALID_ARGUMENT, "reuse must be 0 or 1");
  const Buffers b{H, X0, W_gate, W_up, nullptr, conv_taps, W_target, O, W_state, ws, ws_bytes};
  st = check_buffers(dm, b, false, true, halos);
  if (st) return st;
  int64_t g;
  st = plan_group(dm, desc->mode, ws_bytes, &g);
  if (st) return st;
  return run_layer(dm, desc->mode, false, H, X0, W_gate, W_up, nullptr, conv_taps, W_target, O,
                   W_state, ws, ws_bytes, static_cast<hipStream_t>(stream), reuse == 1);
}

size_t ttt_mlp_carry_size(const ttt_mlp_desc_t* desc) {
  ttt::Dims dm;
  if (make_dims(desc, &dm)) return 0;
  ok();
  return carry_bytes(dm, desc->chunk);
}

size_t ttt_mlp_stream_workspace_size(const ttt_mlp_desc_t* desc, int64_t max_group) {
  ttt::Dims dm;
  if (make_dims(desc, &dm)) return 0;
  if (max_group < 0) {
    fail(TTT_ERR_INVALID_ARGUMENT, "max_group must be >= 0");
    return 0;
  }
  StreamPlan sp;
  if (plan_stream(desc, max_group, 0, &sp)) return 0;
  ok();
  return sp.total;
}

}  // extern "C"

namespace {

// Sessions [b0, b0 + nb) of a stream call, all at position `pos`, through the
// full path: the layer over their pending rows and the new ones.  Pointers are
// those of the whole call; the sessions' rows, states and carries are found by
// offset (each session's carry rows are contiguous, and so are the bf16
// weight copies).
ttt_status_t stream_full(const ttt_mlp_desc_t* desc, int64_t b0, int64_t nb, int64_t pos,
                         int32_t last, const void* H, const void* X0, const void* W_gate,
                         const void* W_up, const void* W_down0, const void* conv_taps,
                         const void* W_target, void* O, float* W_state, void* carry, void* ws,
                         size_t ws_bytes, hipStream_t s) {
  ttt::Dims du;
  make_dims(desc, &du);  // validated by the caller
  const int64_t C = desc->chunk, L = du.T, d = du.d, f = du.f;
  const size_t es = ttt::dtype_bytes(du.dt);
  const size_t carry_seq = (size_t)(2 * C + ttt::kHaloRows) * d;  // elements per session
  char* cb = static_cast<char*>(carry);
  char* rows = cb + (size_t)b0 * carry_seq * es;
  char* wcur = cb + carry_wcur_offset(du, C) + (size_t)b0 * d * f * 2;
  H = static_cast<const char*>(H) + (size_t)(b0 * L * d) * es;
  X0 = static_cast<const char*>(X0) + (size_t)(b0 * L * d) * es;
  O = static_cast<char*>(O) + (size_t)(b0 * L * d) * es;
  W_state += b0 * d * f;

  ttt_mlp_desc_t q = *desc;
  q.batch = nb;
  StreamPlan sp;
  ttt_status_t st = plan_stream(&q, 0, ws_bytes, &sp);
  if (st) return st;
  const int64_t n_pend = pending_tokens(pos, C);
  q.seq_len = n_pend + L;
  ttt::Dims dv;
  st = make_dims(&q, &dv);
  if (st) return st;
  char* base = static_cast<char*>(ws);
  if (pos > 0) {
    dv.halo = rows + (size_t)C * d * es;
    dv.halo_stride = (int64_t)carry_seq;
  }
  dv.skip_last = last == 0;
  dv.out_skip = n_pend;
  dv.out_T = L;
  int64_t G;
  st = plan_group(dv, desc->mode, sp.layer_bytes, &G);
  if (st) return st;

  void* Hv = base + sp.hv_off;
  void* X0v = base + sp.x0v_off;
  hipError_t e = ttt::launch_stream_build(dv, H, X0, rows, Hv, X0v, L, n_pend, C, s);
  if (e != hipSuccess) return hip_fail(e, "stream_build");
  const bool init = desc->init_from_w0 == 1 && pos == 0;
  st = run_layer(dv, desc->mode, init, Hv, X0v, W_gate, W_up, W_down0, conv_taps, W_target, O,
                 W_state, ws, sp.layer_bytes, s);
  if (st) return st;
  if (last == 0) {
    const int64_t c_new = (dv.T - 1) / C * C;
    void* tmp = base + sp.tmp_off;
    e = ttt::launch_stream_save(dv, Hv, X0v, pos > 0 ? rows : nullptr, tmp, c_new, C, s);
    if (e != hipSuccess) return hip_fail(e, "stream_save");
    e = hipMemcpyAsync(rows, tmp, carry_rows_bytes(dv, C), hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return hip_fail(e, "carry copy");
    if (dv.dt == ttt::Dtype::BF16) {
      e = ttt::launch_state_to_bf16(W_state, wcur, nb * d * f, s);
      if (e != hipSuccess) return hip_fail(e, "carry weight");
    }
  }
  return TTT_OK;
}

// A stream call with per-session positions and closing flags.  noalloc:
// every session must be one the decode kernels serve, and their gated
// activations go to the library's static scratch instead of ws.
ttt_status_t stream_call(const ttt_mlp_desc_t* desc, const int64_t* pos, const int32_t* last,
                         const void* H, const void* X0, const void* W_gate, const void* W_up,
                         const void* W_down0, const void* conv_taps, const void* W_target,
                         void* O, float* W_state, void* carry, void* ws, size_t ws_bytes,
                         void* stream, bool noalloc = false) {
  ttt::Dims du;  // the call's own L tokens (user buffers)
  ttt_status_t st = make_dims(desc, &du);
  if (st) return st;
  if (!pos || !last) return fail(TTT_ERR_INVALID_ARGUMENT, "pos and last must be non-NULL");
  const int64_t B = du.B;
  if (noalloc) {
    if (!decode_shape(du))
      return fail(TTT_ERR_UNSUPPORTED,
                  "the allocation-free call serves decode calls only: bf16, at most %lld new "
                  "rows per session and %lld in all", (long long)kDecodeMaxRows,
                  (long long)kDecodeMaxTotal);
    for (int64_t b = 0; b < B; ++b)
      if (pos[b] < 0 || last[b] != 0 ||
          !decode_session(du.T, desc->chunk, pending_tokens(pos[b], desc->chunk), 0))
        return fail(TTT_ERR_UNSUPPORTED,
                    "session %lld needs the full path (closing call, or its new rows go past "
                    "its pending chunk): use ttt_mlp_forward_stream_ragged with a workspace",
                    (long long)b);
    if ((size_t)(B * du.T) * du.f * 2 > ttt::kDecodeScratchBytes)
      return fail(TTT_ERR_UNSUPPORTED,
                  "the gated activations of %lld rows of d_ff %lld exceed the %zu-byte scratch",
                  (long long)(B * du.T), (long long)du.f, ttt::kDecodeScratchBytes);
    const hipError_t e = ttt::decode_scratch_ptr(&ws);
    if (e != hipSuccess) return hip_fail(e, "scratch address");
    ws_bytes = ttt::kDecodeScratchBytes;
  }
  bool need_carry = false, need_w0 = false;
  for (int64_t b = 0; b < B; ++b) {
    if (pos[b] < 0)
      return fail(TTT_ERR_INVALID_ARGUMENT, "pos must be >= 0 (got %lld for session %lld)",
                  (long long)pos[b], (long long)b);
    if (last[b] != 0 && last[b] != 1)
      return fail(TTT_ERR_INVALID_ARGUMENT, "last must be 0 or 1 (session %lld)", (long long)b);
    need_carry |= pos[b] > 0 || last[b] == 0;
    need_w0 |= desc->init_from_w0 == 1 && pos[b] == 0;
  }
  if (need_carry && !carry) return fail(TTT_ERR_INVALID_ARGUMENT, "carry is NULL");
  if (need_carry && !aligned(carry, 16))
    return fail(TTT_ERR_INVALID_ARGUMENT, "carry is not 16-byte aligned");
  const Buffers bufs{H, X0, W_gate, W_up, W_down0, conv_taps, W_target, O, W_state, ws, ws_bytes};
  st = check_buffers(du, bufs, need_w0);
  if (st) return st;
  if (need_carry) {
    const size_t act = (size_t)(du.B * du.T) * du.d * ttt::dtype_bytes(du.dt);
    const Range c = range("carry", carry, carry_bytes(du, desc->chunk));
    const Range others[] = {range("H", H, act), range("X0", X0, act), range("O", O, act),
                            range("W_state", W_state, (size_t)du.B * du.d * du.f * sizeof(float)),
                            range("ws", ws, ws_bytes)};
    for (const Range& o : others)
      if (overlaps(c, o)) return fail(TTT_ERR_INVALID_ARGUMENT, "carry overlaps %s", o.name);
  }
  if (!noalloc) {
    StreamPlan sp;
    st = plan_stream(desc, 0, ws_bytes, &sp);  // the whole batch: the largest sub-call fits
    if (st) return st;
  }

  const int64_t C = desc->chunk, L = du.T, d = du.d, f = du.f;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  char* cb = static_cast<char*>(carry);
  std::vector<int64_t> n_pend(B);
  std::vector<char> dec(B, 0);
  uint64_t mask = 0, zero_halo = 0;
  const bool shape = decode_shape(du);
  for (int64_t b = 0; b < B; ++b) {
    n_pend[b] = pending_tokens(pos[b], C);
    dec[b] = shape && decode_session(L, C, n_pend[b], last[b]);
    if (dec[b]) {
      mask |= uint64_t{1} << b;
      if (pos[b] == 0) zero_halo |= uint64_t{1} << b;
    }
  }
  if (mask) {
    // The decode sessions: their new rows' outputs with the current weight;
    // the rows join their pending chunks, whose updates later calls make.
    char* wcur = cb + carry_wcur_offset(du, C);
    hipError_t e = hipSuccess;
    for (int64_t b = 0; b < B && e == hipSuccess; ++b) {
      if (!dec[b] || pos[b] != 0) continue;
      if (desc->init_from_w0 == 1)
        e = ttt::launch_state_reset(W_state + b * d * f, W_down0, du.dt, 1, d, f, s);
      if (e == hipSuccess)
        e = ttt::launch_state_to_bf16(W_state + b * d * f, wcur + (size_t)b * d * f * 2, d * f, s);
    }
    if (e != hipSuccess) return hip_fail(e, "decode state");
    void* Zd = ws;  // [B·L][f]
    e = ttt::launch_decode_swiglu(H, B * L, W_gate, W_up, Zd, d, f, X0, carry, B, L,
                                  n_pend.data(), C, mask, zero_halo, s);
    if (e == hipSuccess) e = ttt::launch_decode_down(Zd, wcur, O, B, L, d, f, mask, s);
    if (e != hipSuccess) return hip_fail(e, "decode");
  }
  // The other sessions through the full path, one call per run of
  // consecutive sessions at the same position and with the same flag.
  for (int64_t b0 = 0; b0 < B;) {
    if (dec[b0]) {
      ++b0;
      continue;
    }
    int64_t b1 = b0 + 1;
    while (b1 < B && !dec[b1] && pos[b1] == pos[b0] && last[b1] == last[b0]) ++b1;
    st = stream_full(desc, b0, b1 - b0, pos[b0], last[b0], H, X0, W_gate, W_up, W_down0,
                     conv_taps, W_target, O, W_state, carry, ws, ws_bytes, s);
    if (st) return st;
    b0 = b1;
  }
  return ok();
}

}  // namespace

extern "C" {

ttt_status_t ttt_mlp_forward_stream(const ttt_mlp_desc_t* desc, int64_t pos, int32_t last,
                                    const void* H, const void* X0, const void* W_gate,
                                    const void* W_up, const void* W_down0, const void* conv_taps,
                                    const void* W_target, void* O, float* W_state, void* carry,
                                    void* ws, size_t ws_bytes, void* stream) {
  ttt::Dims du;
  ttt_status_t st = make_dims(desc, &du);
  if (st) return st;
  const std::vector<int64_t> p(du.B, pos);
  const std::vector<int32_t> l(du.B, last);
  return stream_call(desc, p.data(), l.data(), H, X0, W_gate, W_up, W_down0, conv_taps, W_target,
                     O, W_state, carry, ws, ws_bytes, stream);
}

ttt_status_t ttt_mlp_forward_stream_ragged(const ttt_mlp_desc_t* desc, const int64_t* pos,
                                           const int32_t* last, const void* H, const void* X0,
                                           const void* W_gate, const void* W_up,
                                           const void* W_down0, const void* conv_taps,
                                           const void* W_target, void* O, float* W_state,
                                           void* carry, void* ws, size_t ws_bytes, void* stream) {
  return stream_call(desc, pos, last, H, X0, W_gate, W_up, W_down0, conv_taps, W_target, O,
                     W_state, carry, ws, ws_bytes, stream);
}

ttt_status_t ttt_fastweight_state_reset(float* W_state, const void* W_down0, ttt_dtype_t w0_dtype,
                                        int64_t batch, int64_t d_model, int64_t d_ff,
                                        void* stream) {
  if (!W_state || !W_down0) return fail(TTT_ERR_INVALID_ARGUMENT, "W_state and W_down0 must be non-NULL");
  if (!aligned(W_state, 16) || !aligned(W_down0, 16))
    return fail(TTT_ERR_INVALID_ARGUMENT, "W_state and W_down0 must be 16-byte aligned");
  if (w0_dtype != TTT_F32 && w0_dtype != TTT_BF16)
    return fail(TTT_ERR_INVALID_ARGUMENT, "w0_dtype must be TTT_F32 or TTT_BF16");
  if (batch < 1 || d_model < 1 || d_ff < 1)
    return fail(TTT_ERR_INVALID_ARGUMENT, "batch, d_model and d_ff must be >= 1");
  if (d_model > kMaxInt32 / d_ff) return fail(TTT_ERR_UNSUPPORTED, "d_model * d_ff must be < 2^31");
  const ttt::Dtype dt = w0_dtype == TTT_BF16 ? ttt::Dtype::BF16 : ttt::Dtype::F32;
  const size_t n = (size_t)d_model * d_ff;
  if (overlaps(range("W_state", W_state, n * batch * sizeof(float)),
               range("W_down0", W_down0, n * ttt::dtype_bytes(dt))))
    return fail(TTT_ERR_INVALID_ARGUMENT, "W_state overlaps W_down0");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = staged(kReset, s, [&] {
    return ttt::launch_state_reset(W_state, W_down0, dt, batch, d_model, d_ff, s);
  });
  if (e != hipSuccess) return hip_fail(e, "state_reset");
  return ok();
}

ttt_status_t ttt_mlp_forward_stream_decode_noalloc(
    const ttt_mlp_desc_t* desc, const int64_t* pos, const int32_t* last, const void* H,
    const void* X0, const void* W_gate, const void* W_up, const void* W_down0,
    const void* conv_taps, const void* W_target, void* O, float* W_state, void* carry,
    void* stream) {
  return stream_call(desc, pos, last, H, X0, W_gate, W_up, W_down0, conv_taps, W_target, O,
                     W_state, carry, nullptr, 0, stream, true);
}

const char* ttt_last_error(void) { return g_err.c_str(); }

ttt_status_t ttt_profile_enable(int enable) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  g_prof.enabled = enable != 0;
  return ok();
}

int ttt_profile_read(double* ms_total, int64_t* launches, int max_stages) {
  std::vector<Profiler::Rec> recs;
  {
    std::lock_guard<std::mutex> lk(g_prof.mu);
    recs.swap(g_prof.recs);
  }
  double ms[TTT_NUM_STAGES] = {0};
  int64_t cnt[TTT_NUM_STAGES] = {0};
  hipError_t first_err = hipSuccess;
  for (const auto& r : recs) {
    hipError_t e = hipEventSynchronize(r.b);
    float t = 0.0f;
    if (e == hipSuccess) e = hipEventElapsedTime(&t, r.a, r.b);
    if (e != hipSuccess && first_err == hipSuccess) first_err = e;
    ms[r.stage] += t;
    cnt[r.stage] += 1;
  }
  {
    std::lock_guard<std::mutex> lk(g_prof.mu);
    for (const auto& r : recs) {
      g_prof.pool.push_back(r.a);
      g_prof.pool.push_back(r.b);
    }
  }
  if (first_err != hipSuccess) return hip_fail(first_err, "profile_read");
  for (int i = 0; i < std::min(max_stages, (int)TTT_NUM_STAGES); ++i) {
    if (ms_total) ms_total[i] = ms[i];
    if (launches) launches[i] = cnt[i];
  }
  ok();
  return TTT_NUM_STAGES;
}

const char* ttt_stage_name(int stage) {
  if (stage < 0 || stage >= TTT_NUM_STAGES) return "";
  return kStageNames[stage];
}

}  // extern "C"
