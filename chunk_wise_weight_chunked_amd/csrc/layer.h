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
struct Dims {
  int64_t B, T, d, f, C, N, Cp, P;
  int32_t K;
  float eta;
  Dtype dt;
};

// Workspace regions (byte offsets from the workspace base, 256-byte aligned).
struct WorkspacePlan {
  size_t z_off, zt_off, vt_off, wgu_off, wtt_off, taps_off, slots_off;
  size_t slot_bytes;   // one chunk slot for all B sequences: B * d * f * es
  size_t fixed_bytes;  // everything except the slots
  int64_t group;       // chunks per group G
  size_t total_bytes;  // fixed_bytes + group * slot_bytes
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
// Conv of X0 into U (scratch of B*T x d elements), then eta * U W_target into Vt.
hipError_t launch_target(const Dims& dm, const void* X0, const void* taps, const void* WtT,
                         void* U, void* Vt, hipStream_t s);
hipError_t launch_prefix_update(const Dims& dm, const void* Vt, const void* Zt, float* W_state,
                                void* slots, int64_t g0, int64_t gc, hipStream_t s);
hipError_t launch_down_proj(const Dims& dm, const void* Z, const void* slots, void* O,
                            int64_t g0, int64_t gc, hipStream_t s);

}  // namespace ttt
