// Decode kernels of the streaming entry point (bf16).
//
// Between two updates of a session's fast weight, the outputs of new tokens
// need only O = Z W_curᵀ with Z = SiLU(H W_gateᵀ) ⊙ (H W_upᵀ) (In-Place TTT
// page, section 3.1 for the gated MLP, section 3.2 for the rule that every
// token of a chunk uses the weight left by the chunks before it).  With a few
// rows per call both products are skinny: each weight element is used by at
// most a handful of tokens, so the work is bound by reading the weights from
// HBM once.  The kernels here stream the weights with 16-byte loads and do
// the arithmetic on the matrix cores (v_mfma_f32_16x16x32_bf16, which also
// does the reductions over k that a vector GEMV would do by lane shuffles).
//
// Operand layout of one k-step of 64 values, shared by both kernels.  Lane l
// of a wave has r = l % 16 and q = l / 16.  As the A operand it holds row r's
// k values [64 s + 16 q, + 16) (one 32-byte run: two 8-value operands), as the
// B operand token r's values at the same k.  The MFMA pairs A and B values
// by (q, position) only, so this permutation of k is the same for both sides
// and the two MFMAs of a step sum every k of the step exactly once.  Output:
// lane l holds rows 4 q .. 4 q + 3 of token r.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <map>
#include <mutex>

#include "gemm_core.h"
#include "layer.h"

namespace ttt {
namespace {

constexpr int kDecRows = 16;  // weight rows per workgroup (MFMA M)
constexpr int kDecKStep = 64;
// k-steps whose loads are issued together (measured: 4 for the SwiGLU rows,
// 2 for the down-projection; the launch shape moves either by a few percent)
constexpr int kDecUnroll = 4;
constexpr int kDecUnrollDown = 2;

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ uint4 load16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

__device__ __forceinline__ float dec_silu(float x) {
  return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

// The new rows of the sessions in `mask` join their pending chunks in the
// carry: H rows at n_pend[b].., X0 rows after the halo; a session at the start
// of its stream (bit b of zero_halo) gets a zero halo (the rows before its
// sequence).  16-byte items, vpr per row.
struct CarryAppend {
  const uint4* H;
  const uint4* X0;
  uint4* carry;
  int64_t B, L, C, vpr;
  uint64_t mask, zero_halo;
  int32_t n_pend[kDecodeMaxSessions];
  __device__ __forceinline__ int64_t items() const { return B * (2 * L + kHaloRows) * vpr; }
  __device__ void run(int64_t first, int64_t stride) const {
    const int64_t rows = 2 * L + kHaloRows, carry_seq = (2 * C + kHaloRows) * vpr;
    for (int64_t it = first; it < items(); it += stride) {
      const int64_t b = it / (rows * vpr), rr = it % (rows * vpr) / vpr, c = it % vpr;
      if (!((mask >> b) & 1)) continue;
      const int64_t np = n_pend[b];
      uint4* seq = carry + b * carry_seq;
      if (rr < L)
        seq[(np + rr) * vpr + c] = H[(b * L + rr) * vpr + c];
      else if (rr < 2 * L)
        seq[(C + kHaloRows + np + rr - L) * vpr + c] = X0[(b * L + rr - L) * vpr + c];
      else if ((zero_halo >> b) & 1)
        seq[(C + rr - 2 * L) * vpr + c] = make_uint4(0, 0, 0, 0);
    }
  }
};

// Z[m][j] = SiLU(H[m] · W_gate[j]) * (H[m] · W_up[j]) for the M = B·L new rows
// (M <= 16 TG).  Workgroup = 16 features; its WAVES waves take interleaved
// k-steps and their partial sums meet in LDS (fixed order, deterministic).
// Workgroups past the f / 16 feature groups append the rows to the carry.
template <int WAVES, int TG>
__global__ __launch_bounds__(64 * WAVES) void decode_swiglu_kernel(
    const uint16_t* __restrict__ H, int64_t M, const uint16_t* __restrict__ Wg,
    const uint16_t* __restrict__ Wu, uint16_t* __restrict__ Z, int64_t d, int64_t f,
    CarryAppend app) {
  static_assert(TG <= WAVES, "one wave finishes each token group");
  __shared__ floatx4_t red[WAVES][TG][2][64];
  const int64_t groups = f / kDecRows;
  if ((int64_t)blockIdx.x >= groups) {
    app.run(((int64_t)blockIdx.x - groups) * blockDim.x + threadIdx.x,
            ((int64_t)gridDim.x - groups) * blockDim.x);
    return;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, q = lane >> 4;
  const int64_t f0 = (int64_t)blockIdx.x * kDecRows;
  const uint16_t* wg = Wg + (f0 + r) * d + 16 * q;
  const uint16_t* wu = Wu + (f0 + r) * d + 16 * q;
  const uint16_t* h[TG];
  bool hv[TG];
  for (int t = 0; t < TG; ++t) {
    const int64_t m = (int64_t)t * 16 + r;
    hv[t] = m < M;
    h[t] = H + (hv[t] ? m : 0) * d + 16 * q;
  }
  floatx4_t ag[TG], au[TG];
  for (int t = 0; t < TG; ++t) ag[t] = au[t] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  const uint4 zero = make_uint4(0, 0, 0, 0);

  const int64_t nks = d / kDecKStep;
  int64_t s = wave;
  for (; s + (kDecUnroll - 1) * WAVES < nks; s += kDecUnroll * WAVES) {
    uint4 g[kDecUnroll][2], u[kDecUnroll][2];
#pragma unroll
    for (int i = 0; i < kDecUnroll; ++i) {
      const int64_t k = (s + i * WAVES) * kDecKStep;
      g[i][0] = load16(wg + k);
      g[i][1] = load16(wg + k + 8);
      u[i][0] = load16(wu + k);
      u[i][1] = load16(wu + k + 8);
    }
#pragma unroll
    for (int i = 0; i < kDecUnroll; ++i) {
      const int64_t k = (s + i * WAVES) * kDecKStep;
#pragma unroll
      for (int t = 0; t < TG; ++t) {
        const uint4 h0 = hv[t] ? load16(h[t] + k) : zero;
        const uint4 h1 = hv[t] ? load16(h[t] + k + 8) : zero;
        ag[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(g[i][0]), as_bf16x8(h0), ag[t], 0, 0, 0);
        ag[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(g[i][1]), as_bf16x8(h1), ag[t], 0, 0, 0);
        au[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(u[i][0]), as_bf16x8(h0), au[t], 0, 0, 0);
        au[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(u[i][1]), as_bf16x8(h1), au[t], 0, 0, 0);
      }
    }
  }
  for (; s < nks; s += WAVES) {
    const int64_t k = s * kDecKStep;
    const uint4 g0 = load16(wg + k), g1 = load16(wg + k + 8);
    const uint4 u0 = load16(wu + k), u1 = load16(wu + k + 8);
#pragma unroll
    for (int t = 0; t < TG; ++t) {
      const uint4 h0 = hv[t] ? load16(h[t] + k) : zero;
      const uint4 h1 = hv[t] ? load16(h[t] + k + 8) : zero;
      ag[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(g0), as_bf16x8(h0), ag[t], 0, 0, 0);
      ag[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(g1), as_bf16x8(h1), ag[t], 0, 0, 0);
      au[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(u0), as_bf16x8(h0), au[t], 0, 0, 0);
      au[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(u1), as_bf16x8(h1), au[t], 0, 0, 0);
    }
  }

  for (int t = 0; t < TG; ++t) {
    red[wave][t][0][lane] = ag[t];
    red[wave][t][1][lane] = au[t];
  }
  __syncthreads();
  if (wave >= TG) return;
  const int t = wave;
  const int64_t m = (int64_t)t * 16 + r;
  if (m >= M) return;
  floatx4_t gs = red[0][t][0][lane], us = red[0][t][1][lane];
  for (int w = 1; w < WAVES; ++w) {
    gs += red[w][t][0][lane];
    us += red[w][t][1][lane];
  }
  uint2 out;
  out.x = pack_bf16x2(dec_silu(gs[0]) * us[0], dec_silu(gs[1]) * us[1]);
  out.y = pack_bf16x2(dec_silu(gs[2]) * us[2], dec_silu(gs[3]) * us[3]);
  *reinterpret_cast<uint2*>(Z + m * f + f0 + 4 * q) = out;
}

// O[b][t][c] = Z[b][t] · W_cur[b][c] for the L <= 16 new rows of each session
// b in `mask`.  Workgroup = 16 output channels of one session; WAVES waves
// split k = f.
template <int WAVES>
__global__ __launch_bounds__(64 * WAVES) void decode_down_kernel(
    const uint16_t* __restrict__ Z, const uint16_t* __restrict__ Wc, uint16_t* __restrict__ O,
    int64_t L, int64_t d, int64_t f, uint64_t mask) {
  __shared__ floatx4_t red[WAVES][64];
  const int64_t b = blockIdx.y;
  if (!((mask >> b) & 1)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, q = lane >> 4;
  const int64_t c0 = (int64_t)blockIdx.x * kDecRows;
  const uint16_t* w = Wc + (b * d + c0 + r) * f + 16 * q;
  const bool zv = r < L;
  const uint16_t* z = Z + (b * L + (zv ? r : 0)) * f + 16 * q;
  floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
  const uint4 zero = make_uint4(0, 0, 0, 0);

  const int64_t nks = f / kDecKStep;
  int64_t s = wave;
  for (; s + (kDecUnrollDown - 1) * WAVES < nks; s += kDecUnrollDown * WAVES) {
    uint4 a[kDecUnrollDown][2], x[kDecUnrollDown][2];
#pragma unroll
    for (int i = 0; i < kDecUnrollDown; ++i) {
      const int64_t k = (s + i * WAVES) * kDecKStep;
      a[i][0] = load16(w + k);
      a[i][1] = load16(w + k + 8);
      x[i][0] = zv ? load16(z + k) : zero;
      x[i][1] = zv ? load16(z + k + 8) : zero;
    }
#pragma unroll
    for (int i = 0; i < kDecUnrollDown; ++i) {
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[i][0]), as_bf16x8(x[i][0]), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[i][1]), as_bf16x8(x[i][1]), acc, 0, 0, 0);
    }
  }
  for (; s < nks; s += WAVES) {
    const int64_t k = s * kDecKStep;
    const uint4 a0 = load16(w + k), a1 = load16(w + k + 8);
    const uint4 x0 = zv ? load16(z + k) : zero, x1 = zv ? load16(z + k + 8) : zero;
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a0), as_bf16x8(x0), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a1), as_bf16x8(x1), acc, 0, 0, 0);
  }

  red[wave][lane] = acc;
  __syncthreads();
  if (wave != 0 || !zv) return;
  floatx4_t sum = red[0][lane];
  for (int v = 1; v < WAVES; ++v) sum += red[v][lane];
  uint2 out;
  out.x = pack_bf16x2(sum[0], sum[1]);
  out.y = pack_bf16x2(sum[2], sum[3]);
  *reinterpret_cast<uint2*>(O + (b * L + r) * d + c0 + 4 * q) = out;
}

// bf16 copy of the fp32 state, round to nearest even (the same rounding as
// the weight slots of the chunk pipeline).  8 values per item.
__global__ void state_to_bf16_kernel(const float* __restrict__ W, uint16_t* __restrict__ out,
                                     int64_t n8) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += stride) {
    const float4 a = reinterpret_cast<const float4*>(W)[2 * i];
    const float4 c = reinterpret_cast<const float4*>(W)[2 * i + 1];
    uint4 v;
    v.x = pack_bf16x2(a.x, a.y);
    v.y = pack_bf16x2(a.z, a.w);
    v.z = pack_bf16x2(c.x, c.y);
    v.w = pack_bf16x2(c.z, c.w);
    reinterpret_cast<uint4*>(out)[i] = v;
  }
}

unsigned grid_cap(int64_t n, int64_t per_block, int64_t cap) {
  const int64_t g = (n + per_block - 1) / per_block;
  return (unsigned)std::max<int64_t>(1, std::min<int64_t>(g, cap));
}

}  // namespace

hipError_t launch_decode_swiglu(const void* H, int64_t M, const void* Wg, const void* Wu, void* Z,
                                int64_t d, int64_t f, const void* X0, void* carry, int64_t B,
                                int64_t L, const int64_t* n_pend, int64_t C, uint64_t mask,
                                uint64_t zero_halo, hipStream_t s) {
  if (B > kDecodeMaxSessions) return hipErrorInvalidValue;
  CarryAppend app;
  app.H = static_cast<const uint4*>(H);
  app.X0 = static_cast<const uint4*>(X0);
  app.carry = static_cast<uint4*>(carry);
  app.B = B;
  app.L = L;
  app.C = C;
  app.vpr = d * 2 / 16;
  app.mask = mask;
  app.zero_halo = zero_halo;
  for (int64_t b = 0; b < kDecodeMaxSessions; ++b) app.n_pend[b] = b < B ? (int32_t)n_pend[b] : 0;
  const int64_t items = B * (2 * L + kHaloRows) * app.vpr;
  const dim3 grid((unsigned)(f / kDecRows + grid_cap(items, 512, 64)));
  const auto h = static_cast<const uint16_t*>(H);
  const auto g = static_cast<const uint16_t*>(Wg);
  const auto u = static_cast<const uint16_t*>(Wu);
  const auto z = static_cast<uint16_t*>(Z);
  if (M <= 16)
    hipLaunchKernelGGL((decode_swiglu_kernel<8, 1>), grid, dim3(512), 0, s, h, M, g, u, z, d, f, app);
  else if (M <= 32)
    hipLaunchKernelGGL((decode_swiglu_kernel<8, 2>), grid, dim3(512), 0, s, h, M, g, u, z, d, f, app);
  else
    hipLaunchKernelGGL((decode_swiglu_kernel<8, 4>), grid, dim3(512), 0, s, h, M, g, u, z, d, f, app);
  return hipGetLastError();
}

hipError_t launch_decode_down(const void* Z, const void* Wc, void* O, int64_t B, int64_t L,
                              int64_t d, int64_t f, uint64_t mask, hipStream_t s) {
  if (B > kDecodeMaxSessions) return hipErrorInvalidValue;
  hipLaunchKernelGGL((decode_down_kernel<8>), dim3((unsigned)(d / kDecRows), (unsigned)B),
                     dim3(512), 0, s, static_cast<const uint16_t*>(Z),
                     static_cast<const uint16_t*>(Wc), static_cast<uint16_t*>(O), L, d, f, mask);
  return hipGetLastError();
}

hipError_t launch_state_to_bf16(const float* W, void* out, int64_t n, hipStream_t s) {
  const int64_t n8 = n / 8;
  hipLaunchKernelGGL(state_to_bf16_kernel, dim3(grid_cap(n8, 256, 16384)), dim3(256), 0, s, W,
                     static_cast<uint16_t*>(out), n8);
  return hipGetLastError();
}

// ------------------------------------------------- allocation-free scratch
// The gated activations of a decode call for callers that cannot allocate: a
// file-scope device array (each GPU holds its own copy until the process
// ends).  Host code never passes the array's name to a kernel or a copy (on
// the host it is only a stand-in for the device symbol): it takes the
// device's address of it once per device and hands that out.
static __device__ __align__(256) char scratch[kDecodeScratchBytes];

hipError_t decode_scratch_ptr(void** out) {
  static std::mutex mu;
  static std::map<int, void*> by_device;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  auto it = by_device.find(dev);
  if (it == by_device.end()) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    it = by_device.emplace(dev, ptr).first;
  }
  *out = it->second;
  return hipSuccess;
}

}  // namespace ttt
