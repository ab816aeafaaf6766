// Kernels of the layer's backward pass that are not plain GEMMs.
//
// The backward follows the chain rule through the forward the In-Place TTT
// page defines (section 3.1 gated MLP, section 3.3 target and update,
// section 3.2 chunk order).  Its chunk-structured part, the sums
// S_j = dW_final + sum_{m > j} dO_mᵀ Z_m, is the forward's streamed prefix
// run over the chunks in reverse order; the kernels here lay the operands out
// for the products (k-blocked token-major), and do the elementwise and
// reduction steps: the conv's transpose and its taps' gradient, and the
// learning rate's gradient.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "gemm_core.h"
#include "layer.h"

namespace ttt {
namespace {

template <typename T>
__device__ __forceinline__ float ld_f32(const T* p);
template <>
__device__ __forceinline__ float ld_f32<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float ld_f32<uint16_t>(const uint16_t* p) {
  return bf16_bits_to_f32(*p);
}

unsigned grid_cap(int64_t n, int64_t per_block, int64_t cap) {
  const int64_t g = (n + per_block - 1) / per_block;
  return (unsigned)std::max<int64_t>(1, std::min<int64_t>(g, cap));
}

// dst = the rows of src ([B][T][R] row-major) in the k-blocked token-major
// layout [P/TB][R][TB] (TB = 128 bytes of tokens: 64 bf16, 32 fp32), with
// zeros in the padding columns.  One TB-token x 64-row tile per workgroup, through LDS;
// global reads and writes are 16 bytes per lane.
template <typename T>
__global__ __launch_bounds__(256) void to_kblocked_kernel(const T* __restrict__ src,
                                                          T* __restrict__ dst, Dims dm,
                                                          int64_t R) {
  constexpr int TB = kRowBytes / (int)sizeof(T);
  constexpr int EPC = 16 / (int)sizeof(T);   // values per 16-byte chunk
  constexpr int IN_CHUNKS = 64 / EPC;         // chunks of a token's 64 rows
  constexpr int OUT_CHUNKS = TB / EPC;        // chunks of a row's TB tokens (8)
  __shared__ __attribute__((aligned(16))) T tile[TB][64 + EPC];  // [token][row], padded
  const int64_t q = blockIdx.x;                 // TB-token block of the layout
  const int64_t r0 = (int64_t)blockIdx.y * 64;  // first row of the tile
  const int64_t tiles_per_chunk = dm.Cp / TB;
  const int64_t chunk = q / tiles_per_chunk, jb = q - chunk * tiles_per_chunk;
  const int64_t b = chunk / dm.N, i = chunk - b * dm.N;
  const int64_t len = std::min<int64_t>(dm.C, dm.T - i * dm.C);  // tokens of chunk i
  for (int it = threadIdx.x; it < TB * IN_CHUNKS; it += 256) {
    const int e = it / IN_CHUNKS, cc = it % IN_CHUNKS;  // token e, chunk cc of its rows
    const int64_t j = jb * TB + e, r = r0 + cc * EPC;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (j < len && r < R)
      v = *reinterpret_cast<const uint4*>(src + (b * dm.T + i * dm.C + j) * R + r);
    *reinterpret_cast<uint4*>(&tile[e][cc * EPC]) = v;
  }
  __syncthreads();
  for (int it = threadIdx.x; it < 64 * OUT_CHUNKS; it += 256) {
    const int rr = it / OUT_CHUNKS, oc = it % OUT_CHUNKS;  // row rr, tokens oc*EPC..
    if (r0 + rr >= R) continue;
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if constexpr (sizeof(T) == 2)
        w[k] = (uint32_t)tile[oc * EPC + 2 * k][rr] | ((uint32_t)tile[oc * EPC + 2 * k + 1][rr] << 16);
      else
        w[k] = __float_as_uint(tile[oc * EPC + k][rr]);
    }
    *reinterpret_cast<uint4*>(dst + (q * R + r0 + rr) * TB + oc * EPC) =
        make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// Four consecutive values of the activation type, as floats.
template <typename T>
__device__ __forceinline__ float4 ld4(const T* p);
template <>
__device__ __forceinline__ float4 ld4<float>(const float* p) {
  return *reinterpret_cast<const float4*>(p);
}
template <>
__device__ __forceinline__ float4 ld4<uint16_t>(const uint16_t* p) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  return make_float4(bf16_bits_to_f32(v.x & 0xffffu), bf16_bits_to_f32(v.x >> 16),
                     bf16_bits_to_f32(v.y & 0xffffu), bf16_bits_to_f32(v.y >> 16));
}
template <typename T>
__device__ __forceinline__ void st4(T* p, float4 v);
template <>
__device__ __forceinline__ void st4<float>(float* p, float4 v) {
  *reinterpret_cast<float4*>(p) = v;
}
template <>
__device__ __forceinline__ void st4<uint16_t>(uint16_t* p, float4 v) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
}
__device__ __forceinline__ float4 fma4(float a, float4 x, float4 y) {
  return make_float4(fmaf(a, x.x, y.x), fmaf(a, x.y, y.y), fmaf(a, x.z, y.z), fmaf(a, x.w, y.w));
}
__device__ __forceinline__ float4 fma4v(float4 a, float4 x, float4 y) {
  return make_float4(fmaf(a.x, x.x, y.x), fmaf(a.y, x.y, y.y), fmaf(a.z, x.z, y.z),
                     fmaf(a.w, x.w, y.w));
}

// The target's backward.  dU[t][c] = scale * src[t][c] (src: fp32, the
// gradient of U, or of V^ = U when there is no projection).  With the conv
// (U[t][c] = sum_k taps[c][k] X0[t + shift - k][c]):
//   dX0[s][c] = sum_k taps[c][k] dU[s - shift + k][c]   (rows of the same sequence)
//   part[r][k][c] = sum over the rows of range r of dU[t][c] X0[t + shift - k][c]
// without it dX0 = dU.  Thread = four consecutive features, walking the rows
// of its token range (blockIdx.y) with the K rows of src and of X0 each row
// needs held in register windows that slide by one row per step (one new row
// of each is read per step); partial tap sums are reduced in a second pass.
template <typename T>
__global__ __launch_bounds__(256) void target_backward_kernel(
    const float* __restrict__ src, float scale, const T* __restrict__ X0,
    const float* __restrict__ tapsT, T* __restrict__ dX0, float* __restrict__ part, Dims dm,
    int64_t rows_per_range) {
  const int64_t c = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (c >= dm.d) return;
  const int64_t d = dm.d, BT = dm.B * dm.T, T_seq = dm.T;
  const int64_t r0 = (int64_t)blockIdx.y * rows_per_range;
  const int64_t r1 = std::min<int64_t>(BT, r0 + rows_per_range);
  const float4 zero = make_float4(0.f, 0.f, 0.f, 0.f);
  if (!dm.conv) {
    for (int64_t t = r0; t < r1; ++t) {
      const float4 du0 = *reinterpret_cast<const float4*>(src + t * d + c);
      st4<T>(dX0 + t * d + c, make_float4(scale * du0.x, scale * du0.y, scale * du0.z,
                                          scale * du0.w));
    }
    return;
  }
  const int K = dm.K, shift = (int)dm.shift;
  float4 tp[8], acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    tp[k] = k < K ? *reinterpret_cast<const float4*>(tapsT + k * d + c) : zero;
    acc[k] = zero;
  }
  // src row s - shift + k of sequence b (zero outside it), and X0 row s + shift - k
  auto src_row = [&](int64_t b, int64_t u) {
    return (u >= 0 && u < T_seq) ? *reinterpret_cast<const float4*>(src + (b * T_seq + u) * d + c)
                                 : zero;
  };
  auto x0_row = [&](int64_t b, int64_t x) {
    return (x >= 0 && x < T_seq) ? ld4<T>(X0 + (b * T_seq + x) * d + c) : zero;
  };
  float4 uwin[8], xwin[8];  // uwin[k] = src row s - shift + k, xwin[k] = X0 row s + shift - k
  int64_t b = r0 / T_seq, s = r0 - b * T_seq;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    uwin[k] = k < K ? src_row(b, s - shift + k) : zero;
    xwin[k] = k < K ? x0_row(b, s + shift - k) : zero;
  }
  for (int64_t t = r0; t < r1; ++t) {
    const float4 du0 = shift < K ? (shift == 0 ? uwin[0] : uwin[1]) : src_row(b, s);
    float4 dx = zero;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (k < K) {
        acc[k] = fma4(scale, fma4v(du0, xwin[k], zero), acc[k]);
        dx = fma4v(tp[k], uwin[k], dx);
      }
    }
    st4<T>(dX0 + t * d + c, make_float4(scale * dx.x, scale * dx.y, scale * dx.z, scale * dx.w));
    // next row: a new sequence restarts both windows, else each slides by one
    if (++s == T_seq) {
      ++b;
      s = 0;
      if (t + 1 < r1) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          uwin[k] = k < K ? src_row(b, s - shift + k) : zero;
          xwin[k] = k < K ? x0_row(b, s + shift - k) : zero;
        }
      }
    } else {
#pragma unroll
      for (int k = 0; k < 7; ++k) uwin[k] = uwin[k + 1];
#pragma unroll
      for (int k = 7; k > 0; --k) xwin[k] = xwin[k - 1];
      const float4 un = src_row(b, s - shift + K - 1), xn = x0_row(b, s + shift);
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (k == K - 1) uwin[k] = un;
      xwin[0] = xn;
    }
  }
#pragma unroll
  for (int k = 0; k < 8; ++k)
    if (k < K) *reinterpret_cast<float4*>(part + ((int64_t)blockIdx.y * 8 + k) * d + c) = acc[k];
}

// dtaps[c][k] = sum over ranges r (in order) of part[r][k][c].
__global__ void taps_reduce_kernel(const float* __restrict__ part, float* __restrict__ dtaps,
                                   int64_t ranges, int64_t d, int K) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= d * K) return;
  const int64_t c = i / K, k = i - c * K;
  float s = 0.f;
  for (int64_t r = 0; r < ranges; ++r) s += part[(r * 8 + k) * d + c];
  dtaps[c * K + k] = s;
}

// Partial sums of sum_i a[i] * b[i] (a: T values, b: fp32), one per
// workgroup; then one workgroup adds the partials in order.
template <typename T>
__global__ __launch_bounds__(256) void dot_partial_kernel(const T* __restrict__ a,
                                                          const float* __restrict__ b, int64_t n,
                                                          float* __restrict__ part) {
  __shared__ float red[256];
  float s = 0.f;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    s = fmaf(ld_f32<T>(a + i), b[i], s);
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) part[blockIdx.x] = red[0];
}

__global__ __launch_bounds__(256) void sum_partials_kernel(const float* __restrict__ part, int n,
                                                           float scale, float* __restrict__ out) {
  __shared__ float red[256];
  float s = 0.f;
  for (int i = threadIdx.x; i < n; i += 256) s += part[i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) *out = scale * red[0];
}

// out[i] = round(in[i]) in the activation type.
template <typename T>
__global__ void from_f32_kernel(const float* __restrict__ in, T* __restrict__ out, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    Elem<T>::store(out + i, in[i]);
}

// out[i] = sum over s (in order) of part[s][i].
__global__ void sum_slices_kernel(const float* __restrict__ part, float* __restrict__ out,
                                  int64_t n, int slices) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    float s = 0.f;
    for (int k = 0; k < slices; ++k) s += part[(int64_t)k * n + i];
    out[i] = s;
  }
}

// out[i] = v.
__global__ void fill_f32_kernel(float* __restrict__ out, int64_t n, float v) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) out[i] = v;
}

}  // namespace

hipError_t launch_to_kblocked(const void* src, void* dst, const Dims& dm, int64_t R,
                              hipStream_t s) {
  const int64_t tb = kRowBytes / (int64_t)dtype_bytes(dm.dt);
  const dim3 grid((unsigned)(dm.P / tb), (unsigned)((R + 63) / 64));
  if (dm.dt == Dtype::BF16)
    hipLaunchKernelGGL(to_kblocked_kernel<uint16_t>, grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(src), static_cast<uint16_t*>(dst), dm, R);
  else
    hipLaunchKernelGGL(to_kblocked_kernel<float>, grid, dim3(256), 0, s,
                       static_cast<const float*>(src), static_cast<float*>(dst), dm, R);
  return hipGetLastError();
}

int64_t target_backward_ranges(const Dims& dm) {
  return (dm.B * dm.T + kTargetBackwardRows - 1) / kTargetBackwardRows;
}

hipError_t launch_target_backward(const float* src, float scale, const void* X0,
                                  const float* tapsT, void* dX0, float* part, float* dtaps,
                                  const Dims& dm, hipStream_t s) {
  const int64_t ranges = target_backward_ranges(dm);
  const dim3 grid((unsigned)((dm.d / 4 + 255) / 256), (unsigned)ranges);
  if (dm.dt == Dtype::BF16)
    hipLaunchKernelGGL(target_backward_kernel<uint16_t>, grid, dim3(256), 0, s, src, scale,
                       static_cast<const uint16_t*>(X0), tapsT, static_cast<uint16_t*>(dX0), part,
                       dm, (int64_t)kTargetBackwardRows);
  else
    hipLaunchKernelGGL(target_backward_kernel<float>, grid, dim3(256), 0, s, src, scale,
                       static_cast<const float*>(X0), tapsT, static_cast<float*>(dX0), part, dm,
                       (int64_t)kTargetBackwardRows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !dm.conv) return e;
  hipLaunchKernelGGL(taps_reduce_kernel, dim3((unsigned)((dm.d * dm.K + 255) / 256)), dim3(256),
                     0, s, part, dtaps, ranges, dm.d, dm.K);
  return hipGetLastError();
}

hipError_t launch_dot(const void* a, const float* b, int64_t n, Dtype dt, float scale, float* part,
                      float* out, hipStream_t s) {
  if (dt == Dtype::BF16)
    hipLaunchKernelGGL(dot_partial_kernel<uint16_t>, dim3(kDotPartials), dim3(256), 0, s,
                       static_cast<const uint16_t*>(a), b, n, part);
  else
    hipLaunchKernelGGL(dot_partial_kernel<float>, dim3(kDotPartials), dim3(256), 0, s,
                       static_cast<const float*>(a), b, n, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sum_partials_kernel, dim3(1), dim3(256), 0, s, part, kDotPartials, scale, out);
  return hipGetLastError();
}

hipError_t launch_from_f32(const float* in, void* out, int64_t n, Dtype dt, hipStream_t s) {
  const dim3 g(grid_cap(n, 256, 65536));
  if (dt == Dtype::BF16)
    hipLaunchKernelGGL(from_f32_kernel<uint16_t>, g, dim3(256), 0, s, in,
                       static_cast<uint16_t*>(out), n);
  else
    hipLaunchKernelGGL(from_f32_kernel<float>, g, dim3(256), 0, s, in, static_cast<float*>(out), n);
  return hipGetLastError();
}

hipError_t launch_sum_slices(const float* part, float* out, int64_t n, int slices,
                             hipStream_t s) {
  hipLaunchKernelGGL(sum_slices_kernel, dim3(grid_cap(n, 256, 16384)), dim3(256), 0, s, part, out,
                     n, slices);
  return hipGetLastError();
}

hipError_t launch_fill_f32(float* out, int64_t n, float v, hipStream_t s) {
  hipLaunchKernelGGL(fill_f32_kernel, dim3(grid_cap(n, 256, 16384)), dim3(256), 0, s, out, n, v);
  return hipGetLastError();
}

}  // namespace ttt
