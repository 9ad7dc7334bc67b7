// RMSNorm row statistics for the decoder layer.
//
// RMSNorm(x) = x * rsqrt(mean(x^2) + eps) * gamma with the statistics in fp32
// ("Chapter 10: the modern LLaMA architecture", section 4; "3.2 Core
// components, one by one", 3.2.1).  gamma is folded into the weights of the
// projection that follows, and the row scale r is applied in that GEMM's
// epilogue, so the norm itself is one HBM pass that writes 4 bytes per row
// (bf16 layers also write the GEMM operand in its 256 x 32 tiled order).
// One wavefront per row, 16-byte loads (eight in flight per lane), shuffle
// reduction.
#include "common.h"
#include "kernels.h"

namespace llk {
namespace {

DEVI float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += shfl_xor(v, m);
  return v;
}

template <typename T>
__global__ __launch_bounds__(256) void rms_rowscale_kernel(const T* __restrict__ x, float* __restrict__ r,
                                                           T* __restrict__ xt, int M, int d, float eps, Upload u) {
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < u.n; i += 256) u.base[(u.idx[i] >> 31) & 1][u.idx[i] & 0x7fffffff] = u.val[i];
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= M) return;
  const T* p = x + (size_t)row * d;
  float acc = 0.f;
#pragma unroll 8
  for (int c = lane * Chunk<T>::N; c < d; c += 64 * Chunk<T>::N) {
    auto v = load_chunk<T>(p + c);
#pragma unroll
    for (int e = 0; e < Chunk<T>::N; ++e) {
      const float f = to_f32(v[e]);
      acc += f * f;
    }
    if constexpr (sizeof(T) == 2) store_chunk<T>(xt + tiled_off(row, c, d), v);  // 8 columns, one tile row
  }
  acc = wave_sum(acc);
  if (lane == 0) r[row] = 1.f / sqrtf(acc / (float)d + eps);
}

// Second norm: statistics of the fp32 residual stream h, plus h * gamma_2
// rounded once to the layer dtype as the next GEMM's operand (the row scale r2
// is applied in that GEMM's epilogue).
template <typename T>
__global__ __launch_bounds__(256) void rms_convert_kernel(const float* __restrict__ h,
                                                          const float* __restrict__ gamma, T* __restrict__ hb,
                                                          float* __restrict__ r, int M, int d, float eps) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= M) return;
  const float* p = h + (size_t)row * d;
  float acc = 0.f;
#pragma unroll 8
  for (int c = lane * 4; c < d; c += 64 * 4) {
    f32x4 v = *reinterpret_cast<const f32x4*>(p + c);
    acc += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
    v *= *reinterpret_cast<const f32x4*>(gamma + c);
    if constexpr (sizeof(T) == 4) {
      *reinterpret_cast<f32x4*>(hb + (size_t)row * d + c) = v;
    } else {
      *reinterpret_cast<bf16x4*>(hb + tiled_off(row, c, d)) =
          bf16x4{from_f32<bf16>(v[0]), from_f32<bf16>(v[1]), from_f32<bf16>(v[2]), from_f32<bf16>(v[3])};
    }
  }
  acc = wave_sum(acc);
  if (lane == 0) r[row] = 1.f / sqrtf(acc / (float)d + eps);
}

// Final RMSNorm of a stack of layers: y = x * rsqrt(mean(x^2) + eps) * gamma
// ("From Transformer to the LLaMA series", sections 3.3 and 8: the norm after
// the last block), x and gamma in the layer dtype, y row-major in the output
// dtype.  One wavefront per row: the statistics pass reads the row from HBM,
// the scaling pass reads it again while it is still in the L2.
template <typename T, typename TO>
__global__ __launch_bounds__(256) void rms_norm_out_kernel(const T* __restrict__ x, const T* __restrict__ gamma,
                                                           TO* __restrict__ y, int M, int d, float eps) {
  constexpr int N = Chunk<T>::N;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= M) return;
  const T* p = x + (size_t)row * d;
  float acc = 0.f;
#pragma unroll 8
  for (int c = lane * N; c < d; c += 64 * N) {
    const auto v = load_chunk<T>(p + c);
#pragma unroll
    for (int e = 0; e < N; ++e) {
      const float f = to_f32(v[e]);
      acc += f * f;
    }
  }
  acc = wave_sum(acc);
  const float r = 1.f / sqrtf(acc / (float)d + eps);
  TO* q = y + (size_t)row * d;
#pragma unroll 4
  for (int c = lane * N; c < d; c += 64 * N) {
    const auto v = load_chunk<T>(p + c);
    const auto g = load_chunk<T>(gamma + c);
    float f[N];
#pragma unroll
    for (int e = 0; e < N; ++e) f[e] = to_f32(v[e]) * r * to_f32(g[e]);
#pragma unroll
    for (int e = 0; e < N; e += 4) {
      if constexpr (sizeof(TO) == 4)
        *reinterpret_cast<f32x4*>(q + c + e) = f32x4{f[e], f[e + 1], f[e + 2], f[e + 3]};
      else
        *reinterpret_cast<bf16x4*>(q + c + e) =
            bf16x4{from_f32<bf16>(f[e]), from_f32<bf16>(f[e + 1]), from_f32<bf16>(f[e + 2]), from_f32<bf16>(f[e + 3])};
    }
  }
}

}  // namespace

hipError_t launch_rms_norm_out(DType t, const void* x, const void* gamma, void* y, DType out_t, int M, int d,
                               float eps, hipStream_t s) {
  const int grid = (M + 3) / 4;
  if (M <= 0 || d % 8 != 0) return hipErrorInvalidValue;
  if (t == DType::BF16) {
    const bf16* xb = reinterpret_cast<const bf16*>(x);
    const bf16* gb = reinterpret_cast<const bf16*>(gamma);
    if (out_t == DType::BF16)
      rms_norm_out_kernel<bf16, bf16><<<grid, 256, 0, s>>>(xb, gb, reinterpret_cast<bf16*>(y), M, d, eps);
    else
      rms_norm_out_kernel<bf16, float><<<grid, 256, 0, s>>>(xb, gb, reinterpret_cast<float*>(y), M, d, eps);
  } else {
    if (out_t != DType::F32) return hipErrorInvalidValue;
    rms_norm_out_kernel<float, float><<<grid, 256, 0, s>>>(reinterpret_cast<const float*>(x),
                                                           reinterpret_cast<const float*>(gamma),
                                                           reinterpret_cast<float*>(y), M, d, eps);
  }
  return hipGetLastError();
}

hipError_t launch_rms_rowscale(DType t, const void* x, float* r, void* xt, int M, int d, float eps,
                               const Upload* up, hipStream_t s) {
  const int grid = (M + 3) / 4;
  Upload u;
  if (up) {
    u = *up;
  } else {
    u.base[0] = u.base[1] = nullptr;
    u.n = 0;
  }
  if (t == DType::BF16) {
    if (!xt || d % kTileCols != 0) return hipErrorInvalidValue;
    rms_rowscale_kernel<bf16><<<grid, 256, 0, s>>>(reinterpret_cast<const bf16*>(x), r, reinterpret_cast<bf16*>(xt),
                                                   M, d, eps, u);
  } else {
    rms_rowscale_kernel<float><<<grid, 256, 0, s>>>(reinterpret_cast<const float*>(x), r, nullptr, M, d, eps, u);
  }
  return hipGetLastError();
}

hipError_t launch_rms_convert(DType t, const float* h, const float* gamma, void* hb, float* r, int M, int d,
                              float eps, hipStream_t s) {
  const int grid = (M + 3) / 4;
  if (t == DType::BF16 && d % kTileCols != 0) return hipErrorInvalidValue;
  if (t == DType::BF16)
    rms_convert_kernel<bf16><<<grid, 256, 0, s>>>(h, gamma, reinterpret_cast<bf16*>(hb), r, M, d, eps);
  else
    rms_convert_kernel<float><<<grid, 256, 0, s>>>(h, gamma, reinterpret_cast<float*>(hb), r, M, d, eps);
  return hipGetLastError();
}

}  // namespace llk
