// Small data-movement kernels: weight packing, zero fill, host-argument
// uploads, and copies between contiguous K/V and the paged cache.
#include "common.h"
#include "kernels.h"

namespace llk {
namespace {

// dst row (r * row_mul + row_add), columns [0, cols): src[r][c] * gamma[c],
// computed in fp32 and rounded once to the storage type.  bf16 weights are
// stored K block first over drows rows (wtiled_off); fp32 weights row-major
// with ldd columns.
template <typename T>
__global__ __launch_bounds__(256) void pack_kernel(const T* __restrict__ src, const T* __restrict__ gamma,
                                                   T* __restrict__ dst, int rows, int cols, int ldd, int drows,
                                                   int row_mul, int row_add, int head_pairs) {
  const size_t total = (size_t)rows * cols;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (size_t)gridDim.x * 256) {
    int r = (int)(i / cols);
    const int c = (int)(i % cols);
    float v = to_f32(src[i]);
    if (gamma) v *= to_f32(gamma[c]);
    if (head_pairs > 0) {  // rows w and w + D/2 of a head become adjacent
      const int D = head_pairs, w = r % D, half = D / 2;
      r = r - w + (w < half ? 2 * w : 2 * (w - half) + 1);
    }
    const int dr = r * row_mul + row_add;
    if constexpr (sizeof(T) == 2)
      dst[wtiled_off(dr, c, drows)] = from_f32<T>(v);
    else
      dst[(size_t)dr * ldd + c] = from_f32<T>(v);
  }
}

__global__ __launch_bounds__(256) void fill_kernel(u32x4* __restrict__ p, size_t n16, uint8_t* __restrict__ tail,
                                                   int ntail, uint32_t byte) {
  const uint32_t w = byte * 0x01010101u;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
    p[i] = u32x4{w, w, w, w};
  if (blockIdx.x == 0 && (int)threadIdx.x < ntail) tail[threadIdx.x] = (uint8_t)byte;
}

template <typename T>
__global__ __launch_bounds__(256) void to_f32_kernel(const T* __restrict__ src, float* __restrict__ dst, int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) dst[i] = to_f32(src[i]);
}

__global__ __launch_bounds__(256) void upload_kernel(Upload u) {
  for (int i = threadIdx.x; i < u.n; i += 256) u.base[(u.idx[i] >> 31) & 1][u.idx[i] & 0x7fffffff] = u.val[i];
}

// K pool [blk][G][16][D]; V pool [blk][G][D][16] (V transposed per block;
// bf16 rows hold the keys in vperm_pos order).
template <typename T>
__global__ __launch_bounds__(256) void kv_copy_kernel(CacheView c, int seq, int start, int n, T* __restrict__ k,
                                                      T* __restrict__ v, int to_cache) {
  const int G = c.G, D = c.D;
  const size_t total = (size_t)n * G * D;
  T* kp = reinterpret_cast<T*>(c.k_pool);
  T* vp = reinterpret_cast<T*>(c.v_pool);
  const int32_t* bt = c.block_table + (size_t)seq * c.max_blocks;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (size_t)gridDim.x * 256) {
    const int d = (int)(i % D);
    const int g = (int)((i / D) % G);
    const int t = (int)(i / ((size_t)D * G));
    const int pos = start + t;
    const size_t blk = (size_t)bt[pos >> 4];
    const size_t ko = ((blk * G + g) * 16 + (pos & 15)) * D + d;
    const size_t vo = ((blk * G + g) * D + d) * 16 + (sizeof(T) == 2 ? vperm_pos(pos & 15) : (pos & 15));
    if (to_cache) {
      kp[ko] = k[i];
      vp[vo] = v[i];
    } else {
      k[i] = kp[ko];
      v[i] = vp[vo];
    }
  }
}

int grid_for(size_t n) {
  size_t g = (n + 255) / 256;
  if (g > 65536) g = 65536;
  return g < 1 ? 1 : (int)g;
}

}  // namespace

hipError_t launch_pack(DType t, const void* src, const void* gamma, void* dst, int rows, int cols, int ldd,
                       int drows, int row_mul, int row_add, int head_pairs, hipStream_t s) {
  if (head_pairs < 0 || head_pairs % 2 != 0 || (head_pairs > 0 && rows % head_pairs != 0)) return hipErrorInvalidValue;
  const int grid = grid_for((size_t)rows * cols);
  if (t == DType::BF16)
    pack_kernel<bf16><<<grid, 256, 0, s>>>(reinterpret_cast<const bf16*>(src), reinterpret_cast<const bf16*>(gamma),
                                           reinterpret_cast<bf16*>(dst), rows, cols, ldd, drows, row_mul, row_add,
                                           head_pairs);
  else
    pack_kernel<float><<<grid, 256, 0, s>>>(reinterpret_cast<const float*>(src),
                                            reinterpret_cast<const float*>(gamma), reinterpret_cast<float*>(dst),
                                            rows, cols, ldd, drows, row_mul, row_add, head_pairs);
  return hipGetLastError();
}

hipError_t launch_fill(void* dst, size_t bytes, uint8_t byte, hipStream_t s) {
  const size_t n16 = bytes / 16;
  const int ntail = (int)(bytes % 16);
  fill_kernel<<<grid_for(n16), 256, 0, s>>>(reinterpret_cast<u32x4*>(dst), n16,
                                            reinterpret_cast<uint8_t*>(dst) + n16 * 16, ntail, byte);
  return hipGetLastError();
}

hipError_t launch_zero(void* dst, size_t bytes, hipStream_t s) { return launch_fill(dst, bytes, 0, s); }

hipError_t launch_to_f32(DType t, const void* src, float* dst, int n, hipStream_t s) {
  if (t == DType::BF16)
    to_f32_kernel<bf16><<<grid_for(n), 256, 0, s>>>(reinterpret_cast<const bf16*>(src), dst, n);
  else
    to_f32_kernel<float><<<grid_for(n), 256, 0, s>>>(reinterpret_cast<const float*>(src), dst, n);
  return hipGetLastError();
}

hipError_t launch_upload(const Upload& u, hipStream_t s) {
  if (u.n <= 0) return hipSuccess;
  upload_kernel<<<1, 256, 0, s>>>(u);
  return hipGetLastError();
}

hipError_t copy_to_device(void* dst, const void* src, size_t bytes, hipStream_t s) {
  return hipMemcpyAsync(dst, src, bytes, hipMemcpyHostToDevice, s);
}

hipError_t stream_sync(hipStream_t s) { return hipStreamSynchronize(s); }

hipError_t event_create(void** ev) {
  hipEvent_t e;
  hipError_t r = hipEventCreate(&e);
  *ev = r == hipSuccess ? reinterpret_cast<void*>(e) : nullptr;
  return r;
}
hipError_t event_destroy(void* ev) { return hipEventDestroy(reinterpret_cast<hipEvent_t>(ev)); }
hipError_t event_record(void* ev, hipStream_t s) { return hipEventRecord(reinterpret_cast<hipEvent_t>(ev), s); }
hipError_t event_elapsed_ms(float* ms, void* start, void* stop) {
  hipError_t r = hipEventSynchronize(reinterpret_cast<hipEvent_t>(stop));
  if (r != hipSuccess) return r;
  return hipEventElapsedTime(ms, reinterpret_cast<hipEvent_t>(start), reinterpret_cast<hipEvent_t>(stop));
}

hipError_t launch_kv_copy(DType t, const CacheView& c, int seq, int start, int n, void* k, void* v, bool to_cache,
                          hipStream_t s) {
  const int grid = grid_for((size_t)n * c.G * c.D);
  if (t == DType::BF16)
    kv_copy_kernel<bf16><<<grid, 256, 0, s>>>(c, seq, start, n, reinterpret_cast<bf16*>(k),
                                              reinterpret_cast<bf16*>(v), to_cache ? 1 : 0);
  else
    kv_copy_kernel<float><<<grid, 256, 0, s>>>(c, seq, start, n, reinterpret_cast<float*>(k),
                                               reinterpret_cast<float*>(v), to_cache ? 1 : 0);
  return hipGetLastError();
}

}  // namespace llk
