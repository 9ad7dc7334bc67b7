// Device-side building blocks shared by the gfx950 kernels of the decoder layer:
// element types, 16-byte chunk loads, fp32 <-> bf16 conversion, and MFMA wrappers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define DEVI __device__ __forceinline__

// ---------------------------------------------------------------------------
// scalar conversions (fp32 -> bf16 is round-to-nearest-even on gfx950)
// ---------------------------------------------------------------------------
DEVI float to_f32(float v) { return v; }
DEVI float to_f32(bf16 v) { return static_cast<float>(v); }
template <typename T> DEVI T from_f32(float v);
template <> DEVI float from_f32<float>(float v) { return v; }
template <> DEVI bf16 from_f32<bf16>(float v) { return static_cast<bf16>(v); }

// ---------------------------------------------------------------------------
// 16-byte chunks: 8 bf16 or 4 fp32 elements
// ---------------------------------------------------------------------------
template <typename T> struct Chunk;
template <> struct Chunk<bf16> {
  static constexpr int N = 8;
  typedef bf16x8 vec;
};
template <> struct Chunk<float> {
  static constexpr int N = 4;
  typedef f32x4 vec;
};

template <typename T>
DEVI typename Chunk<T>::vec load_chunk(const T* p) {
  return *reinterpret_cast<const typename Chunk<T>::vec*>(p);
}
template <typename T>
DEVI void store_chunk(T* p, typename Chunk<T>::vec v) {
  *reinterpret_cast<typename Chunk<T>::vec*>(p) = v;
}
template <typename T>
DEVI typename Chunk<T>::vec zero_chunk() {
  typename Chunk<T>::vec z;
  for (int i = 0; i < Chunk<T>::N; ++i) z[i] = from_f32<T>(0.f);
  return z;
}

// ---------------------------------------------------------------------------
// MFMA 16x16: one 16-byte chunk per lane of each operand.
//   A: lane l holds row (l & 15); B: lane l holds column (l & 15); lane group
//   g = l >> 4 supplies k-elements from its chunk.  Any assignment of k to
//   (lane group, element) works as long as A and B use the same one.
//   C/D: lane l holds column (l & 15), rows 4 * (l >> 4) + {0,1,2,3}.
// bf16: one v_mfma_f32_16x16x32_bf16.  fp32: four v_mfma_f32_16x16x4_f32.
// ---------------------------------------------------------------------------
DEVI f32x4 mfma16_chunk(f32x4 c, bf16x8 a, bf16x8 b) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
DEVI f32x4 mfma16_chunk(f32x4 c, f32x4 a, f32x4 b) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
  return c;
}

// ---------------------------------------------------------------------------
// MFMA 32x32: A lane l holds row (l & 31), B lane l holds column (l & 31),
// lane group h = l >> 5 supplies k-elements.  C/D (16 floats): lane l holds
// column (l & 31), rows 8 * (i / 4) + 4 * h + (i % 4) for register i.
// bf16: one v_mfma_f32_32x32x16_bf16 per chunk; fp32: four v_mfma_f32_32x32x2_f32.
// ---------------------------------------------------------------------------
DEVI f32x16 mfma32_chunk(f32x16 c, bf16x8 a, bf16x8 b) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
DEVI f32x16 mfma32_chunk(f32x16 c, f32x4 a, f32x4 b) {
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[0], b[0], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[1], b[1], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[2], b[2], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[3], b[3], c, 0, 0, 0);
  return c;
}

DEVI int lane_id() { return __lane_id(); }

// gfx950 device builtins, wrapped in plain device functions so that kernel
// templates using them still get their host-side launch stubs.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ void wait_all_loads() { __builtin_amdgcn_s_waitcnt(0); }
// Workgroup barrier that orders LDS only: waits for this wave's LDS
// operations, not for its outstanding global loads / LDS DMAs (which
// __syncthreads would drain).  The memory clobber keeps the compiler from
// moving memory accesses across it.
// The LDS wait is the compiler's own s_waitcnt (0xC07F: lgkmcnt 0, vmcnt and
// expcnt at their maxima), so its wait bookkeeping knows those reads are done.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  asm volatile("s_barrier" ::: "memory");
}

// Workgroup barrier with no wait of its own: for callers that have already
// ordered the memory the barrier publishes (the memory clobber keeps the
// compiler from moving memory accesses across it).
__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }

// Wait until at most N vector-memory operations of this wave are outstanding
// (gfx9 s_waitcnt encoding: vmcnt bits [3:0] and [15:14], expcnt and lgkmcnt
// left at their maxima, i.e. not waited on).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Buffer resource (V#) of a raw byte buffer: base address, num_records in
// bytes (loads at offsets past it return zero), gfx9 raw-buffer flags.
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
DEVI i32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return i32x4{(int32_t)(uint32_t)a, (int32_t)(uint32_t)(a >> 32), (int32_t)bytes, 0x00020000};
}
// LDS byte address of a __shared__ object (wave-uniform).
__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p);
}
// Buffer LDS DMA (lane i's 16 bytes at rsrc base + voffset land at lds + 16 i)
// written as inline assembly, to the LDS byte address lds (an SGPR value).
// The compiler then does not know that it writes LDS, so it never makes an
// LDS read wait for it (it cannot always tell slots of a ring apart and would
// otherwise drain every outstanding DMA before each read): the caller orders
// LDS itself, with wait_vmcnt and a barrier between a stage's DMAs and the
// reads of that stage.  The asm sets M0 (the DMA's LDS base).  The compiler
// warns that M0 is a reserved register; nothing else in these kernels uses M0
// (no compiler-generated LDS DMA, GWS, message or indexed-register
// instructions), so no compiler-held M0 value can be disturbed.
__device__ __forceinline__ void buf_dma16_to(i32x4 rsrc, uint32_t lds, int voffset) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(lds), "v"(voffset), "s"(rsrc)
               : "memory", "m0");
}
// LDS DMA from a flat global address (lane i's 16 bytes at g land at lds + 16 i),
// hidden from the compiler in the same way: the caller orders LDS with
// wait_vmcnt and barriers.
__device__ __forceinline__ void glb_dma16_to(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(g) : "memory", "m0");
}
__device__ __forceinline__ void buf_dma16_async(i32x4 rsrc, const void* lds_base, int voffset) {
  buf_dma16_to(rsrc, lds_address(lds_base), voffset);
}
__device__ __forceinline__ bool wave_any(bool p) { return __any(p); }

// Maximum of v over lanes l and l ^ 32 (hl = l >> 5).  v_permlane32_swap
// exchanges the upper 32 lanes of its first operand with the lower 32 lanes of
// its second.  Given the same value as both operands, the compiler takes the
// two results to be equal and keeps only the first, so the maximum would see
// one lane half only; each half is therefore swapped against a zero register:
// lanes 0-31 find lane l + 32's value in the second result of the first swap,
// lanes 32-63 find lane l - 32's in the first result of the second.
DEVI float max_lane_halves(float v, int hl) {
  const unsigned a = __builtin_bit_cast(unsigned, v);
  const auto lo = __builtin_amdgcn_permlane32_swap(a, 0u, false, false);
  const auto hi = __builtin_amdgcn_permlane32_swap(0u, a, false, false);
  return fmaxf(v, __builtin_bit_cast(float, hl ? hi[0] : lo[1]));
}

// Exchange with lane l ^ m within a wave (m < 64).
DEVI float shfl_xor(float v, int m) { return __shfl_xor(v, m, 64); }

template <typename T> DEVI T ceil_div(T a, T b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------------------
// Tiled storage of the bf16 activations the layer's own kernels produce for a
// GEMM: blocks of 256 rows x 32 columns (16 KB, row-major inside), ordered by
// row block, then column block.  One 32-deep K stage of a 256-row tile is then
// one contiguous 16 KB piece, so its LDS DMAs fetch whole cache lines.  K is a
// multiple of 32; storage holds the row count rounded up to 256.  tiled_off
// returns the element offset of (r, k).
//
// Packed bf16 weights use the same 64-byte rows of 32 columns, ordered K block
// first: [K/32][rows][32] (wtiled_off), rows rounded up to 256.  A stage of
// any run of rows is still one contiguous piece (16 KB for 256 rows, 4 KB for
// the 64 rows of a decode workgroup), and all rows of one K block lie side by
// side, so the workgroups of a weight-streaming GEMM, which advance through K
// together, read a narrow window of memory at any time: measured 6-11% faster
// than the row-block-first order for the decode GEMMs, prefill unchanged.
// ---------------------------------------------------------------------------
constexpr int kTileRows = 256, kTileCols = 32, kTileElems = kTileRows * kTileCols;

// bf16 V cache blocks hold V^T ([D][16 keys]) with the keys of a row in the
// order 0-3, 8-11, 4-7, 12-15: each 16-byte half of a row then holds exactly
// the eight keys one lane group feeds to a 32x32x16 MFMA (keys 4h..4h+3 and
// 8+4h..8+4h+3 for lane group h).  Position of key k (0..15) in the row:
DEVI int vperm_pos(int k) { return (k & 3) | ((k & 4) << 1) | ((k & 8) >> 1); }
DEVI size_t tiled_off(int r, int k, int K) {
  return ((size_t)(r >> 8) * (size_t)(K >> 5) + (size_t)(k >> 5)) * kTileElems + (size_t)((r & 255) * 32 + (k & 31));
}
DEVI size_t wtiled_off(int r, int k, int rows) {
  return ((size_t)(k >> 5) * (size_t)rows + (size_t)r) * kTileCols + (size_t)(k & 31);
}
