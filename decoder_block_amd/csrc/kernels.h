// Internal launch interface between the host runtime (llama_layer.cpp) and the
// gfx950 kernels.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace llk {

enum class DType : int { F32 = 0, BF16 = 1 };

inline size_t dsize(DType t) { return t == DType::F32 ? 4 : 2; }

// Per-call description of the batch, resident in device memory:
// desc[2*b] = seq_id, desc[2*b+1] = first new position of sequence b.
struct BatchView {
  const int32_t* desc;
  int batch;
  int seq_len;  // new tokens per sequence (1 for decode)
};

// Paged KV cache as the kernels see it.  K and V pools are
// [num_blocks][G][16][D]; the block table is [max_seqs][max_blocks].
struct CacheView {
  void* k_pool;
  void* v_pool;
  const int32_t* block_table;
  int max_blocks;
  int G, D;
};

enum class Epi : int { QKV = 0, RESID_H = 1, SWIGLU = 2, RESID_OUT = 3 };

// bf16 activations are stored in 256 x 32 tiles (tiled_off in common.h) with M
// rounded up to 256 rows; bf16 packed weights K block first (wtiled_off) with
// N rounded up to 256 rows (w_rows).  fp32 operands are row-major.
struct GemmArgs {
  const void* W;  // packed weights [N][K] (features x K): bf16 K-block-major (wtiled_off), fp32 row-major
  int w_rows;     // bf16 W: its padded row count, so K block kb starts at byte kb * w_rows * 64
  const void* X;  // activations [M][K]: bf16 tiled; fp32 row-major with pitch ldx
  int M, N, K, ldx;
  Epi epi;
  const float* rowscale;  // QKV / SWIGLU: per-token RMSNorm scale
  // QKV epilogue
  void* q_out;  // [M][H*D]
  CacheView cache;
  BatchView batch;
  const float* rope_cos;  // [max_position][D/2]
  const float* rope_sin;
  int rope_half;  // 1: the packed q/k rows of a head are ordered 0, D/2, 1, D/2+1, ... (half-split RoPE)
  int H;
  // residual / output epilogues
  const void* resid;  // RESID_H: x [M][N] (layer dtype); RESID_OUT: h [M][N] fp32
  void* out;          // RESID_H: h fp32; SWIGLU: s [M][ldo] (bf16 tiled); RESID_OUT: out
  int ldo;
  DType out_dtype;    // RESID_OUT only
  // SKINNY tiles split K over workgroups; their fp32 partial sums [ks][M][N]
  // go here (skinny_partial_bytes) before one pass adds them and runs the epilogue
  float* split_ws;
  size_t split_ws_bytes;
  // RMSNorm_2 folded into a split RESID_H pass (bf16 SKINNY, norm_gamma set):
  // that pass also writes h * gamma as bf16 tiled [M][N] to norm_out and the
  // row's sums of h^2 over 1024-feature segments to ss_part [M][ss_nseg]
  const float* norm_gamma;
  void* norm_out;
  // QKV / SWIGLU: with ss_part set, the row scale is rsqrt(sum of the row's
  // ss_nseg partial sums / ss_d + eps) instead of rowscale[t]
  float* ss_part;
  int ss_nseg, ss_d;
  float eps;
};

// Tile shape chosen by the host for a GEMM.  SKINNY (bf16, M <= 128) is the
// weight-streaming shape of decode: 64 x 64 tiles with K split across
// workgroups so that even N = hidden size fills the chip.
enum class GemmTile : int { LARGE = 0, SMALL = 1, SKINNY = 2 };
int gemm_tile_n(GemmTile t);  // features per workgroup tile
// workgroups a SKINNY GEMM splits K into, and the partial-sum bytes it needs
int skinny_ksplit(int M, int N, int K);
size_t skinny_partial_bytes(int M, int N, int K);
// feature segments of the folded RMSNorm_2 partial sums (one per 1024 features)
constexpr int kNormSeg = 1024;

hipError_t launch_gemm(DType t, GemmTile tile, const GemmArgs& a, hipStream_t s);

// RMSNorm row scale r[t] = rsqrt(mean(x[t]^2) + eps) of x [M][d] (layer dtype),
// plus (bf16, xt non-null) a tiled copy of x as the QKV GEMM operand.
struct Upload;
// `up` (may be null) is a batch of int32 stores applied by the same launch
// before any later kernel on the stream runs (host bookkeeping of the step).
hipError_t launch_rms_rowscale(DType t, const void* x, float* r, void* xt, int M, int d, float eps,
                               const Upload* up, hipStream_t s);
// Second norm: r2[t] from h [M][d] fp32, plus hb = h * gamma (fp32 gamma) rounded
// once to the layer dtype (bf16: tiled).
hipError_t launch_rms_convert(DType t, const float* h, const float* gamma, void* hb, float* r,
                              int M, int d, float eps, hipStream_t s);

// Final RMSNorm of a layer stack: y [M][d] (out_t, row-major) = x * rsqrt(mean(x^2)
// + eps) * gamma, x [M][d] and gamma [d] in the layer dtype t.
hipError_t launch_rms_norm_out(DType t, const void* x, const void* gamma, void* y, DType out_t, int M, int d,
                               float eps, hipStream_t s);

// Causal GQA prefill attention: q [B*S][H*D] -> attn [B*S][H*D] (bf16 tiled),
// keys from the cache.
hipError_t launch_attn_prefill(DType t, const void* q, void* attn, int H, const CacheView& c,
                               const BatchView& b, hipStream_t s);

// Split-K paged decode attention.  partial: [B][H][max_splits][D + 2] fp32
// holding (running max, sum, unnormalised output) per key chunk; the combine
// kernel merges the chunks into attn [B][H*D] (bf16 tiled).  units: the
// number of (sequence, chunk) work units, sum over b of
// ceil(kv_len_b / decode_split_keys()) with kv_len_b the length including
// the new token (the host knows the lengths; the kernel derives each
// workgroup's unit from the batch descriptor).
int decode_split_keys();
hipError_t launch_attn_decode(DType t, const void* q, float* partial, int max_splits, int H,
                              const CacheView& c, const BatchView& b, int units, hipStream_t s);
hipError_t launch_attn_decode_combine(DType t, const float* partial, void* attn, int max_splits,
                                      int H, int D, const BatchView& b, hipStream_t s);

// Weight packing.  dst[r][c] = src[r][c] * (gamma ? gamma[c] : 1) for r < rows,
// c < cols (bf16: K-block-major over drows destination rows, wtiled_off; fp32:
// row-major with ldd columns); the caller zeroes
// the buffer first, so padded rows and columns stay zero.  Row r of the source
// lands at dst row (r' * row_mul + row_add), where r' = r, or with head_pairs
// = D > 0 the rows of each D-row head reordered so that rows w and w + D/2
// become adjacent: w < D/2 -> 2w, w >= D/2 -> 2(w - D/2) + 1.
hipError_t launch_pack(DType t, const void* src, const void* gamma, void* dst, int rows,
                       int cols, int ldd, int drows, int row_mul, int row_add, int head_pairs, hipStream_t s);
hipError_t launch_zero(void* dst, size_t bytes, hipStream_t s);
// Every byte of dst[0, bytes) set to `byte`.
hipError_t launch_fill(void* dst, size_t bytes, uint8_t byte, hipStream_t s);
// dst[i] = float(src[i]) for n elements of the layer dtype.
hipError_t launch_to_f32(DType t, const void* src, float* dst, int n, hipStream_t s);

// Small host -> device updates carried in kernel arguments: base[idx[i]] = val[i].
constexpr int kUploadMax = 240;
struct Upload {
  int32_t* base[2];  // entry i stores val[i] at base[idx[i] >> 31][idx[i] & 0x7fffffff]
  int n;
  int32_t idx[kUploadMax];
  int32_t val[kUploadMax];
};
hipError_t launch_upload(const Upload& u, hipStream_t s);

// Host -> device copy on a stream, and a stream wait (set-up calls only).
hipError_t copy_to_device(void* dst, const void* src, size_t bytes, hipStream_t s);
hipError_t stream_sync(hipStream_t s);

// Events for per-kernel timing (opaque hipEvent_t handles).
hipError_t event_create(void** ev);
hipError_t event_destroy(void* ev);
hipError_t event_record(void* ev, hipStream_t s);
hipError_t event_elapsed_ms(float* ms, void* start, void* stop);  // waits for `stop`

// The calling thread's current device's copy of the library's static scratch
// array (LLAMA_SCRATCH_BYTES bytes): its device address, looked up once per
// device.
hipError_t scratch_region(void** ptr, size_t* bytes);

// Contiguous [n][G][D] <-> paged cache for positions start.. of one sequence.
hipError_t launch_kv_copy(DType t, const CacheView& c, int seq, int start, int n, void* k,
                          void* v, bool to_cache, hipStream_t s);

}  // namespace llk
