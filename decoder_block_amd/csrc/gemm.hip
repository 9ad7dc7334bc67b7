// Dense projections of the decoder layer on gfx950 MFMA, with fused epilogues.
//
// Every projection of the layer is y = x W^T with W in nn.Linear layout
// [out_features, in_features] ("From Transformer to the LLaMA series",
// section 8; "LLaMA3 Block", 4.1).  The kernel computes the transposed tile
// C^T = W_tile * X_tile^T: the MFMA A operand is a block of weight rows
// (features), the B operand a block of token rows, both K-contiguous.  In the
// 16x16 MFMA result layout each lane then owns ONE token and FOUR consecutive
// features, so every epilogue is lane-local:
//   QKV       row scale r1 (RMSNorm_1 with gamma_1 folded into W), RoPE on
//             interleaved pairs (2i, 2i+1) of q and k, q -> q buffer, k and v
//             -> their slot in the paged cache (V transposed per block)
//             ("Chapter 10", sections 3, 7);
//   RESID_H   h = x + attn W_o^T kept in fp32  ("LLaMA3 Block", 4.2 step 4);
//   SWIGLU    gate/up rows are interleaved at pack time (row 2j = gate_j,
//             2j+1 = up_j), so s_j = SiLU(r2 g_j) * (r2 u_j) is formed in
//             registers  ("3.2 Core components", 3.2.2);
//   RESID_OUT out = h + s W_down^T  ("LLaMA3 Block", 4.2 step 8).
//
// Tiles: BN features x BM tokens per workgroup, K staged 128 bytes per row
// (64 bf16 / 32 fp32) through a double-buffered LDS ring with an XOR swizzle
// of the 16-byte chunk index, global loads for stage k+1 in flight while
// stage k feeds the MFMAs.  The workgroup -> tile map keeps the tiles that
// share weight panels on one XCD (8 XCDs, each with its own L2).
#include "common.h"
#include "kernels.h"

namespace llk {
namespace {

template <typename T, int BN_, int BM_, int WN_, int WM_>
struct Cfg {
  static constexpr int BN = BN_, BM = BM_, WN = WN_, WM = WM_;
  static constexpr int NT = 64 * WN * WM;
  static constexpr int CPR = 8;  // 16-byte chunks per tile row
  static constexpr int BK = CPR * Chunk<T>::N;
  static constexpr int FW = BN / WN, TW = BM / WM;
  static constexpr int FI = FW / 16, TJ = TW / 16;
  static constexpr int RSTEP = NT / CPR;  // tile rows covered by one pass of the threads
  static constexpr int LW = BN / RSTEP, LX = BM / RSTEP;
  static_assert(BN % RSTEP == 0 && BM % RSTEP == 0, "tile rows must split evenly");
  static_assert(FW % 16 == 0 && TW % 16 == 0, "wave tile must be 16-aligned");
};

DEVI int swz(int row, int c) { return row * 8 + (c ^ (row & 7)); }

DEVI float silu(float z) { return z / (1.f + __expf(-z)); }

template <typename T>
DEVI void store4(T* p, float a, float b, float c, float d) {
  if constexpr (sizeof(T) == 4) {
    *reinterpret_cast<f32x4*>(p) = f32x4{a, b, c, d};
  } else {
    *reinterpret_cast<bf16x4*>(p) = bf16x4{from_f32<bf16>(a), from_f32<bf16>(b),
                                           from_f32<bf16>(c), from_f32<bf16>(d)};
  }
}
template <typename T>
DEVI f32x4 load4(const T* p) {
  if constexpr (sizeof(T) == 4) {
    return *reinterpret_cast<const f32x4*>(p);
  } else {
    bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
    return f32x4{to_f32(v[0]), to_f32(v[1]), to_f32(v[2]), to_f32(v[3])};
  }
}

// Epilogue for one lane-quad: token t, features f .. f+3, accumulator v.
template <typename T, int EPI>
DEVI void epilogue(const GemmArgs& a, int t, int f, f32x4 v) {
  if constexpr (EPI == (int)Epi::QKV) {
    const float r = a.rowscale[t];
    v *= r;
    const int D = a.cache.D, G = a.cache.G;
    const int HD = a.H * D, KD = G * D;
    if (f >= HD + 2 * KD) return;  // zero padding rows of the packed weights
    const int b = t / a.batch.seq_len;
    const int s = t - b * a.batch.seq_len;
    const int seq = a.batch.desc[2 * b];
    const int pos = a.batch.desc[2 * b + 1] + s;
    if (f < HD + KD) {  // q or k: rotate pairs (f, f+1) and (f+2, f+3)
      const int dd = (f < HD ? f : f - HD) % D;
      const float* cs = a.rope_cos + (size_t)pos * (D / 2) + dd / 2;
      const float* sn = a.rope_sin + (size_t)pos * (D / 2) + dd / 2;
      const float c0 = cs[0], s0 = sn[0], c1 = cs[1], s1 = sn[1];
      const float e0 = v[0], o0 = v[1], e1 = v[2], o1 = v[3];
      v[0] = e0 * c0 - o0 * s0;
      v[1] = e0 * s0 + o0 * c0;
      v[2] = e1 * c1 - o1 * s1;
      v[3] = e1 * s1 + o1 * c1;
    }
    if (f < HD) {
      store4(reinterpret_cast<T*>(a.q_out) + (size_t)t * HD + f, v[0], v[1], v[2], v[3]);
    } else {
      const bool is_k = f < HD + KD;
      const int kf = is_k ? f - HD : f - HD - KD;
      const int g = kf / D, dd = kf - g * D;
      const size_t blk = (size_t)a.cache.block_table[(size_t)seq * a.cache.max_blocks + (pos >> 4)];
      if (is_k) {  // K block [16 slots][D]
        T* dst = reinterpret_cast<T*>(a.cache.k_pool) + ((blk * G + g) * 16 + (pos & 15)) * D + dd;
        store4(dst, v[0], v[1], v[2], v[3]);
      } else {     // V block kept transposed: [D][16 slots]
        T* dst = reinterpret_cast<T*>(a.cache.v_pool) + ((blk * G + g) * D + dd) * 16 + (pos & 15);
        dst[0] = from_f32<T>(v[0]);
        dst[16] = from_f32<T>(v[1]);
        dst[32] = from_f32<T>(v[2]);
        dst[48] = from_f32<T>(v[3]);
      }
    }
  } else if constexpr (EPI == (int)Epi::RESID_H) {
    const size_t o = (size_t)t * a.ldo + f;
    f32x4 x = load4(reinterpret_cast<const T*>(a.resid) + o);
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + o) = x + v;
  } else if constexpr (EPI == (int)Epi::SWIGLU) {
    const float r = a.rowscale[t];
    v *= r;
    const float s0 = silu(v[0]) * v[1];
    const float s1 = silu(v[2]) * v[3];
    T* o = reinterpret_cast<T*>(a.out) + (size_t)t * a.ldo + f / 2;
    o[0] = from_f32<T>(s0);
    o[1] = from_f32<T>(s1);
  } else {  // RESID_OUT
    const size_t o = (size_t)t * a.ldo + f;
    f32x4 h = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(a.resid) + o);
    h += v;
    if (a.out_dtype == DType::F32)
      *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + o) = h;
    else
      store4(reinterpret_cast<bf16*>(a.out) + o, h[0], h[1], h[2], h[3]);
  }
}

template <typename T, typename C, int EPI>
__global__ __launch_bounds__(C::NT) void gemm_kernel(GemmArgs a) {
  using vec = typename Chunk<T>::vec;
  __shared__ u32x4 sW[2][C::BN * C::CPR];
  __shared__ u32x4 sX[2][C::BM * C::CPR];

  // ---- workgroup -> tile: XCD-contiguous ranges, then grouped along M ----
  const int tiles_n = a.N / C::BN;
  const int tiles_m = (a.M + C::BM - 1) / C::BM;
  const int total = tiles_n * tiles_m;
  int pid = blockIdx.x;
  if (total % 8 == 0) pid = (pid % 8) * (total / 8) + pid / 8;
  constexpr int GROUP = 8;
  const int per_group = GROUP * tiles_n;
  const int gid = pid / per_group;
  const int first_m = gid * GROUP;
  const int gsize = min(tiles_m - first_m, GROUP);
  const int tm = first_m + (pid % per_group) % gsize;
  const int tn = (pid % per_group) / gsize;
  const int n0 = tn * C::BN, m0 = tm * C::BM;

  const int tid = threadIdx.x;
  const int lc = tid & 7, lr = tid >> 3;
  const int lane = tid & 63, wave = tid >> 6;
  const int wn = wave % C::WN, wm = wave / C::WN;

  const T* W = reinterpret_cast<const T*>(a.W);
  const T* X = reinterpret_cast<const T*>(a.X);
  u32x4 rw[C::LW], rx[C::LX];
  const u32x4 zero = {0u, 0u, 0u, 0u};

  auto gload = [&](int kt) {
    const int kel = kt * C::BK + lc * Chunk<T>::N;
#pragma unroll
    for (int i = 0; i < C::LW; ++i) {
      const int row = lr + i * C::RSTEP;
      rw[i] = *reinterpret_cast<const u32x4*>(W + (size_t)(n0 + row) * a.K + kel);
    }
#pragma unroll
    for (int i = 0; i < C::LX; ++i) {
      const int m = m0 + lr + i * C::RSTEP;
      rx[i] = m < a.M ? *reinterpret_cast<const u32x4*>(X + (size_t)m * a.ldx + kel) : zero;
    }
  };
  auto sstore = [&](int st) {
#pragma unroll
    for (int i = 0; i < C::LW; ++i) sW[st][swz(lr + i * C::RSTEP, lc)] = rw[i];
#pragma unroll
    for (int i = 0; i < C::LX; ++i) sX[st][swz(lr + i * C::RSTEP, lc)] = rx[i];
  };

  f32x4 acc[C::FI][C::TJ];
#pragma unroll
  for (int i = 0; i < C::FI; ++i)
#pragma unroll
    for (int j = 0; j < C::TJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = a.K / C::BK;
  gload(0);
  sstore(0);
  __syncthreads();

  const int l16 = lane & 15, lg = lane >> 4;
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int c = ks * 4 + lg;
      vec af[C::FI], bf[C::TJ];
#pragma unroll
      for (int i = 0; i < C::FI; ++i) {
        const int row = wn * C::FW + 16 * i + l16;
        af[i] = __builtin_bit_cast(vec, sW[st][swz(row, c)]);
      }
#pragma unroll
      for (int j = 0; j < C::TJ; ++j) {
        const int row = wm * C::TW + 16 * j + l16;
        bf[j] = __builtin_bit_cast(vec, sX[st][swz(row, c)]);
      }
#pragma unroll
      for (int i = 0; i < C::FI; ++i)
#pragma unroll
        for (int j = 0; j < C::TJ; ++j) acc[i][j] = mfma16_chunk(acc[i][j], af[i], bf[j]);
    }
    if (kt + 1 < nk) sstore(st ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < C::FI; ++i) {
    const int f = n0 + wn * C::FW + 16 * i + 4 * lg;
#pragma unroll
    for (int j = 0; j < C::TJ; ++j) {
      const int t = m0 + wm * C::TW + 16 * j + l16;
      if (t < a.M) epilogue<T, EPI>(a, t, f, acc[i][j]);
    }
  }
}

template <typename T, typename C>
hipError_t launch_cfg(const GemmArgs& a, hipStream_t s) {
  if (a.N % C::BN != 0 || a.K % C::BK != 0 || a.M <= 0) return hipErrorInvalidValue;
  const int grid = (a.N / C::BN) * ((a.M + C::BM - 1) / C::BM);
  switch (a.epi) {
    case Epi::QKV: gemm_kernel<T, C, 0><<<grid, C::NT, 0, s>>>(a); break;
    case Epi::RESID_H: gemm_kernel<T, C, 1><<<grid, C::NT, 0, s>>>(a); break;
    case Epi::SWIGLU: gemm_kernel<T, C, 2><<<grid, C::NT, 0, s>>>(a); break;
    case Epi::RESID_OUT: gemm_kernel<T, C, 3><<<grid, C::NT, 0, s>>>(a); break;
  }
  return hipGetLastError();
}

using LargeBF = Cfg<bf16, 256, 256, 2, 4>;
using SmallBF = Cfg<bf16, 64, 64, 2, 2>;
using LargeF = Cfg<float, 256, 256, 2, 4>;
using SmallF = Cfg<float, 64, 64, 2, 2>;

}  // namespace

int gemm_tile_n(GemmTile t) { return t == GemmTile::LARGE ? 256 : 64; }

hipError_t launch_gemm(DType t, GemmTile tile, const GemmArgs& a, hipStream_t s) {
  if (t == DType::BF16)
    return tile == GemmTile::LARGE ? launch_cfg<bf16, LargeBF>(a, s) : launch_cfg<bf16, SmallBF>(a, s);
  return tile == GemmTile::LARGE ? launch_cfg<float, LargeF>(a, s) : launch_cfg<float, SmallF>(a, s);
}

}  // namespace llk
