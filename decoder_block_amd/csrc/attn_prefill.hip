// Causal grouped-query attention for prefill, flash style, on gfx950 MFMA.
//
// o[t, h] = sum_{j <= t} softmax_j(q[t,h] . k[j,g] / sqrt(D)) v[j,g] with
// g = h / (H/G) ("From Transformer to LLaMA: an overview", 1.1; "Chapter 10:
// the modern LLaMA architecture", section 6 -- K/V are broadcast to the query
// heads of their group inside the kernel, never materialised).  Keys come
// from the paged cache, so new tokens also see every cached key before them
// (absolute positions, "Chapter 10", section 7).
//
// Work split: one workgroup (4 waves, 128 query rows) per (sequence, KV
// group, block of positions).  The 128 rows are the R = H/G query heads of
// the group times 128/R positions, so every K/V tile staged in LDS serves all
// heads of the group.  Row blocks are issued latest-position first (the
// longest causal rows start first) and the KV groups of a row block sit on
// consecutive workgroup ids, i.e. one group per XCD.
//
// Per wave, transposed formulation with 32x32 MFMAs:
//   S^T [keys x rows] = K_tile [keys x D] * Q^T        (Q resident in registers)
//   online softmax: each lane owns one query row and 32 of the 64 scores of a
//   tile; the row max needs one exchange with lane l^32, the running sum none
//   O^T [D x rows]   += V_tile^T [D x keys] * P^T     (P straight from registers)
// The cache keeps V transposed per block ([D][16 keys]), so V^T tiles are
// staged with plain 16-byte copies.  K and V^T tiles are double buffered in
// LDS (XOR-swizzled 16-byte chunks); the next tile's global loads are in
// flight during the MFMAs.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace llk {
namespace {

template <typename T, int D_>
struct ACfg {
  static constexpr int D = D_;
  static constexpr int CH = Chunk<T>::N;            // elements per 16-byte chunk
  static constexpr int KT = 64;                     // keys per tile
  static constexpr int CPRK = D * (int)sizeof(T) / 16;  // chunks per K row
  static constexpr int NQ = D / (2 * CH);           // QK k-steps
  static constexpr int NDB = D / 32;                // 32-row blocks of O^T
  static constexpr int VROW = KT * (int)sizeof(T) / 16;  // chunks per V^T row
  static constexpr int LK = KT * CPRK / 256;        // K chunks loaded per thread
  static constexpr int LV = D * VROW / 256;         // V^T chunks loaded per thread
  static_assert(LK >= 1 && LV >= 1, "tile too small for 256 threads");
};


template <typename T, int D>
__global__ __launch_bounds__(256) void attn_prefill_kernel(const T* __restrict__ q, T* __restrict__ attn,
                                                           int H, CacheView cache, BatchView batch) {
  using C = ACfg<T, D>;
  using vec = typename Chunk<T>::vec;
  __shared__ u32x4 sK[2][C::KT * C::CPRK];
  __shared__ u32x4 sV[2][D * C::VROW];

  const int G = cache.G;
  const int R = H / G;
  const int P = 128 / R;  // positions per workgroup
  const int S = batch.seq_len;
  const int b = blockIdx.x / G, g = blockIdx.x % G;
  const int nrb = (S + P - 1) / P;
  const int rb = nrb - 1 - (int)blockIdx.y;
  const int seq = batch.desc[2 * b];
  const int start = batch.desc[2 * b + 1];
  const int kv_len = start + S;
  const int HD = H * D;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5;            // lane group
  const int j = wave * 32 + (lane & 31);  // this lane's query row in the block
  const int r = j / P, pp = j % P;
  const int sidx = rb * P + pp;
  const bool active = sidx < S;
  const int head = g * R + r;
  const int qpos = start + (active ? sidx : rb * P);  // inactive rows mirror a valid one
  const size_t tok = (size_t)b * S + (active ? sidx : rb * P);

  // wave-uniform position range
  int wmax = qpos, wmin = qpos;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    wmax = max(wmax, __shfl_xor(wmax, m, 64));
    wmin = min(wmin, __shfl_xor(wmin, m, 64));
  }
  const int last_s = min(S, (rb + 1) * P) - 1;
  const int ntiles = (start + last_s) / C::KT + 1;

  // Q fragments (B operand of S^T), resident for the whole key loop
  vec qf[C::NQ];
  {
    const T* qp = q + tok * HD + (size_t)head * D;
#pragma unroll
    for (int kk = 0; kk < C::NQ; ++kk) qf[kk] = load_chunk<T>(qp + (2 * kk + hl) * C::CH);
    if (!active) {
#pragma unroll
      for (int kk = 0; kk < C::NQ; ++kk) qf[kk] = zero_chunk<T>();
    }
  }

  const T* kpool = reinterpret_cast<const T*>(cache.k_pool);
  const T* vpool = reinterpret_cast<const T*>(cache.v_pool);
  const int32_t* btab = cache.block_table + (size_t)seq * cache.max_blocks;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  u32x4 rk[C::LK], rv[C::LV];

  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < C::LK; ++i) {
      const int item = tid + 256 * i;
      const int key = item / C::CPRK, c = item % C::CPRK;
      const int kp = kt * C::KT + key;
      if (kp < kv_len) {
        const int blk = btab[kp >> 4];
        rk[i] = *reinterpret_cast<const u32x4*>(kpool + (((size_t)blk * G + g) * 16 + (kp & 15)) * D + c * C::CH);
      } else {
        rk[i] = zero;
      }
    }
#pragma unroll
    for (int i = 0; i < C::LV; ++i) {
      const int item = tid + 256 * i;
      const int d = item / C::VROW, c = item % C::VROW;
      const int kp = kt * C::KT + c * C::CH;  // first key of this chunk
      if (kp < kv_len) {
        const int blk = btab[kp >> 4];
        rv[i] = *reinterpret_cast<const u32x4*>(vpool + (((size_t)blk * G + g) * D + d) * 16 + (kp & 15));
        if (kp + C::CH > kv_len) {  // keys past the end may hold stale data: zero them
          vec v = __builtin_bit_cast(vec, rv[i]);
#pragma unroll
          for (int e = 0; e < C::CH; ++e)
            if (kp + e >= kv_len) v[e] = from_f32<T>(0.f);
          rv[i] = __builtin_bit_cast(u32x4, v);
        }
      } else {
        rv[i] = zero;
      }
    }
  };
  auto sstore = [&](int st) {
#pragma unroll
    for (int i = 0; i < C::LK; ++i) {
      const int item = tid + 256 * i;
      const int key = item / C::CPRK, c = item % C::CPRK;
      sK[st][key * C::CPRK + (c ^ (key & 7))] = rk[i];
    }
#pragma unroll
    for (int i = 0; i < C::LV; ++i) {
      const int item = tid + 256 * i;
      const int d = item / C::VROW, c = item % C::VROW;
      sV[st][d * C::VROW + (c ^ (d & 7))] = rv[i];
    }
  };

  const float scale = 1.4426950408889634f / sqrtf((float)D);  // log2(e) / sqrt(D)
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 o[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.f;

  gload(0);
  sstore(0);
  __syncthreads();

  for (int kt = 0; kt < ntiles; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < ntiles) gload(kt + 1);
    const int k0 = kt * C::KT;
    if (k0 <= wmax) {
      // ---- S^T = K Q^T ----
      f32x16 sc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) sc[kb][i] = 0.f;
        const int key = 32 * kb + (lane & 31);
#pragma unroll
        for (int kk = 0; kk < C::NQ; ++kk) {
          const int c = 2 * kk + hl;
          const vec a = __builtin_bit_cast(vec, sK[st][key * C::CPRK + (c ^ (key & 7))]);
          sc[kb] = mfma32_chunk(sc[kb], a, qf[kk]);
        }
      }
      // ---- online softmax (lane = one query row) ----
      const bool need_mask = k0 + C::KT - 1 > wmin;
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float s = sc[kb][i] * scale;
          if (need_mask) {
            const int kp = k0 + 32 * kb + 8 * (i >> 2) + 4 * hl + (i & 3);
            if (kp > qpos) s = -INFINITY;
          }
          sc[kb][i] = s;
          mx = fmaxf(mx, s);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = exp2f(m_run - m_new);
      float psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = exp2f(sc[kb][i] - m_new);
          sc[kb][i] = p;
          psum += p;
        }
      l_run = l_run * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) o[db] *= alpha;

      // ---- O^T += V^T P^T ----
      // A operand: lane (row d, group hl) supplies keys 16m+4hl+{0..3} and
      // 16m+8+4hl+{0..3}, matching the keys its P registers hold.
      const char* vb = reinterpret_cast<const char*>(&sV[st][0]);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          vec pv[8 / C::CH];
#pragma unroll
          for (int e = 0; e < 8; ++e) pv[e / C::CH][e % C::CH] = from_f32<T>(sc[kb][8 * m + e]);
#pragma unroll
          for (int db = 0; db < C::NDB; ++db) {
            const int d = 32 * db + (lane & 31);
            const char* row = vb + (size_t)d * C::VROW * 16;
            auto piece = [&](int key) {  // 4 consecutive keys of row d
              const int byte = key * (int)sizeof(T);
              return row + (((byte >> 4) ^ (d & 7)) << 4) + (byte & 15);
            };
            const int kA = 32 * kb + 16 * m + 4 * hl, kB = kA + 8;
            if constexpr (sizeof(T) == 2) {
              const u32x2 lo = *reinterpret_cast<const u32x2*>(piece(kA));
              const u32x2 hi = *reinterpret_cast<const u32x2*>(piece(kB));
              const vec a = __builtin_bit_cast(vec, u32x4{lo[0], lo[1], hi[0], hi[1]});
              o[db] = mfma32_chunk(o[db], a, pv[0]);
            } else {
              const vec a0 = *reinterpret_cast<const vec*>(piece(kA));
              const vec a1 = *reinterpret_cast<const vec*>(piece(kB));
              o[db] = mfma32_chunk(o[db], a0, pv[0]);
              o[db] = mfma32_chunk(o[db], a1, pv[8 / C::CH - 1]);
            }
          }
        }
    }
    if (kt + 1 < ntiles) sstore(st ^ 1);
    __syncthreads();
  }

  if (!active) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.f / l_tot;
  T* op = attn + tok * HD + (size_t)head * D;
#pragma unroll
  for (int db = 0; db < C::NDB; ++db)
#pragma unroll
    for (int ig = 0; ig < 4; ++ig) {
      const int d0 = 32 * db + 8 * ig + 4 * hl;
      if constexpr (sizeof(T) == 2) {
        *reinterpret_cast<bf16x4*>(op + d0) =
            bf16x4{from_f32<bf16>(o[db][4 * ig] * inv), from_f32<bf16>(o[db][4 * ig + 1] * inv),
                   from_f32<bf16>(o[db][4 * ig + 2] * inv), from_f32<bf16>(o[db][4 * ig + 3] * inv)};
      } else {
        *reinterpret_cast<f32x4*>(op + d0) =
            f32x4{o[db][4 * ig] * inv, o[db][4 * ig + 1] * inv, o[db][4 * ig + 2] * inv, o[db][4 * ig + 3] * inv};
      }
    }
}

template <typename T, int D>
hipError_t launch_d(const void* q, void* attn, int H, const CacheView& c, const BatchView& b, hipStream_t s) {
  const int R = H / c.G;
  const int P = 128 / R;
  dim3 grid(c.G * b.batch, (b.seq_len + P - 1) / P);
  attn_prefill_kernel<T, D><<<grid, 256, 0, s>>>(reinterpret_cast<const T*>(q), reinterpret_cast<T*>(attn), H, c, b);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_prefill(DType t, const void* q, void* attn, int H, const CacheView& c, const BatchView& b,
                               hipStream_t s) {
  if (H % c.G != 0 || 128 % (H / c.G) != 0) return hipErrorInvalidValue;
  if (t == DType::BF16) {
    if (c.D == 128) return launch_d<bf16, 128>(q, attn, H, c, b, s);
    if (c.D == 64) return launch_d<bf16, 64>(q, attn, H, c, b, s);
  } else {
    if (c.D == 128) return launch_d<float, 128>(q, attn, H, c, b, s);
    if (c.D == 64) return launch_d<float, 64>(q, attn, H, c, b, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace llk
