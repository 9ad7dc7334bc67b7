// Grouped-query decode attention over the paged KV cache (split-K), gfx950.
//
// One new token per sequence at position len attends to all len + 1 keys of
// its sequence (the cached ones plus its own, appended by the QKV epilogue
// before this kernel runs): "Chapter 10: the modern LLaMA architecture",
// section 7 (q_len = 1, k_len = past_len + 1).  Query head h reads KV head
// g = h / (H/G) (section 6).  The step is bound by HBM: every key and value
// of the batch is read once per KV group, shared by the R = H/G query heads.
//
// Split kernel: a workgroup (4 waves) takes one (sequence, group, chunk of
// 1024 keys) and the group's query heads in 16-column MFMA groups (bf16: one
// group up to R = 16, two at R = 32, so K and V are read once per KV group
// either way; fp32: one workgroup per 16 heads); each wave walks its keys
// block by block and runs both products on
// 16x16 MFMAs with the heads as the 16 columns:
//   S^T [16 keys x heads] = K_block [16 x D] * Q^T   (K loaded straight from HBM)
//   O^T [D x heads]      += V_block^T [D x 32 keys] * P^T
// V is kept transposed per block in the cache, so the A operand of the second
// product is a plain 8/16-byte load.  The online softmax state (running max
// and sum per head) lives in the lanes; the four waves are merged through LDS
// and the chunk's (max, sum, unnormalised output) go to a partial buffer.
// Combine kernel: per (sequence, head), a log-sum-exp merge of the chunks.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace llk {
namespace {

constexpr int kChunkKeys = 1024;

template <typename T, int D_>
struct DCfg {
  static constexpr int D = D_;
  static constexpr int CH = Chunk<T>::N;
  static constexpr int NQK = D / (4 * CH);  // 16x16 MFMA chunk-steps over D
  static constexpr int NDB = D / 16;        // 16-row blocks of O^T
};

template <typename T>
struct VPiece;  // 4 consecutive keys of one V^T row
template <> struct VPiece<bf16> { typedef u32x2 type; };
template <> struct VPiece<float> { typedef u32x4 type; };

// Zero the elements e >= n of a 4-key piece (bf16: two words, fp32: four words).
DEVI u32x2 keep_first(u32x2 w, int n) {
  w[0] = n >= 2 ? w[0] : (n == 1 ? (w[0] & 0xFFFFu) : 0u);
  w[1] = n >= 4 ? w[1] : (n == 3 ? (w[1] & 0xFFFFu) : 0u);
  return w;
}
DEVI u32x4 keep_first(u32x4 w, int n) {
#pragma unroll
  for (int e = 0; e < 4; ++e) w[e] = e < n ? w[e] : 0u;
  return w;
}

// Work unit u of a launch -> (sequence b, 1024-key chunk c); b = -1 past the
// last unit.  The units are every full chunk first, sequence by sequence, then
// the partial last chunk of each sequence that has one, so the launch has no
// empty workgroups and its last workgroups are the shorter partial chunks.
// Each wave derives the map from the batch's lengths (scans over 64
// sequences at a time); every lane gets the same (b, c).
DEVI void unit_chunk(const BatchView& batch, int u, int lane, int& b, int& c) {
  const int B = batch.batch;
  int base = 0;
  for (int b0 = 0; b0 < B; b0 += 64) {  // full chunks
    const int bb = b0 + lane;
    const int f = bb < B ? (batch.desc[2 * bb + 1] + 1) / kChunkKeys : 0;
    int incl = f;  // inclusive prefix sum over the lanes
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    const int tot = __shfl(incl, 63, 64);
    if (u < base + tot) {
      const int ln = __ffsll((unsigned long long)__ballot(incl > u - base)) - 1;
      b = b0 + ln;
      c = u - base - (__shfl(incl, ln, 64) - __shfl(f, ln, 64));
      return;
    }
    base += tot;
  }
  for (int b0 = 0; b0 < B; b0 += 64) {  // partial chunks
    const int bb = b0 + lane;
    const int len = bb < B ? batch.desc[2 * bb + 1] + 1 : 0;
    const bool part = bb < B && len % kChunkKeys != 0;
    const unsigned long long m = __ballot(part);
    const int cnt = __popcll(m);
    if (u < base + cnt) {  // the (u - base)-th sequence of this group with a partial chunk
      const bool mine = part && __popcll(m & ((1ull << lane) - 1)) == u - base;
      const int ln = __ffsll((unsigned long long)__ballot(mine)) - 1;
      b = b0 + ln;
      c = __shfl(len, ln, 64) / kChunkKeys;
      return;
    }
    base += cnt;
  }
  b = -1;
  c = 0;
}

template <typename T, int D>
__global__ __launch_bounds__(256) void attn_decode_split_kernel(const T* __restrict__ q, float* __restrict__ part,
                                                                int max_splits, int H, CacheView cache,
                                                                BatchView batch) {
  using C = DCfg<T, D>;
  using vec = typename Chunk<T>::vec;
  using piece = typename VPiece<T>::type;
  __shared__ float sm[4][16][D + 2];

  const int G = cache.G;
  const int R = H / G;
  // workgroup -> (sequence b, KV group g, 16-head subset sub of the group's R
  // query heads): a group with more than 16 heads (R = 32, MQA at 32 heads)
  // takes one workgroup per subset, each reading the group's K/V
  const int nsub = (R + 15) / 16;
  const int gs = blockIdx.x % (G * nsub);
  const int g = gs / nsub, hsub = gs % nsub;
  const int h0 = g * R + 16 * hsub, RS = min(16, R - 16 * hsub);  // first head, heads in the subset
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int b, split;
  unit_chunk(batch, blockIdx.x / (G * nsub), lane, b, split);
  if (b < 0) return;
  const int seq = batch.desc[2 * b];
  const int kv_len = batch.desc[2 * b + 1] + 1;
  const int k_begin = split * kChunkKeys;
  if (k_begin >= kv_len) return;
  const int k_end = min(kv_len, k_begin + kChunkKeys);

  const int c16 = lane & 15, g4 = lane >> 4;
  const int HD = H * D;

  // Q^T fragments: column c16 = query head h0 + c16 (zero for c16 >= RS)
  vec qf[C::NQK];
  {
    const T* qp = q + (size_t)b * HD + (size_t)(h0 + c16) * D;
#pragma unroll
    for (int s = 0; s < C::NQK; ++s)
      qf[s] = c16 < RS ? load_chunk<T>(qp + (4 * s + g4) * C::CH) : zero_chunk<T>();
  }

  const T* kpool = reinterpret_cast<const T*>(cache.k_pool);
  const T* vpool = reinterpret_cast<const T*>(cache.v_pool);
  const int32_t* btab = cache.block_table + (size_t)seq * cache.max_blocks;

  // q arrives multiplied by log2(e)/sqrt(D) (QKV epilogue): scores are in exp2 units
  constexpr float scale = 1.f;
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int key0 = k_begin + 32 * wave; key0 < k_end; key0 += 128) {
    vec kf[2][C::NQK];
    piece vf[2][C::NDB];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int kb0 = key0 + 16 * u;
      if (kb0 < kv_len) {
        const size_t blk = (size_t)btab[kb0 >> 4];
        const T* kp = kpool + ((blk * G + g) * 16 + c16) * D;
#pragma unroll
        for (int s = 0; s < C::NQK; ++s) kf[u][s] = load_chunk<T>(kp + (4 * s + g4) * C::CH);
        const T* vp = vpool + (blk * G + g) * D * 16;
#pragma unroll
        for (int db = 0; db < C::NDB; ++db)
          vf[u][db] = *reinterpret_cast<const piece*>(vp + (16 * db + c16) * 16 + 4 * g4);
        if (kb0 + 16 > kv_len) {  // keys past the end may hold stale data: zero their values
          const int nvalid = kv_len - (kb0 + 4 * g4);
#pragma unroll
          for (int db = 0; db < C::NDB; ++db) vf[u][db] = keep_first(vf[u][db], nvalid);
        }
      } else {
#pragma unroll
        for (int s = 0; s < C::NQK; ++s) kf[u][s] = zero_chunk<T>();
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) vf[u][db] = piece{};
      }
    }

    // scores: lane holds head c16, keys key0 + 16u + 4*g4 + i
    f32x4 sc[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      sc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < C::NQK; ++s) sc[u] = mfma16_chunk(sc[u], kf[u][s], qf[s]);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = key0 + 16 * u + 4 * g4 + i;
        const float sv = key < kv_len ? sc[u][i] * scale : -INFINITY;
        sc[u][i] = sv;
        mx = fmaxf(mx, sv);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2f(m_run - m_new);
    float psum = 0.f;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = exp2f(sc[u][i] - m_new);
        sc[u][i] = p;
        psum += p;
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) o[db] *= alpha;

    // O^T += V^T P^T: element e < 4 of a lane's operand is key 4*g4+e of the
    // first block, e >= 4 the same key of the second block.
    if constexpr (sizeof(T) == 2) {
      const bf16x8 pb = {from_f32<bf16>(sc[0][0]), from_f32<bf16>(sc[0][1]), from_f32<bf16>(sc[0][2]),
                         from_f32<bf16>(sc[0][3]), from_f32<bf16>(sc[1][0]), from_f32<bf16>(sc[1][1]),
                         from_f32<bf16>(sc[1][2]), from_f32<bf16>(sc[1][3])};
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
        const u32x2 lo = __builtin_bit_cast(u32x2, vf[0][db]);
        const u32x2 hi = __builtin_bit_cast(u32x2, vf[1][db]);
        const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
        o[db] = mfma16_chunk(o[db], a, pb);
      }
    } else {
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
        o[db] = mfma16_chunk(o[db], __builtin_bit_cast(f32x4, vf[0][db]), sc[0]);
        o[db] = mfma16_chunk(o[db], __builtin_bit_cast(f32x4, vf[1][db]), sc[1]);
      }
    }
  }

  // ---- merge the four waves ----
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
#pragma unroll
  for (int db = 0; db < C::NDB; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) sm[wave][c16][2 + 16 * db + 4 * g4 + i] = o[db][i];
  if (g4 == 0) {
    sm[wave][c16][0] = m_run;
    sm[wave][c16][1] = l_run;
  }
  __syncthreads();
  // 256 threads: head hh = tid / 16 (16 heads), 16 threads per head over D + 2 values
  const int hh = tid >> 4, sub = tid & 15;
  if (hh >= RS) return;
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < 4; ++w) M = fmaxf(M, sm[w][hh][0]);
  float f[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) f[w] = exp2f(sm[w][hh][0] - M);  // waves without keys: exp2(-inf) = 0
  float* dst = part + (((size_t)b * H + h0 + hh) * max_splits + split) * (D + 2);
  for (int x = sub; x < D + 2; x += 16) {
    float v;
    if (x == 0) {
      v = M;
    } else {
      v = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) v += f[w] * sm[w][hh][x];
    }
    dst[x] = v;
  }
}

// ---------------------------------------------------------------------------
// bf16 split kernel.  A workgroup takes one (sequence, group, chunk of 1024
// keys); each of its four waves walks its own quarter (256 keys = 16 cache
// blocks) and the quarters are merged through LDS at the end.  Per 16-key
// block:
//   S^T [16 keys x heads] = K_block [16 x D] * Q^T     (16x16x32 MFMAs)
//   O^T [D x heads]      += V_block^T [D x 16] * P^T   (16x16x16 MFMAs)
// The score layout (lane: head column, four consecutive keys) is exactly the
// B operand layout of the second product, so P never leaves the lane.  The
// K and V blocks of block i+1 are loaded while block i is computed (two
// register buffers).  Short per-wave ranges keep the waves' work even, and
// the small register footprint keeps several waves per SIMD in flight.
// ---------------------------------------------------------------------------
constexpr int kWaveKeys = kChunkKeys / 4;

template <int D>
struct KV16 {
  bf16x8 k[D / 32];   // K rows: lane (key c16, k-group g4) holds D-chunks 4s + g4
  u32x2 v[D / 16];    // V^T rows 16 db + c16, keys 4 g4 .. 4 g4 + 3 (stored at vperm_pos(4 g4))
};

// Loads of block blk (group g) through buffer descriptors; a block that is not
// live gets an empty descriptor, so the load moves no memory and returns zeros
// while keeping every iteration's load count the same.
template <int D>
DEVI void load_kv16(KV16<D>& r, const bf16* kpool, const bf16* vpool, int blk, bool live, int G, int g, int c16,
                    int g4) {
  constexpr uint32_t kBytes = 16 * D * 2;
  const size_t off = ((size_t)blk * G + g) * 16 * D;
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(kpool + off), 0, live ? kBytes : 0u, 0x00020000);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(vpool + off), 0, live ? kBytes : 0u, 0x00020000);
#pragma unroll
  for (int s = 0; s < D / 32; ++s)
    r.k[s] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, (c16 * D + (4 * s + g4) * 8) * 2, 0, 0));
#pragma unroll
  for (int db = 0; db < D / 16; ++db)
    r.v[db] = __builtin_amdgcn_raw_buffer_load_b64(rv, ((16 * db + c16) * 16 + vperm_pos(4 * g4)) * 2, 0, 0);
}

DEVI f32x4 mfma16x16x16(f32x4 c, u32x2 a, u32x2 b) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c, 0, 0,
                                                    0);
}

// NG head groups of 16 per workgroup: NG = 2 serves the 32 query heads of an
// MQA group (R = 32) with one read of its K/V instead of one per 16 heads.
template <int D, int NG>
__global__ __launch_bounds__(256, NG == 1 ? 3 : 2) void attn_decode_wave_kernel(
    const bf16* __restrict__ q, float* __restrict__ part, int max_splits, int H, CacheView cache, BatchView batch) {
  constexpr int HW = 16 * NG;  // heads per workgroup
  __shared__ float sm[4][HW][D + 2];
  const int G = cache.G;
  const int R = H / G;
  // workgroup -> (sequence b, KV group g, subset hsub of up to HW of the
  // group's R query heads); each subset's workgroup reads the group's K/V
  const int nsub = (R + HW - 1) / HW;
  const int gs = blockIdx.x % (G * nsub);
  const int g = gs / nsub, hsub = gs % nsub;
  const int h0 = g * R + HW * hsub, RS = min(HW, R - HW * hsub);  // first head, heads in the subset
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int b, split;
  unit_chunk(batch, blockIdx.x / (G * nsub), lane, b, split);
  b = __builtin_amdgcn_readfirstlane(b);
  split = __builtin_amdgcn_readfirstlane(split);
  if (b < 0) return;
  const int seq = batch.desc[2 * b];
  const int kv_len = batch.desc[2 * b + 1] + 1;
  if (split * kChunkKeys >= kv_len) return;
  const int k_begin = split * kChunkKeys + wave * kWaveKeys;
  const int nkeys = max(0, min(kv_len - k_begin, kWaveKeys));
  const int nblk = (nkeys + 15) >> 4;

  const int c16 = lane & 15, g4 = lane >> 4;
  bf16x8 qf[NG][D / 32];
#pragma unroll
  for (int ng = 0; ng < NG; ++ng) {
    const int hc = 16 * ng + c16;
    const bf16* qp = q + (size_t)b * H * D + (size_t)(h0 + hc) * D;
#pragma unroll
    for (int s = 0; s < D / 32; ++s)
      qf[ng][s] = hc < RS ? load_chunk<bf16>(qp + (4 * s + g4) * 8) : zero_chunk<bf16>();
  }
  const int32_t* btab = cache.block_table + (size_t)seq * cache.max_blocks + (k_begin >> 4);
  const bf16* kpool = reinterpret_cast<const bf16*>(cache.k_pool);
  const bf16* vpool = reinterpret_cast<const bf16*>(cache.v_pool);

  // q arrives multiplied by log2(e)/sqrt(D) (QKV epilogue): scores are in exp2 units
  float m_run[NG], l_run[NG];
  f32x4 o[NG][D / 16];
#pragma unroll
  for (int ng = 0; ng < NG; ++ng) {
    m_run[ng] = -INFINITY;
    l_run[ng] = 0.f;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) o[ng][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  auto compute = [&](KV16<D>& r, int i) {
    const int key0 = 16 * i;  // within the wave's range
    if (key0 + 16 > nkeys) {  // keys past the end may hold stale data: zero their values
      const int nvalid = nkeys - (key0 + 4 * g4);
#pragma unroll
      for (int db = 0; db < D / 16; ++db) r.v[db] = keep_first(r.v[db], nvalid);
    }
#pragma unroll
    for (int ng = 0; ng < NG; ++ng) {
      f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < D / 32; ++s) sc = mfma16_chunk(sc, r.k[s], qf[ng][s]);
      float mx = -INFINITY;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float sv = key0 + 4 * g4 + e < nkeys ? sc[e] : -INFINITY;
        sc[e] = sv;
        mx = fmaxf(mx, sv);
      }
      mx = fmaxf(mx, shfl_xor(mx, 16));
      mx = fmaxf(mx, shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run[ng], mx);
      const float alpha = fast_exp2(m_run[ng] - m_new);
      float p[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) p[e] = fast_exp2(sc[e] - m_new);
      // P in bf16 (the O^T product's operand); the row sum adds the same
      // bf16 values, so O / l is a weighted mean of V with weights summing to one
      const bf16x4 pb = {from_f32<bf16>(p[0]), from_f32<bf16>(p[1]), from_f32<bf16>(p[2]), from_f32<bf16>(p[3])};
      const bf16x2 ones2 = {from_f32<bf16>(1.f), from_f32<bf16>(1.f)};
      float ps = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[0], pb[1]}, ones2, 0.f, false);
      ps = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[2], pb[3]}, ones2, ps, false);
      l_run[ng] = l_run[ng] * alpha + ps;
      m_run[ng] = m_new;
      const u32x2 pw = __builtin_bit_cast(u32x2, pb);
#pragma unroll
      for (int db = 0; db < D / 16; ++db) o[ng][db] = mfma16x16x16(o[ng][db] * alpha, r.v[db], pw);
    }
  };

  // Two register buffers; every iteration issues the same loads (blocks past
  // the range are empty), so the waits for block i never cover block i+1.
  if (nblk > 0) {
    KV16<D> ra, rb;
    load_kv16<D>(ra, kpool, vpool, btab[0], true, G, g, c16, g4);
    int id_b = btab[min(1, nblk - 1)];
#pragma unroll 1
    for (int i = 0; i < nblk; i += 2) {
      load_kv16<D>(rb, kpool, vpool, id_b, i + 1 < nblk, G, g, c16, g4);
      const int id_a = btab[min(i + 2, nblk - 1)];
      compute(ra, i);
      load_kv16<D>(ra, kpool, vpool, id_a, i + 2 < nblk, G, g, c16, g4);
      id_b = btab[min(i + 3, nblk - 1)];
      if (i + 1 < nblk) compute(rb, i + 1);
    }
  }

  // ---- merge the four waves (a wave without keys has m = -inf, l = 0, o = 0) ----
#pragma unroll
  for (int ng = 0; ng < NG; ++ng) {
    float l = l_run[ng];
    l += shfl_xor(l, 16);
    l += shfl_xor(l, 32);
    const int hc = 16 * ng + c16;
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
#pragma unroll
      for (int e = 0; e < 4; ++e) sm[wave][hc][2 + 16 * db + 4 * g4 + e] = o[ng][db][e];
    if (g4 == 0) {
      sm[wave][hc][0] = m_run[ng];
      sm[wave][hc][1] = l;
    }
  }
  __syncthreads();
  const int sub = tid & 15;
#pragma unroll
  for (int ng = 0; ng < NG; ++ng) {
    const int hh = 16 * ng + (tid >> 4);
    if (hh >= RS) continue;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sm[w][hh][0]);
    float f[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) f[w] = fast_exp2(sm[w][hh][0] - M);  // waves without keys: exp2(-inf) = 0
    float* dst = part + (((size_t)b * H + h0 + hh) * max_splits + split) * (D + 2);
    for (int x = sub; x < D + 2; x += 16) {
      float v;
      if (x == 0) {
        v = M;
      } else {
        v = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) v += f[w] * sm[w][hh][x];
      }
      dst[x] = v;
    }
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void attn_decode_combine_kernel(const float* __restrict__ part, T* __restrict__ attn,
                                                                  int max_splits, int H, BatchView batch) {
  const int bh = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (bh >= batch.batch * H) return;
  const int b = bh / H, h = bh % H;
  const int kv_len = batch.desc[2 * b + 1] + 1;
  const int ns = (kv_len + kChunkKeys - 1) / kChunkKeys;
  const float* p = part + (size_t)bh * max_splits * (D + 2);
  // Up to kFew splits (contexts up to 8192 keys): every value the merge needs
  // is loaded before any is used, one round of load latency in all; the sums
  // run in split order, as in the general path below.
  constexpr int kFew = 8;
  if (ns <= kFew) {
    float mv[kFew], lv[kFew], av[kFew][D / 64];
#pragma unroll
    for (int s = 0; s < kFew; ++s) {
      const float* ps = p + min(s, ns - 1) * (D + 2);  // in bounds for every s (ns <= max_splits)
      mv[s] = s < ns ? ps[0] : -INFINITY;
      lv[s] = s < ns ? ps[1] : 0.f;
#pragma unroll
      for (int e = 0; e < D / 64; ++e) av[s][e] = s < ns ? ps[2 + lane + 64 * e] : 0.f;
    }
    float M = -INFINITY;
#pragma unroll
    for (int s = 0; s < kFew; ++s) M = fmaxf(M, mv[s]);
    float L = 0.f, acc[D / 64];
#pragma unroll
    for (int e = 0; e < D / 64; ++e) acc[e] = 0.f;
#pragma unroll
    for (int s = 0; s < kFew; ++s) {
      if (s >= ns) break;
      const float f = exp2f(mv[s] - M);
      L += f * lv[s];
#pragma unroll
      for (int e = 0; e < D / 64; ++e) acc[e] += f * av[s][e];
    }
    const float inv = 1.f / L;
#pragma unroll
    for (int e = 0; e < D / 64; ++e) {
      const int col = h * D + lane + 64 * e;
      const size_t o = sizeof(T) == 2 ? tiled_off(b, col, H * D) : (size_t)b * H * D + col;
      attn[o] = from_f32<T>(acc[e] * inv);
    }
    return;
  }
  // More splits: their maxima and sums are fetched one split per lane, all
  // at once, so the pass costs two rounds of load latency, not two per split.
  float M = -INFINITY;
  for (int s0 = 0; s0 < ns; s0 += 64)
    if (s0 + lane < ns) M = fmaxf(M, p[(s0 + lane) * (D + 2)]);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) M = fmaxf(M, shfl_xor(M, m));
  float L = 0.f;
  float acc[D / 64];
#pragma unroll
  for (int e = 0; e < D / 64; ++e) acc[e] = 0.f;
  for (int s0 = 0; s0 < ns; s0 += 64) {
    const int n = min(64, ns - s0);
    float f_l = 0.f, l_l = 0.f;
    if (lane < n) {
      f_l = exp2f(p[(s0 + lane) * (D + 2)] - M);
      l_l = p[(s0 + lane) * (D + 2) + 1];
    }
    // splits added in order (the same sums whatever the lane count)
#pragma unroll 4
    for (int i = 0; i < n; ++i) {
      const float* ps = p + (s0 + i) * (D + 2);
      const float f = __shfl(f_l, i, 64);
      L += f * __shfl(l_l, i, 64);
#pragma unroll
      for (int e = 0; e < D / 64; ++e) acc[e] += f * ps[2 + lane + 64 * e];
    }
  }
  const float inv = 1.f / L;
#pragma unroll
  for (int e = 0; e < D / 64; ++e) {
    const int col = h * D + lane + 64 * e;
    // bf16: the o_proj GEMM's tiled operand; fp32: row-major [B][H*D]
    const size_t o = sizeof(T) == 2 ? tiled_off(b, col, H * D) : (size_t)b * H * D + col;
    attn[o] = from_f32<T>(acc[e] * inv);
  }
}

template <typename T, int D>
hipError_t launch_split(const void* q, float* part, int max_splits, int H, const CacheView& c, const BatchView& b,
                        int units, hipStream_t s) {
  dim3 grid(c.G * ((H / c.G + 15) / 16) * units);
  attn_decode_split_kernel<T, D><<<grid, 256, 0, s>>>(reinterpret_cast<const T*>(q), part, max_splits, H, c, b);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_combine(const float* part, void* attn, int max_splits, int H, const BatchView& b, hipStream_t s) {
  const int nbh = b.batch * H;
  attn_decode_combine_kernel<T, D><<<(nbh + 3) / 4, 256, 0, s>>>(part, reinterpret_cast<T*>(attn), max_splits, H, b);
  return hipGetLastError();
}

}  // namespace

int decode_split_keys() { return kChunkKeys; }

hipError_t launch_attn_decode(DType t, const void* q, float* partial, int max_splits, int H, const CacheView& c,
                              const BatchView& b, int units, hipStream_t s) {
  if (H % c.G != 0 || H / c.G > 32) return hipErrorInvalidValue;
  if (units <= 0 || units > b.batch * max_splits) return hipErrorInvalidValue;
  if (t == DType::BF16) {
    const bf16* qb = reinterpret_cast<const bf16*>(q);
    if (H / c.G > 16) {  // 32 heads per group: both 16-head halves in one workgroup
      dim3 grid(c.G * ((H / c.G + 31) / 32) * units);
      if (c.D == 128)
        attn_decode_wave_kernel<128, 2><<<grid, 256, 0, s>>>(qb, partial, max_splits, H, c, b);
      else if (c.D == 64)
        attn_decode_wave_kernel<64, 2><<<grid, 256, 0, s>>>(qb, partial, max_splits, H, c, b);
      else
        return hipErrorInvalidValue;
    } else {
      dim3 grid(c.G * units);
      if (c.D == 128)
        attn_decode_wave_kernel<128, 1><<<grid, 256, 0, s>>>(qb, partial, max_splits, H, c, b);
      else if (c.D == 64)
        attn_decode_wave_kernel<64, 1><<<grid, 256, 0, s>>>(qb, partial, max_splits, H, c, b);
      else
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
  } else {
    if (c.D == 64) return launch_split<float, 64>(q, partial, max_splits, H, c, b, units, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attn_decode_combine(DType t, const float* partial, void* attn, int max_splits, int H, int D,
                                      const BatchView& b, hipStream_t s) {
  if (t == DType::BF16) {
    if (D == 128) return launch_combine<bf16, 128>(partial, attn, max_splits, H, b, s);
    if (D == 64) return launch_combine<bf16, 64>(partial, attn, max_splits, H, b, s);
  } else {
    if (D == 64) return launch_combine<float, 64>(partial, attn, max_splits, H, b, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace llk
