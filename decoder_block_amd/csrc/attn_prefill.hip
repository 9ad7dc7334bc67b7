// Causal grouped-query attention for prefill, flash style, on gfx950 MFMA.
//
// o[t, h] = sum_{j <= t} softmax_j(q[t,h] . k[j,g] / sqrt(D)) v[j,g] with
// g = h / (H/G) ("From Transformer to LLaMA: an overview", 1.1; "Chapter 10:
// the modern LLaMA architecture", section 6 -- K/V are broadcast to the query
// heads of their group inside the kernel, never materialised).  Keys come
// from the paged cache, so new tokens also see every cached key before them
// (absolute positions, "Chapter 10", section 7).
//
// Work split: one workgroup (8 waves = 2 per SIMD, 256 query rows, 32 per
// wave) per (sequence, KV group, block of positions).  The 256 rows are the
// R = H/G query heads of the group times 256/R positions, so every K/V tile
// staged in LDS serves all heads of the group.  Two waves per SIMD let one
// wave's softmax (exp on the transcendental unit, VALU) overlap the other
// wave's MFMAs.  Row blocks are issued latest-position first (the
// longest causal rows start first) and the KV groups of a row block sit on
// consecutive workgroup ids, i.e. one group per XCD.  A launch of at most one
// workgroup per CU instead pairs a late and an early half block of positions
// in each workgroup, so that all of them do the same causal work.
//
// Per wave, transposed formulation with 32x32 MFMAs:
//   S^T [keys x rows] = K_tile [keys x D] * Q^T        (Q resident in registers)
//   online softmax: each lane owns one query row and 32 of the 64 scores of a
//   tile; the row max needs one exchange with lane l^32 (only when the lazy
//   running max may move), the running sum none
//   O^T [D x rows]   += V_tile^T [D x keys] * P^T     (P straight from registers)
// The cache keeps V transposed per block ([D][16 keys]), so V^T tiles are
// staged with plain 16-byte copies.  K and V^T tiles go through a 4-slot LDS
// ring (XOR-swizzled 16-byte chunks), moved by the gfx950 LDS DMA
// (global_load_lds_dwordx4) three tiles ahead of the MFMAs, without passing
// through registers.  With one tile of look-ahead the DMA latency (K/V come
// from L2 or the last-level cache, at a few KB per block) stalled the loop:
// the DMAs took about 40% of the kernel's time on top of the math.
#include <math.h>

#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace llk {
namespace {

template <typename T, int D_>
struct ACfg {
  static constexpr int D = D_;
  static constexpr int CH = Chunk<T>::N;                 // elements per 16-byte chunk
  static constexpr int KT = 64;                          // keys per tile
  static constexpr int NW = 8;                           // waves per workgroup (2 per SIMD)
  static constexpr int NT = 64 * NW;
  static constexpr int RB = 1;                           // 32-row blocks per wave
  static constexpr int ROWS = NW * 32 * RB;              // query rows per workgroup
  static constexpr int CPRK = D * (int)sizeof(T) / 16;   // chunks per K (and Q) row
  static constexpr int NQ = D / (2 * CH);                // QK k-steps
  static constexpr int NDB = D / 32;                     // 32-row blocks of O^T
  static constexpr int VROW = KT * (int)sizeof(T) / 16;  // chunks per V^T row
  static constexpr int KSLOTS = KT * CPRK, VSLOTS = D * VROW;
  static constexpr int LK = KSLOTS / NT;                 // K chunks moved per thread
  static constexpr int LV = VSLOTS / NT;                 // V^T chunks moved per thread
  static constexpr int PER = LK + LV;                    // DMAs per thread per tile
  static constexpr int NST = 4;                          // LDS ring slots (tiles)
  static_assert(LK >= 1 && LV >= 1, "tile too small for the workgroup");
  static_assert(NT == 512, "the kernel's launch bounds assume 512 threads");
};

// LDS chunk slots.  K and Q rows are CPRK chunks wide: XOR with the low bits
// of the row spreads the 32 rows an MFMA fragment reads over all slots.  V^T
// rows (d) are 128 or 256 bytes: XOR with d/2 keeps neighbouring row pairs in
// different slots of a 256-byte bank window.  The swizzle is an involution
// within a row, so the same function maps logical -> physical and back.
template <int CPRK>
DEVI int k_swz(int row) { return row & (CPRK - 1) & 15; }
template <int VROW>
DEVI int v_swz(int d) { return (d >> 1) & 7; }

// Lazy rescaling (fp32 kernel): the running max of a row is only raised when
// a new score exceeds it by more than 8 in exp2 units, so unnormalised P
// stays <= 256.
constexpr float kRescaleLog2 = 8.f;
// bf16 kernel: the running max starts at 0 and rises only when a score
// exceeds it by more than kRiseLog2 (unnormalised P <= 2^32); on the first
// tile also when the row's max is below -kLowLog2 (its largest P stays a
// normal number).
constexpr float kRiseLog2 = 32.f;
constexpr float kLowLog2 = 64.f;

template <typename T, int D>
__global__ __launch_bounds__(512) void attn_prefill_f32_kernel(const T* __restrict__ q, T* __restrict__ attn,
                                                           int H, CacheView cache, BatchView batch) {
  using C = ACfg<T, D>;
  using vec = typename Chunk<T>::vec;
  __shared__ u32x4 sK[C::NST][C::KSLOTS];
  __shared__ u32x4 sV[C::NST][C::VSLOTS];

  const int G = cache.G;
  const int R = H / G;
  const int P = C::ROWS / R;  // positions per workgroup
  const int S = batch.seq_len;
  const int b = blockIdx.x / G, g = blockIdx.x % G;
  const int nrb = (S + P - 1) / P;
  const int rb = nrb - 1 - (int)blockIdx.y;
  const int seq = batch.desc[2 * b];
  const int start = batch.desc[2 * b + 1];
  const int kv_len = start + S;
  const int HD = H * D;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int hl = lane >> 5;  // lane group

  // query row j of the workgroup -> (head, sequence index); rows past the end
  // mirror the block's first row (computed, never stored)
  auto row_head = [&](int j) { return g * R + j / P; };
  auto row_sidx = [&](int j) {
    const int sidx = rb * P + j % P;
    return sidx < S ? sidx : rb * P;
  };

  const T* kpool = reinterpret_cast<const T*>(cache.k_pool);
  const T* vpool = reinterpret_cast<const T*>(cache.v_pool);
  // block-table reads are wave-uniform: through the constant address space
  // they become scalar loads, so the vector-memory counter counts DMAs only
  const __attribute__((address_space(4))) int32_t* btab =
      (const __attribute__((address_space(4))) int32_t*)(cache.block_table + (size_t)seq * cache.max_blocks);

  // this lane's query rows (one per 32-row block)
  int qpos[C::RB];
  bool active[C::RB];
  int wmax = 0, wmin = 1 << 30;
#pragma unroll
  for (int x = 0; x < C::RB; ++x) {
    const int j = wave * 32 * C::RB + 32 * x + (lane & 31);
    active[x] = rb * P + j % P < S;
    qpos[x] = start + row_sidx(j);
    wmax = max(wmax, qpos[x]);
    wmin = min(wmin, qpos[x]);
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    wmax = max(wmax, __shfl_xor(wmax, m, 64));
    wmin = min(wmin, __shfl_xor(wmin, m, 64));
  }
  // equal in every lane after the butterfly; in SGPRs the tile tests below are
  // uniform branches instead of per-element selects
  wmax = __builtin_amdgcn_readfirstlane(wmax);
  wmin = __builtin_amdgcn_readfirstlane(wmin);
  const int last_s = min(S, (rb + 1) * P) - 1;
  const int ntiles = (start + last_s) / C::KT + 1;

  // Q fragments (B operand of S^T), resident for the whole key loop
  vec qf[C::RB][C::NQ];
#pragma unroll
  for (int x = 0; x < C::RB; ++x) {
    const int j = wave * 32 * C::RB + 32 * x + (lane & 31);
    const T* qp = q + ((size_t)b * S + row_sidx(j)) * HD + (size_t)row_head(j) * D;
#pragma unroll
    for (int kk = 0; kk < C::NQ; ++kk) qf[x][kk] = load_chunk<T>(qp + (2 * kk + hl) * C::CH);
  }

  // Physical block ids of a tile's four 16-key blocks, fetched one tile ahead
  // so that the DMA addresses never wait on a fresh block-table load.
  static_assert(C::KT == 64, "four 16-key blocks per tile");
  typedef int32_t i32x4v __attribute__((ext_vector_type(4)));
  auto fetch_blocks = [&](int kt) {
    const int last = cache.max_blocks - 1;
    kt = __builtin_amdgcn_readfirstlane(kt);
    return i32x4v{btab[min(kt * 4 + 0, last)], btab[min(kt * 4 + 1, last)], btab[min(kt * 4 + 2, last)],
                  btab[min(kt * 4 + 3, last)]};
  };
  auto pick = [&](i32x4v blk, int u) {  // blk[u] with a lane-varying u, without dynamic indexing
    return u == 0 ? blk[0] : u == 1 ? blk[1] : u == 2 ? blk[2] : blk[3];
  };

  // Tile kt -> LDS stage st.  Every 16-byte slot is owned by one lane and
  // filled by the LDS DMA (global_load_lds_dwordx4: lane i of a wave lands at
  // base + 16 i).  Keys past the end of the sequence are clamped into its
  // last block, so every lane loads from an allocated block with no branch:
  // their scores are masked (every query row precedes them) and `finish`
  // zeroes their values.
  auto issue = [&](int kt, int st, i32x4v blk) {
    const int last = kv_len - 1;
#pragma unroll
    for (int i = 0; i < C::LK; ++i) {
      const int base = (wave * C::LK + i) * 64;
      const int slot = base + lane;
      const int key = slot / C::CPRK;
      const int c = (slot % C::CPRK) ^ k_swz<C::CPRK>(key);
      const int kp = min(kt * C::KT + key, last);
      const size_t bk = (size_t)pick(blk, (kp - kt * C::KT) >> 4);
      glb_dma16_to(kpool + ((bk * G + g) * 16 + (kp & 15)) * D + c * C::CH, lds_address(&sK[st][base]));
    }
#pragma unroll
    for (int i = 0; i < C::LV; ++i) {
      const int base = (wave * C::LV + i) * 64;
      const int slot = base + lane;
      const int d = slot / C::VROW;
      const int c = (slot % C::VROW) ^ v_swz<C::VROW>(d);
      const int kp = min(kt * C::KT + c * C::CH, last & ~(C::CH - 1));  // first key of this chunk
      const size_t bk = (size_t)pick(blk, (kp - kt * C::KT) >> 4);
      glb_dma16_to(vpool + ((bk * G + g) * D + d) * 16 + (kp & 15), lds_address(&sV[st][base]));
    }
  };
  // After the DMA has landed: zero the values of keys past the end (a chunk
  // that reaches past it may hold stale data of another sequence, and the
  // chunks past it hold a clamped copy).  Only the last tile has any.
  auto finish = [&](int kt, int st) {
    if ((kt + 1) * C::KT <= kv_len) return;
#pragma unroll
    for (int i = 0; i < C::LV; ++i) {
      const int slot = (wave * C::LV + i) * 64 + lane;
      const int d = slot / C::VROW;
      const int c = (slot % C::VROW) ^ v_swz<C::VROW>(d);
      const int kp = kt * C::KT + c * C::CH;
      if (kp + C::CH > kv_len) {
        vec v = __builtin_bit_cast(vec, sV[st][slot]);
#pragma unroll
        for (int e = 0; e < C::CH; ++e)
          if (kp + e >= kv_len) v[e] = from_f32<T>(0.f);
        sV[st][slot] = __builtin_bit_cast(u32x4, v);
      }
    }
  };

  // q arrives multiplied by log2(e)/sqrt(D) (QKV epilogue): scores are in exp2 units
  constexpr float scale = 1.f;
  float m_run[C::RB], l_run[C::RB];
  f32x16 o[C::RB][C::NDB];
#pragma unroll
  for (int x = 0; x < C::RB; ++x) {
    m_run[x] = -INFINITY;
    l_run[x] = 0.f;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[x][db][i] = 0.f;
  }

  // Ring: tile kt sits in slot kt % NST.  Tiles kt+1 .. kt+NST-1 are in
  // flight while tile kt computes; each thread waits for its own DMAs of a
  // tile (vmcnt: the DMAs of the tiles issued after it may stay outstanding)
  // and the barrier that ends an iteration publishes the tile to every wave
  // and frees the slot of the tile just computed.
  auto wait_tile = [&](int kt) {  // tile kt landed, for this thread's DMAs
    const int after = min(ntiles - 1, kt + C::NST - 2) - kt;  // tiles issued after kt
    if (after >= 2) wait_vmcnt<2 * C::PER>();
    else if (after == 1) wait_vmcnt<C::PER>();
    else wait_vmcnt<0>();
  };
  i32x4v blk_next = fetch_blocks(0);
#pragma unroll
  for (int t = 0; t < C::NST - 1; ++t) {
    if (t < ntiles) issue(t, t, blk_next);
    blk_next = fetch_blocks(t + 1);
  }
  wait_tile(0);
  finish(0, 0);
  __syncthreads();

  for (int kt = 0; kt < ntiles; ++kt) {
    const int st = kt % C::NST;
    const int k0 = kt * C::KT;
    if (kt + C::NST - 1 < ntiles) {  // into the slot of tile kt-1 (freed by the last barrier)
      issue(kt + C::NST - 1, (kt + C::NST - 1) % C::NST, blk_next);
      blk_next = fetch_blocks(kt + C::NST);
    }
    // the 64-key tile is consumed in two 32-key halves (fewer live registers)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int kh = k0 + 32 * kb;
      if (kh > wmax) continue;  // every row of this wave is before these keys
      // ---- S^T = K Q^T: each K fragment feeds both row blocks ----
      f32x16 sc[C::RB];
#pragma unroll
      for (int x = 0; x < C::RB; ++x)
#pragma unroll
        for (int i = 0; i < 16; ++i) sc[x][i] = 0.f;
      const int key = 32 * kb + (lane & 31);
      // all K fragments of the half are read before the first MFMA, so the
      // LDS latency is paid once per half, not once per k-step
      vec ka[C::NQ];
#pragma unroll
      for (int kk = 0; kk < C::NQ; ++kk) {
        const int c = 2 * kk + hl;
        ka[kk] = __builtin_bit_cast(vec, sK[st][key * C::CPRK + (c ^ k_swz<C::CPRK>(key))]);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kk = 0; kk < C::NQ; ++kk)
#pragma unroll
        for (int x = 0; x < C::RB; ++x) sc[x] = mfma32_chunk(sc[x], ka[kk], qf[x][kk]);
      // the V^T fragments of the half are read now: their latency hides
      // behind the softmax below
      const char* vb = reinterpret_cast<const char*>(&sV[st][0]);
      vec va[2][C::NDB][8 / C::CH];
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        // A operand: lane (row d, group hl) supplies keys 16m+4hl+{0..3} and
        // 16m+8+4hl+{0..3}, matching the keys its P registers hold.
        const int kA = 32 * kb + 16 * m + 4 * hl, kB = kA + 8;
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
          const int d = 32 * db + (lane & 31);
          auto piece = [&](int kk2) {  // 4 consecutive keys of row d
            const int byte = kk2 * (int)sizeof(T);
            return vb + (size_t)(d * C::VROW + ((byte >> 4) ^ v_swz<C::VROW>(d))) * 16 + (byte & 15);
          };
          if constexpr (sizeof(T) == 2) {
            const u32x2 lo = *reinterpret_cast<const u32x2*>(piece(kA));
            const u32x2 hi = *reinterpret_cast<const u32x2*>(piece(kB));
            va[m][db][0] = __builtin_bit_cast(vec, u32x4{lo[0], lo[1], hi[0], hi[1]});
          } else {
            va[m][db][0] = *reinterpret_cast<const vec*>(piece(kA));
            va[m][db][8 / C::CH - 1] = *reinterpret_cast<const vec*>(piece(kB));
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      // ---- online softmax (lane = one query row per block) ----
      // Only the halves that reach the diagonal of some row of this wave need
      // the causal mask; the test is wave-uniform, so the common case takes
      // the branch without any per-element compare.
      float mx[C::RB];
      bool grow = false;
      if (kh + 31 > wmin) {
#pragma unroll
        for (int x = 0; x < C::RB; ++x)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int kp = kh + 8 * (i >> 2) + 4 * hl + (i & 3);
            if (kp > qpos[x]) sc[x][i] = -INFINITY;
          }
      }
#pragma unroll
      for (int x = 0; x < C::RB; ++x) {
        float m = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) m = fmaxf(m, sc[x][i]);
        mx[x] = fmaxf(m, __shfl_xor(m, 32, 64));
        grow = grow || (mx[x] - m_run[x]) * scale > kRescaleLog2;
      }
      if (wave_any(grow)) {  // rare after the first tile
#pragma unroll
        for (int x = 0; x < C::RB; ++x) {
          const float m_new = fmaxf(m_run[x], mx[x]);
          const float alpha = fast_exp2((m_run[x] - m_new) * scale);
          l_run[x] *= alpha;
#pragma unroll
          for (int db = 0; db < C::NDB; ++db) o[x][db] *= alpha;
          m_run[x] = m_new;
        }
      }
      vec pv[C::RB][2][8 / C::CH];
#pragma unroll
      for (int x = 0; x < C::RB; ++x) {
        const float msc = m_run[x] * scale;
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = fast_exp2(fmaf(sc[x][i], scale, -msc));
          psum += p;
          pv[x][i >> 3][(i & 7) / C::CH][(i & 7) % C::CH] = from_f32<T>(p);
        }
        l_run[x] += psum;
      }

      // ---- O^T += V^T P^T: each V^T fragment feeds both row blocks ----
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int db = 0; db < C::NDB; ++db)
#pragma unroll
          for (int x = 0; x < C::RB; ++x) {
            if constexpr (sizeof(T) == 2) {
              o[x][db] = mfma32_chunk(o[x][db], va[m][db][0], pv[x][m][0]);
            } else {
              o[x][db] = mfma32_chunk(o[x][db], va[m][db][0], pv[x][m][0]);
              o[x][db] = mfma32_chunk(o[x][db], va[m][db][8 / C::CH - 1], pv[x][m][8 / C::CH - 1]);
            }
          }
    }
    if (kt + 1 < ntiles) {
      wait_tile(kt + 1);
      finish(kt + 1, (kt + 1) % C::NST);
    }
    __syncthreads();
  }

#pragma unroll
  for (int x = 0; x < C::RB; ++x) {
    if (!active[x]) continue;
    const int j = wave * 32 * C::RB + 32 * x + (lane & 31);
    const float l_tot = l_run[x] + __shfl_xor(l_run[x], 32, 64);
    const float inv = 1.f / l_tot;
    const int tok = b * S + row_sidx(j), col0 = row_head(j) * D;
    T* op = attn + (size_t)tok * HD + col0;  // fp32: row-major [B*S][H*D]
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int ig = 0; ig < 4; ++ig) {
        const int d0 = 32 * db + 8 * ig + 4 * hl;
        const f32x16& ov = o[x][db];
        if constexpr (sizeof(T) == 2) {  // bf16: the o_proj GEMM's tiled operand
          *reinterpret_cast<bf16x4*>(attn + tiled_off(tok, col0 + d0, HD)) =
              bf16x4{from_f32<bf16>(ov[4 * ig] * inv), from_f32<bf16>(ov[4 * ig + 1] * inv),
                     from_f32<bf16>(ov[4 * ig + 2] * inv), from_f32<bf16>(ov[4 * ig + 3] * inv)};
        } else {
          *reinterpret_cast<f32x4*>(op + d0) =
              f32x4{ov[4 * ig] * inv, ov[4 * ig + 1] * inv, ov[4 * ig + 2] * inv, ov[4 * ig + 3] * inv};
        }
      }
  }
}


// ---------------------------------------------------------------------------
// bf16 kernel.  Same work split and MFMA formulation as above; the loop is
// built to keep per-tile VALU work to the softmax itself:
//  * K/V tiles move through a 4-slot LDS ring by buffer LDS DMA, three tiles
//    ahead.  One DMA instruction never spans two 16-key cache blocks, so its
//    source is a per-block base held in SGPRs (from the block table, read by
//    scalar loads) plus a per-lane offset computed once.  V^T is kept in LDS
//    block by block ([4][D][16 keys], a copy of the cache layout, whose key
//    order vperm_pos makes each 16-byte half of a row one lane group's MFMA
//    operand) with the two halves swapped on rows 8..15 of every 16, which
//    keeps the fragment reads free of bank conflicts.
//  * LDS fragment addresses are per-lane bases computed once plus the slot
//    offset.
//  * q arrives scaled by log2(e)/sqrt(D), so scores come out in exp2 units.
//  * The online softmax runs per 64-key tile: both 32-key halves' S^T
//    products, one max and rescale decision per tile, then the second half's
//    exponentials overlap the first half's O^T product in the matrix core.
//    The causal mask is applied only on the tiles that reach a row's
//    diagonal (a separate copy of the tile loop).  The running max starts
//    at 0 and moves only for scores far from it, and until it moves for
//    some row of the wave the tiles take a copy of the loop that feeds the
//    scores to exp2 unshifted (32 fewer VALU instructions per tile and
//    wave: 974-990 -> 1007 TFLOP/s in the 8B layer).  P is rounded to
//    bf16 for the O^T product and the row sum adds those same bf16 values.
// ---------------------------------------------------------------------------
template <int D>
struct BCfg {
  static constexpr int KT = 64;                 // keys per tile: four 16-key cache blocks
  static constexpr int NW = 8, NT = 64 * NW;    // waves (2 per SIMD), threads
  static constexpr int ROWS = NW * 32;          // query rows per workgroup
  static constexpr int NST = 4;                 // LDS ring slots (tiles)
  static constexpr int CPRK = D / 8;            // 16-byte chunks per K row
  static constexpr int NQ = D / 16;             // QK k-steps
  static constexpr int NDB = D / 32;            // 32-row blocks of O^T
  static constexpr int PIECE = 16 * D * 2;      // bytes of one block's K (or V^T) for one KV group
  static constexpr int TILE = 4 * PIECE;        // bytes of a K (or V^T) tile
  static constexpr int SLOT = 2 * TILE;         // K tile, then V^T tile
  static constexpr int LK = TILE / 1024 / NW;   // K DMAs per thread per tile (= V DMAs)
  static constexpr int PER = 2 * LK;            // DMAs per thread per tile
  static_assert(LK >= 1 && PIECE % 1024 == 0, "one DMA instruction per 1 KB, inside one block");
  static_assert(NST * SLOT <= 160 * 1024, "LDS");
};

template <int D>
__global__ __launch_bounds__(512) void attn_prefill_bf16_kernel(const bf16* __restrict__ q, bf16* __restrict__ attn,
                                                                int H, CacheView cache, BatchView batch,
                                                                int paired) {
  using C = BCfg<D>;
  __shared__ u32x4 ring[C::NST * C::SLOT / 16];

  const int G = cache.G;
  const int R = H / G;
  const int P = C::ROWS / R;  // positions per workgroup
  const int S = batch.seq_len;
  const int b = blockIdx.x / G, g = blockIdx.x % G;
  const int seq = batch.desc[2 * b];
  const int start = batch.desc[2 * b + 1];
  const int kv_len = start + S;
  const int HD = H * D;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5, l32 = lane & 31;

  // query row j of the workgroup -> (head, sequence index); rows past the end
  // mirror a row of the workgroup that exists (computed, never stored).
  // Plain: the workgroup takes the P positions of block rb of its R heads.
  // Paired (for launches of at most one workgroup per CU, where the longest
  // causal row block would set the time): the sequence is cut into half
  // blocks of P/2 positions, and workgroup y takes half block nhb-1-y on
  // waves 0-3 and half block y on waves 4-7, so every workgroup does the
  // same causal work; once the short half is done, each SIMD runs one wave.
  const int j = wave * 32 + l32;
  int head, pidx, last_s, first_s;
  bool active;
  if (!paired) {
    const int nrb = (S + P - 1) / P;
    const int rb = nrb - 1 - (int)blockIdx.y;
    head = g * R + j / P;
    pidx = rb * P + j % P;
    active = pidx < S;
    first_s = rb * P;
    last_s = min(S, (rb + 1) * P) - 1;
  } else {
    const int HP = P / 2, nhb = (S + HP - 1) / HP;
    const int hb_long = nhb - 1 - (int)blockIdx.y, hb_short = (int)blockIdx.y;
    const int half = j / (C::ROWS / 2), jj = j % (C::ROWS / 2);
    head = g * R + jj / HP;
    pidx = (half ? hb_short : hb_long) * HP + jj % HP;
    active = pidx < S && !(half && hb_short == hb_long);  // odd nhb: the middle half block once
    first_s = hb_long * HP;
    last_s = min(S, (hb_long + 1) * HP) - 1;
  }
  const int sidx = active ? pidx : first_s;
  const int qpos = start + sidx;
  int wmax = qpos, wmin = qpos;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    wmax = max(wmax, __shfl_xor(wmax, m, 64));
    wmin = min(wmin, __shfl_xor(wmin, m, 64));
  }
  wmax = __builtin_amdgcn_readfirstlane(wmax);
  wmin = __builtin_amdgcn_readfirstlane(wmin);
  const int ntiles = (start + last_s) / C::KT + 1;

  // Q fragments (B operand of S^T), resident for the whole key loop
  bf16x8 qf[C::NQ];
  {
    const bf16* qp = q + ((size_t)b * S + sidx) * HD + (size_t)head * D;
#pragma unroll
    for (int kk = 0; kk < C::NQ; ++kk) qf[kk] = load_chunk<bf16>(qp + (2 * kk + hl) * 8);
  }
  // The Q loads complete here, before the first DMA: the compiler does not
  // see the DMAs (inline assembly), and a Q load it still believed pending
  // would make it wait on the vector-memory counter inside the loop, which
  // would drain the DMAs of the tiles in flight.
  wait_vmcnt<0>();

  // ---- DMA plan (per thread, fixed for all tiles) ----
  // K DMA i: 16-byte LDS slot (wave * LK + i) * 64 + lane of the K tile =
  // row `key`, physical chunk p holding logical chunk p ^ (key & (CPRK-1));
  // V DMA i: byte (wave * LK + i) * 1024 + 16 * lane of the V^T tile.
  // Every DMA of a wave touches the same 16-key block of the tile, block
  // wave / 2 (8 waves x PER KB cover the 4 blocks' K and V^T pieces in order).
  static_assert(C::NW == 8 && C::PIECE == 2 * C::LK * 1024, "two waves per 16-key block");
  const int my_u = wave >> 1;
  int koff[C::LK], voff[C::LK], vchk[C::LK];
#pragma unroll
  for (int i = 0; i < C::LK; ++i) {
    const int qd = wave * C::LK + i;
    const int slot = qd * 64 + lane;
    const int key = slot / C::CPRK, p = slot % C::CPRK;
    const int c = p ^ (key & (C::CPRK - 1));
    koff[i] = (key & 15) * D * 2 + c * 16;
    const int byte = qd * 1024 + lane * 16;
    const int o = byte % C::PIECE, d = o >> 5, vp = (o >> 4) & 1, vc = vp ^ ((d >> 3) & 1);
    voff[i] = d * 32 + vc * 16;
    vchk[i] = vc;  // row half: keys 4vc..4vc+3 and 8+4vc..8+4vc+3 of block my_u
  }
  const char* kpool = reinterpret_cast<const char*>(cache.k_pool);
  const char* vpool = reinterpret_cast<const char*>(cache.v_pool);
  // block-table reads are wave-uniform: through the constant address space
  // they become scalar loads, so the vector-memory counter counts DMAs only
  const __attribute__((address_space(4))) int32_t* btab =
      (const __attribute__((address_space(4))) int32_t*)(cache.block_table + (size_t)seq * cache.max_blocks);
  const uint32_t ring_lds = lds_address(ring);
  // The physical block this wave moves for tile kt; blocks past the
  // sequence's last one are replaced by it (their keys are masked and their
  // values zeroed).  Read one tile ahead of its use.
  auto block_of = [&](int kt) {
    const int ulast = ((kv_len - 1) >> 4) - kt * 4;
    return btab[kt * 4 + min(my_u, ulast)];
  };
  auto issue = [&](int st, int32_t bk) {
    const uint32_t base = ring_lds + (uint32_t)(st * C::SLOT);
    const size_t piece = ((size_t)bk * G + g) * C::PIECE;
    const i32x4 rk = make_rsrc(kpool + piece, C::PIECE), rv = make_rsrc(vpool + piece, C::PIECE);
#pragma unroll
    for (int i = 0; i < C::LK; ++i) buf_dma16_to(rk, base + (uint32_t)((wave * C::LK + i) * 1024), koff[i]);
#pragma unroll
    for (int i = 0; i < C::LK; ++i)
      buf_dma16_to(rv, base + (uint32_t)(C::TILE + (wave * C::LK + i) * 1024), voff[i]);
  };
  // After the DMA has landed: zero the values of keys past the end (only the
  // last tile has any); each thread fixes the chunks its own DMAs wrote.
  auto finish = [&](int kt, int st) {
    if ((kt + 1) * C::KT <= kv_len) return;
    u32x4* vt = ring + (st * C::SLOT + C::TILE) / 16;
#pragma unroll
    for (int i = 0; i < C::LK; ++i) {
      const int k0 = kt * C::KT + 16 * my_u + 4 * vchk[i];  // element e holds key k0 + e + 4 (e >= 4)
      if (k0 + 12 > kv_len) {
        const int idx = (wave * C::LK + i) * 64 + lane;
        bf16x8 v = __builtin_bit_cast(bf16x8, vt[idx]);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (k0 + e + (e & 4) >= kv_len) v[e] = from_f32<bf16>(0.f);
        vt[idx] = __builtin_bit_cast(u32x4, v);
      }
    }
  };
  auto wait_tile = [&](int kt) {  // tile kt landed, for this thread's DMAs
    const int after = min(ntiles - 1, kt + C::NST - 2) - kt;  // tiles issued after kt
    if (after >= 2) wait_vmcnt<2 * C::PER>();
    else if (after == 1) wait_vmcnt<C::PER>();
    else wait_vmcnt<0>();
  };

  // ---- fragment addresses (bytes from the slot base) ----
  // K (A operand of S^T): key l32 of the half, chunk 2kk + hl
  int kaddr[C::NQ];
#pragma unroll
  for (int kk = 0; kk < C::NQ; ++kk)
    kaddr[kk] = l32 * C::CPRK * 16 + (((2 * kk + hl) ^ (l32 & (C::CPRK - 1))) * 16);
  // V^T (A operand of O^T): row d = 32 db + l32 of block 2kb + m; lane group
  // hl takes row half hl (keys 4hl..4hl+3 and 8+4hl..8+4hl+3, the keys its
  // P registers hold)
  const int vaddr = C::TILE + l32 * 32 + ((hl ^ ((l32 >> 3) & 1)) * 16);

  // m_run: the row's running max in exp2 units, raised lazily (below).  It
  // starts at 0 and stays there while the row's first-tile max lies in
  // [-kLowLog2, kRiseLog2] and no later score exceeds kRiseLog2; while every
  // row of the wave has m_run = 0 the tiles take a copy that feeds the scores
  // to exp2 with no subtraction.  `shifted` (wave-uniform) is set once some
  // row's m_run moved.
  float m_run = 0.f, l_run = 0.f;
  bool first = true, shifted = false;
  f32x16 o[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.f;

  // Ring: tile kt sits in slot kt % NST; tiles kt+1 .. kt+NST-1 are in flight
  // while tile kt computes.  The barrier ending an iteration publishes tile
  // kt+1 to every wave and frees the slot of tile kt.
#pragma unroll
  for (int t = 0; t < C::NST - 1; ++t)
    if (t < ntiles) issue(t, block_of(t));
  int32_t bk_next = block_of(min(C::NST - 1, ntiles - 1));
  wait_tile(0);
  finish(0, 0);
  __syncthreads();

  // One 64-key tile of the online softmax.  Both 32-key halves' S^T products
  // are issued back to back; the running max is checked once per tile; then
  // the exponentials of the second half run while the first half's O^T
  // product is in the matrix core.  The whole tile is one straight-line block
  // apart from the rare rescale, so the compiler can interleave one half's
  // VALU work with the other half's MFMAs.  Only tiles that reach a row's
  // diagonal (DIAG) apply the causal mask.
  const char* lds = reinterpret_cast<const char*>(ring);
  const bf16x2 ones2 = {from_f32<bf16>(1.f), from_f32<bf16>(1.f)};
  auto tile = [&](const char* sb, int k0, auto diag_, auto shift_) {
    constexpr bool DIAG = decltype(diag_)::value;
    constexpr bool SHIFT = decltype(shift_)::value;  // some row of the wave has m_run != 0
    auto kfrag = [&](int kb, int kk) {
      return *reinterpret_cast<const bf16x8*>(sb + kaddr[kk] + kb * 32 * C::CPRK * 16);
    };
    auto vfrag = [&](int kb, int m, int db) {
      return *reinterpret_cast<const bf16x8*>(sb + vaddr + (2 * kb + m) * C::PIECE + db * 32 * 32);
    };
    auto start = [&](int) {  // the accumulator S^T starts from
      f32x16 init;
#pragma unroll
      for (int i = 0; i < 16; ++i) init[i] = 0.f;
      return init;
    };
    // causal mask on tiles that reach a row's diagonal: scores of keys after
    // the row's position are replaced (not added to: the K rows of positions
    // past the sequence's end hold whatever the pool held, possibly NaN bits)
    auto mask = [&](f32x16& sc, int kb) {
      if constexpr (DIAG) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kp = k0 + 32 * kb + 8 * (i >> 2) + 4 * hl + (i & 3);
          if (kp > qpos) sc[i] = -INFINITY;
        }
      }
    };
    // stage 1: K fragments of the first half
    bf16x8 ka[C::NQ], kb1[C::NQ];
#pragma unroll
    for (int kk = 0; kk < C::NQ; ++kk) ka[kk] = kfrag(0, kk);
    __builtin_amdgcn_sched_barrier(0);
    // stage 2: S^T of the first half || K fragments of the second half
    f32x16 sc0 = mfma32_chunk(start(0), ka[0], qf[0]);
#pragma unroll
    for (int kk = 1; kk < C::NQ; ++kk) sc0 = mfma32_chunk(sc0, ka[kk], qf[kk]);
#pragma unroll
    for (int kk = 0; kk < C::NQ; ++kk) kb1[kk] = kfrag(1, kk);
#pragma unroll
    for (int kk = 0; kk < C::NQ; ++kk) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
    }
    __builtin_amdgcn_sched_barrier(0);
    // stage 3: S^T of the second half || max of the first half
    // (scores are in exp2 units: q arrives scaled by log2(e)/sqrt(D))
    f32x16 sc1 = mfma32_chunk(start(1), kb1[0], qf[0]);
#pragma unroll
    for (int kk = 1; kk < C::NQ; ++kk) sc1 = mfma32_chunk(sc1, kb1[kk], qf[kk]);
    mask(sc0, 0);
    float mx = sc0[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sc0[i]);
#pragma unroll
    for (int kk = 0; kk < C::NQ; ++kk) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // VALU
    }
    __builtin_amdgcn_sched_barrier(0);
    // stage 4: V^T fragments of the first half (their latency hides behind
    // the rest of the softmax), then the online softmax: lane = one query row,
    // 32 of the tile's 64 keys
    bf16x8 va0[2][C::NDB];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) va0[m][db] = vfrag(0, m, db);
    mask(sc1, 1);
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc1[i]);
    // the running max m is raised lazily: only when a score exceeds it by
    // more than kRiseLog2 (so unnormalised P stays <= 2^32, and the sums of
    // P and of P V stay far inside fp32), or, on the first tile, when the
    // row's max lies outside [-kLowLog2, kRiseLog2] (so that the largest P of
    // every row is a normal number); the final division uses the same stale
    // max, so the result is exact.  The bf16 rounding of P is relative, so
    // the shift does not change its precision.
    // mx is this lane's half of the row (32 keys).  A row whose max passes
    // a bound has a half whose max passes it (the low bound: both halves),
    // so the halves are tested alone, and the row max over both halves
    // (lane l ^ 32) is taken only in the rare branch, where it decides.
    const bool grow_half = first ? (mx > kRiseLog2 || mx < -kLowLog2) : mx - m_run > kRiseLog2;
    if (wave_any(grow_half)) {
      mx = max_lane_halves(mx, hl);
      const bool grow = first ? (mx > kRiseLog2 || mx < -kLowLog2) : mx - m_run > kRiseLog2;
      const float m_new = grow ? mx : m_run;
      const float alpha = first ? 0.f : fast_exp2(m_run - m_new);  // first tile: o and l are 0
      if constexpr (!SHIFT) {  // m_run was 0: this tile's exponents are s - m_new
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          sc0[i] -= m_new;
          sc1[i] -= m_new;
        }
      }
      m_run = m_new;
      shifted = shifted || wave_any(m_run != 0.f);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) o[db] *= alpha;
    }
    first = false;
    // P in bf16 (the O^T product's operand); the row sum adds the same bf16
    // values, so O / l is a weighted mean of V with weights summing to one
    auto expo = [&](float sv) { return SHIFT ? sv - m_run : sv; };
    bf16x8 p0[2], p1[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) p0[i >> 3][i & 7] = from_f32<bf16>(fast_exp2(expo(sc0[i])));
    __builtin_amdgcn_sched_barrier(0);
    // stage 5: O^T += V^T P^T for the first half || exponentials of the second
    // half, V^T fragments of the second half
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) o[db] = mfma32_chunk(o[db], va0[m][db], p0[m]);
    bf16x8 va1[2][C::NDB];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) va1[m][db] = vfrag(1, m, db);
#pragma unroll
    for (int i = 0; i < 16; ++i) p1[i >> 3][i & 7] = from_f32<bf16>(fast_exp2(expo(sc1[i])));
#pragma unroll
    for (int kk = 0; kk < 2 * C::NDB; ++kk) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // VALU
    }
    __builtin_amdgcn_sched_barrier(0);
    // stage 6: O^T += V^T P^T for the second half || row sums
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) o[db] = mfma32_chunk(o[db], va1[m][db], p1[m]);
    float psum = 0.f;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        psum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{p0[m][2 * e], p0[m][2 * e + 1]}, ones2, psum, false);
        psum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{p1[m][2 * e], p1[m][2 * e + 1]}, ones2, psum, false);
      }
    l_run += psum;
#pragma unroll
    for (int kk = 0; kk < 2 * C::NDB; ++kk) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // VALU
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // One iteration of the tile loop: the next DMA into the freed slot, the
  // tile (skipped when it is past every row of this wave), then the wait for
  // the next tile and the barrier that publishes it.
  auto step = [&](int kt, auto diag, auto shift) {
    const int st = kt % C::NST;
    const int k0 = kt * C::KT;
    if (kt + C::NST - 1 < ntiles) {
      issue((kt + C::NST - 1) % C::NST, bk_next);
      bk_next = block_of(min(kt + C::NST, ntiles - 1));
    }
    if (k0 <= wmax) tile(lds + st * C::SLOT, k0, diag, shift);
    if (kt + 1 < ntiles) {
      wait_tile(kt + 1);
      finish(kt + 1, (kt + 1) % C::NST);
    }
    __syncthreads();
  };
  // Tiles up to the first one holding a key after some row of this wave need
  // no mask; from there on every tile takes the masked path (keys past the
  // sequence's end are after every row, so the last tile is always masked).
  // Two loops rather than a branch per tile: each holds one copy of the tile,
  // which keeps the register allocation of each free of the other.
  const int kt_diag = min(ntiles, wmin >= C::KT - 1 ? (wmin - (C::KT - 1)) / C::KT + 1 : 0);
  int kt = 0;
  // (and a loop without the shift by m_run until some row's m_run moves)
  for (; kt < kt_diag && !shifted; ++kt) step(kt, std::false_type{}, std::false_type{});
  for (; kt < kt_diag; ++kt) step(kt, std::false_type{}, std::true_type{});
  for (; kt < ntiles && !shifted; ++kt) step(kt, std::true_type{}, std::false_type{});
  for (; kt < ntiles; ++kt) step(kt, std::true_type{}, std::true_type{});

  if (!active) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.f / l_tot;
  const int tok = b * S + sidx, col0 = head * D;
#pragma unroll
  for (int db = 0; db < C::NDB; ++db)
#pragma unroll
    for (int ig = 0; ig < 4; ++ig) {
      const int d0 = 32 * db + 8 * ig + 4 * hl;
      // the o_proj GEMM's operand: tiled bf16
      *reinterpret_cast<bf16x4*>(attn + tiled_off(tok, col0 + d0, HD)) =
          bf16x4{from_f32<bf16>(o[db][4 * ig] * inv), from_f32<bf16>(o[db][4 * ig + 1] * inv),
                 from_f32<bf16>(o[db][4 * ig + 2] * inv), from_f32<bf16>(o[db][4 * ig + 3] * inv)};
    }
}

// Compute units of the current device (the launch shape below depends on
// whether a launch fills them more than once).
int cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) !=
                                               hipSuccess || n <= 0)
    return 256;
  return n;
}

template <typename T, int D>
hipError_t launch_d(const void* q, void* attn, int H, const CacheView& c, const BatchView& b, hipStream_t s) {
  const int R = H / c.G;
  const int P = ACfg<T, D>::ROWS / R;
  static_assert(ACfg<T, D>::ROWS == BCfg<D>::ROWS, "same rows per workgroup");
  const int nrb = (b.seq_len + P - 1) / P;
  if constexpr (sizeof(T) == 2) {
    // one workgroup per CU at a time: a launch within one round takes the
    // paired row blocks (equal causal work per workgroup)
    const bool paired = nrb > 1 && c.G * b.batch * nrb <= cu_count();
    const int HP = P / 2;
    dim3 grid(c.G * b.batch, paired ? ((b.seq_len + HP - 1) / HP + 1) / 2 : nrb);
    attn_prefill_bf16_kernel<D><<<grid, BCfg<D>::NT, 0, s>>>(reinterpret_cast<const bf16*>(q),
                                                             reinterpret_cast<bf16*>(attn), H, c, b, paired ? 1 : 0);
  } else {
    dim3 grid(c.G * b.batch, nrb);
    attn_prefill_f32_kernel<T, D><<<grid, ACfg<T, D>::NT, 0, s>>>(reinterpret_cast<const T*>(q),
                                                                  reinterpret_cast<T*>(attn), H, c, b);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_prefill(DType t, const void* q, void* attn, int H, const CacheView& c, const BatchView& b,
                               hipStream_t s) {
  if (H % c.G != 0 || 64 % (H / c.G) != 0) return hipErrorInvalidValue;
  if (t == DType::BF16) {
    if (c.D == 128) return launch_d<bf16, 128>(q, attn, H, c, b, s);
    if (c.D == 64) return launch_d<bf16, 64>(q, attn, H, c, b, s);
  } else {
    if (c.D == 64) return launch_d<float, 64>(q, attn, H, c, b, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace llk
