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
// Tiles: BN features x BM tokens per workgroup, K staged 64 bytes per row
// (32 bf16 / 16 fp32) through a 4-deep LDS ring with an XOR swizzle of the
// 16-byte chunk index.  Stages are moved by the buffer LDS DMA (buffer_load
// ... lds, no register staging) three stages ahead of the MFMAs; each stage
// waits only for its own DMAs (s_waitcnt vmcnt) and one barrier, and LDS
// reads never wait for the DMAs of other stages.  The workgroup -> tile map
// keeps the tiles that share weight panels on one XCD (8 XCDs, each with its
// own L2).
//
// bf16 operands are stored in 64-byte rows of 32 columns: the activations the
// layer writes for a GEMM in 256-row x 32-column tiles (tiled_off), the packed
// weights K block first (wtiled_off, w_rows rows per K block).  A stage of a
// tile is then one contiguous piece of 64-byte rows, and its DMAs fetch whole
// 128-byte lines.  With row-major operands a 32-deep stage touches half of
// every line of its rows, and the DMA stream into LDS was measured at about
// 60% of the rate for whole lines; that stream set the GEMMs' speed.
#include "common.h"
#include "kernels.h"
#include <algorithm>
#include <type_traits>

namespace llk {
namespace {

template <typename T, int BN_, int BM_, int WN_, int WM_>
struct Cfg {
  static constexpr int BN = BN_, BM = BM_, WN = WN_, WM = WM_;
  static constexpr int NT = 64 * WN * WM;
  static constexpr int CPR = 4;     // 16-byte chunks per tile row and stage (64 bytes of K)
  static constexpr int NSTAGE = 4;  // LDS ring depth
  static constexpr int BK = CPR * Chunk<T>::N;
  static constexpr int FW = BN / WN, TW = BM / WM;
  static constexpr int FI = FW / 16, TJ = TW / 16;
  static constexpr int LW = BN * CPR / NT, LX = BM * CPR / NT;  // 16-byte DMAs per thread per stage
  static_assert(LW * NT == BN * CPR && LX * NT == BM * CPR && LW >= 1 && LX >= 1, "tile must split evenly");
  static_assert(FW % 16 == 0 && TW % 16 == 0, "wave tile must be 16-aligned");
};

// 16-byte slot of (row, chunk) in a stage: XOR with row/4 spreads the 16 rows
// a fragment reads over all four slots of each 64-byte row group.
DEVI int swz(int row, int c) { return row * 4 + (c ^ ((row >> 2) & 3)); }

// z * sigmoid(z) with the hardware exp2 and reciprocal (about 1 ulp each)
DEVI float silu(float z) { return z * fast_rcp(1.f + fast_exp2(-1.4426950408889634f * z)); }

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

// RoPE on two interleaved pairs (e, o) = (v0, v1), (v2, v3) at position pos,
// pair index dd/2 and dd/2 + 1 of the head ("Chapter 10", section 3)
DEVI f32x4 rotate4(f32x4 v, f32x2 cs, f32x2 sn) {
  const float e0 = v[0], o0 = v[1], e1 = v[2], o1 = v[3];
  return f32x4{e0 * cs[0] - o0 * sn[0], e0 * sn[0] + o0 * cs[0], e1 * cs[1] - o1 * sn[1], e1 * sn[1] + o1 * cs[1]};
}
DEVI f32x4 rope4(f32x4 v, const GemmArgs& a, int pos, int dd) {
  const int D = a.cache.D;
  const f32x2 cs = *reinterpret_cast<const f32x2*>(a.rope_cos + (size_t)pos * (D / 2) + dd / 2);
  const f32x2 sn = *reinterpret_cast<const f32x2*>(a.rope_sin + (size_t)pos * (D / 2) + dd / 2);
  return rotate4(v, cs, sn);
}
DEVI float q_scale(int D) { return 1.4426950408889634f * __frsqrt_rn((float)D); }

// Rotated q or k values of features dd..dd+3 of one head, to the head's first
// element `head`.  Interleaved RoPE: in place.  Half-split RoPE: the packed
// rows of the head were reordered so that pair i = (i, i + D/2) sits in rows
// 2i, 2i+1; (v0, v2) go back to positions dd/2, dd/2 + 1 and (v1, v3) to
// dd/2 + D/2, dd/2 + D/2 + 1.
template <typename T>
DEVI void store_head4(T* head, int dd, f32x4 v, int half_split, int D) {
  if (!half_split) {
    store4(head + dd, v[0], v[1], v[2], v[3]);
    return;
  }
  T* lo = head + dd / 2;
  T* hi = lo + D / 2;
  if constexpr (sizeof(T) == 4) {
    *reinterpret_cast<f32x2*>(lo) = f32x2{v[0], v[2]};
    *reinterpret_cast<f32x2*>(hi) = f32x2{v[1], v[3]};
  } else {
    *reinterpret_cast<bf16x2*>(lo) = bf16x2{from_f32<bf16>(v[0]), from_f32<bf16>(v[2])};
    *reinterpret_cast<bf16x2*>(hi) = bf16x2{from_f32<bf16>(v[1]), from_f32<bf16>(v[3])};
  }
}

// RMSNorm row scale of token t: precomputed, or from the per-segment sums of
// squares that a folded norm pass left (added in segment order).
DEVI float row_scale(const GemmArgs& a, int t) {
  if (a.ss_part == nullptr) return a.rowscale[t];
  const float* p = a.ss_part + (size_t)t * a.ss_nseg;
  float acc = 0.f;
  for (int i = 0; i < a.ss_nseg; ++i) acc += p[i];
  return 1.f / sqrtf(acc / (float)a.ss_d + a.eps);
}

// Epilogue for one lane-quad: token t, features f .. f+3, accumulator v.
template <typename T, int EPI>
DEVI void epilogue(const GemmArgs& a, int t, int f, f32x4 v) {
  if constexpr (EPI == (int)Epi::QKV) {
    const float r = row_scale(a, t);
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
      v = rope4(v, a, pos, dd);
    }
    if (f < HD) {
      // q is stored pre-multiplied by log2(e)/sqrt(D), so the attention kernels'
      // scores come out in exp2 units (scaled in fp32, then rounded once)
      v *= q_scale(D);
      const int dd = f % D;
      store_head4(reinterpret_cast<T*>(a.q_out) + (size_t)t * HD + (f - dd), dd, v, a.rope_half, D);
    } else {
      const bool is_k = f < HD + KD;
      const int kf = is_k ? f - HD : f - HD - KD;
      const int g = kf / D, dd = kf - g * D;
      const size_t blk = (size_t)a.cache.block_table[(size_t)seq * a.cache.max_blocks + (pos >> 4)];
      if (is_k) {  // K block [16 slots][D]
        T* row = reinterpret_cast<T*>(a.cache.k_pool) + ((blk * G + g) * 16 + (pos & 15)) * D;
        store_head4(row, dd, v, a.rope_half, D);
      } else {     // V block kept transposed: [D][16 slots] (bf16: keys in vperm_pos order)
        const int slot = sizeof(T) == 2 ? vperm_pos(pos & 15) : (pos & 15);
        T* dst = reinterpret_cast<T*>(a.cache.v_pool) + ((blk * G + g) * D + dd) * 16 + slot;
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
    const float r = row_scale(a, t);
    v *= r;
    const float s0 = silu(v[0]) * v[1];
    const float s1 = silu(v[2]) * v[3];
    // s columns f/2, f/2 + 1 (f/2 even: one tile row of the down GEMM's operand)
    T* o = reinterpret_cast<T*>(a.out) +
           (sizeof(T) == 2 ? tiled_off(t, f / 2, a.ldo) : (size_t)t * a.ldo + f / 2);
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
  // One LDS array per ring slot (the slot's W rows, then its X rows).  With
  // distinct arrays the compiler can tell that a fragment read of one slot
  // does not depend on DMAs still landing in the others, and so does not
  // drain them before the read.
  static_assert(C::NSTAGE == 4, "four ring slots");
  constexpr int SLOT = (C::BN + C::BM) * C::CPR;
  __shared__ u32x4 L0[SLOT];
  __shared__ u32x4 L1[SLOT];
  __shared__ u32x4 L2[SLOT];
  __shared__ u32x4 L3[SLOT];

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
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wn = wave % C::WN, wm = wave / C::WN;

  // Global -> LDS by buffer DMA: lane i of a wave fills slot base + i.  Slot s
  // of a stage holds logical chunk (s % 4) ^ swizzle(row) of row s / 4, so the
  // lane loads exactly that chunk (the swizzle is its own inverse).  Rows of X
  // past M fall outside the buffer's range and arrive as zeros.
  constexpr int ES = (int)sizeof(T);
  // bf16 operands: a stage of BN (BM) rows is one contiguous piece of 64-byte
  // rows, the next stage w_rows * 64 bytes further for W (K-block-major) and
  // 16 KB further for X (256 x 32 tiles).  fp32 operands are row-major with
  // pitch K (W) and ldx (X).
  constexpr bool TILED = sizeof(T) == 2;
  int vW[C::LW], vX[C::LX];
#pragma unroll
  for (int i = 0; i < C::LW; ++i) {
    const int slot = (wave * C::LW + i) * 64 + lane;
    const int row = slot >> 2, c = (slot & 3) ^ ((row >> 2) & 3);
    vW[i] = TILED ? row * 64 + c * 16 : (row * a.K + c * Chunk<T>::N) * ES;
  }
#pragma unroll
  for (int i = 0; i < C::LX; ++i) {
    const int slot = (wave * C::LX + i) * 64 + lane;
    const int row = slot >> 2, c = (slot & 3) ^ ((row >> 2) & 3);
    vX[i] = TILED ? row * 64 + c * 16 : (row * a.ldx + c * Chunk<T>::N) * ES;
  }
  const char* Wt = reinterpret_cast<const char*>(a.W) + (TILED ? (size_t)n0 * 64 : (size_t)n0 * a.K * ES);
  const char* Xt = reinterpret_cast<const char*>(a.X) +
                   (TILED ? tiled_off(m0, 0, a.K) * ES : (size_t)m0 * a.ldx * ES);
  // bytes of X from the tile's first row to the end of the matrix (< 2^31 for
  // every supported shape), kept wave-uniform so the descriptor lives in SGPRs;
  // tiled X holds whole 256-row tiles, so a stage never reads past them
  const uint64_t xb = TILED ? (uint64_t)C::BM * 64 : (uint64_t)(a.M - m0) * (uint64_t)a.ldx * ES;
  const int x_bytes = __builtin_amdgcn_readfirstlane((int)(xb < 0x7fffffffull ? xb : 0x7fffffffull));
  const int nk = a.K / C::BK;
  constexpr int STAGE_BYTES = TILED ? kTileElems * 2 : C::BK * ES;  // distance between X stages
  const size_t w_stage = TILED ? (size_t)a.w_rows * 64 : (size_t)STAGE_BYTES;  // ... and W stages

  auto slot_of = [&](auto s_) -> u32x4* {
    constexpr int S = decltype(s_)::value & 3;
    if constexpr (S == 0) return L0;
    else if constexpr (S == 1) return L1;
    else if constexpr (S == 2) return L2;
    else return L3;
  };
  // Stages past the end are issued against an empty buffer (zero records):
  // they move no memory but keep the DMA count per stage uniform, so every
  // stage waits with the same count.
  auto issue = [&](int kt, u32x4* L) {
    const bool live = kt < nk;
    const int kb = live ? kt * STAGE_BYTES : 0;
    const i32x4 rW = make_rsrc(Wt + (live ? kt * w_stage : 0), live ? (TILED ? (uint32_t)C::BN * 64 : 0x7fffffffu) : 0u);
    const i32x4 rX = make_rsrc(Xt + kb, live ? (uint32_t)(TILED ? x_bytes : x_bytes - kb) : 0u);
#pragma unroll
    for (int i = 0; i < C::LW; ++i) buf_dma16_async(rW, L + (wave * C::LW + i) * 64, vW[i]);
#pragma unroll
    for (int i = 0; i < C::LX; ++i) buf_dma16_async(rX, L + C::BN * C::CPR + (wave * C::LX + i) * 64, vX[i]);
  };
  constexpr int PER = C::LW + C::LX;  // DMAs per thread per stage

  f32x4 acc[C::FI][C::TJ];
#pragma unroll
  for (int i = 0; i < C::FI; ++i)
#pragma unroll
    for (int j = 0; j < C::TJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int l16 = lane & 15, lg = lane >> 4;
  // Stage kt in ring slot kt & 3: it has landed once at most this wave's DMAs
  // of stages kt+1 and kt+2 are outstanding; after the barrier every wave's
  // part is in LDS and every wave is done with stage kt-1, whose slot takes
  // stage kt+3.  One 32-deep k-step per stage: lane group lg reads chunk lg.
  auto stage = [&](int kt, auto s_) {
    using S = decltype(s_);
    wait_vmcnt<2 * PER>();
    lds_barrier();
    issue(kt + 3, slot_of(std::integral_constant<int, S::value + 3>{}));
    const u32x4* L = slot_of(s_);
    vec af[C::FI], bf[C::TJ];
#pragma unroll
    for (int i = 0; i < C::FI; ++i) af[i] = __builtin_bit_cast(vec, L[swz(wn * C::FW + 16 * i + l16, lg)]);
#pragma unroll
    for (int j = 0; j < C::TJ; ++j)
      bf[j] = __builtin_bit_cast(vec, L[C::BN * C::CPR + swz(wm * C::TW + 16 * j + l16, lg)]);
#pragma unroll
    for (int i = 0; i < C::FI; ++i)
#pragma unroll
      for (int j = 0; j < C::TJ; ++j) acc[i][j] = mfma16_chunk(acc[i][j], af[i], bf[j]);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;

  issue(0, L0);
  issue(1, L1);
  issue(2, L2);
  int kt = 0;
  for (; kt + 4 <= nk; kt += 4) {
    stage(kt, I0{});
    stage(kt + 1, I1{});
    stage(kt + 2, I2{});
    stage(kt + 3, I3{});
  }
  // K is a multiple of 2 * BK, so at most two stages remain (slots 0 and 1)
  if (kt < nk) {
    stage(kt, I0{});
    stage(kt + 1, I1{});
  }
  wait_vmcnt<0>();  // the (empty) DMAs issued past the end have retired

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

// ---------------------------------------------------------------------------
// Large bf16 tiles: 256 features x BM tokens (BM 256 or 128), four waves (one
// per SIMD) as 2 x 2, each wave 128 features x BM/2 tokens as 8 x BM/32
// blocks of v_mfma_f32_16x16x32_bf16 whose accumulators stay in the matrix
// core's register file.  The 16x16x32 form does the same work per fragment
// read as 32x32x16 at this wave tile, but the chip holds a higher clock
// under it (less accumulator traffic per flop), so more flops per second
// fit the same power.  BM 128 is for launches that 256 x 256 tiles would give
// fewer than two rounds of the 256 CUs (e.g. the 4096-feature projections of
// a 2048-token prefill: 128 tiles).
// K is staged 32 elements at a time (one 32-deep k-step) in a 4-slot LDS
// ring.  A stage is BM/16 slices of four MFMAs; the slices also read the
// next stage's fragments (in the order the MFMAs consume them) and issue the
// DMAs of stage kt+3, so with a single wave per SIMD the matrix core does not
// wait for LDS:
//   wait for this wave's DMAs of stage kt+1, barrier (every wave is done
//   with stage kt-1);
//   MFMAs of stage kt || reads of stage kt+1 || DMAs of stage kt+3 into
//   stage kt-1's slot.
// 16x16 result layout: lane l holds token (l & 15) and features
// 4(l >> 4) + {0..3} of its 16-feature block: a lane-local group of four
// consecutive features, so the same epilogues apply.
// ---------------------------------------------------------------------------
template <int BM_>
struct BigCfg {
  static constexpr int BN = 256, BM = BM_, NT = 256, CPR = 4, NS = 4, BK = 32;
  static constexpr int TW = BM / 2;                 // tokens per wave
  static constexpr int FI = 8;                      // 16-feature MFMA blocks per wave
  static constexpr int TJ = TW / 16;                // 16-token MFMA blocks per wave
  static constexpr int NF = FI + TJ;                // fragments per stage: 8 of W, TJ of X
  static constexpr int NSL = FI * TJ / 4;           // slices of four MFMAs per stage
  static constexpr int PER = (BN + BM) * CPR / NT;  // DMAs per thread per stage
  static constexpr int SLOT = (BN + BM) * CPR;      // 16-byte chunks per slot
  static constexpr int HALVES = BM / 128;           // 128-token passes of the staged epilogues
  // LDS: the ring, which the epilogues reuse to stage 128 tokens x 256 fp32
  // features (128 KB) at a time
  static constexpr int LDS_CHUNKS = NS * SLOT > 128 * 64 ? NS * SLOT : 128 * 64;
  static_assert(BM == 256 || BM == 128, "256 or 128 tokens per tile");
  static_assert(TJ % 4 == 0, "a slice is four MFMAs of one W fragment");
  // Chunk position of logical chunk c in row r (rows are 64 bytes, four to a
  // 256-byte bank window).  A fragment read has lane l on row 16k + (l & 15),
  // chunk l >> 4, and a ds_read_b128 serves 16 lanes per cycle: those with
  // equal bit 5 and equal parity of bits 2, 3, 4 (measured on this part).
  // Flipping the chunk's high bit with row bit 2 gives those 16 lanes 16
  // distinct 16-byte positions; the XOR with row bits 2-3 that suits 32
  // rows per chunk (lanes 0-31 on one chunk) puts pairs of them on one.
  static DEVI int swz(int r, int c) { return r * 4 + (c ^ (((r >> 2) & 1) << 1)); }
  // the staged epilogues handle 128 tokens at a time: wave row wm writes its
  // accumulators in pass hh when its tokens fall in that pass
  static DEVI bool in_pass(int wm, int hh) { return (wm * TW) / 128 == hh; }
  static DEVI int pass_row(int wm, int hh) { return wm * TW - hh * 128; }
};

template <int EPI, int BM>
__global__ __launch_bounds__(256) void gemm_big_kernel(GemmArgs a) {
  using C = BigCfg<BM>;
  constexpr int NS = C::NS, TJ = C::TJ, FI = C::FI, NF = C::NF, NSL = C::NSL;
  using T = bf16;
  __shared__ u32x4 ring[C::LDS_CHUNKS];

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

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave & 1, wm = wave >> 1;

  // The tile's stage kt is one 16 KB piece of 64-byte rows for W (K-block-major,
  // stages w_rows * 64 bytes apart) and a 16 KB (BM 256) or 8 KB (BM 128, half
  // of a 256-row tile) piece for X (256 x 32 tiles, 16 KB apart), so every DMA
  // fetches whole cache lines.  A lane's 16 bytes sit at the same offset inside
  // every stage.
  static_assert(C::BK == kTileCols, "one tile column block per stage");
  constexpr int STAGE_BYTES = kTileElems * 2;
  int voff[C::PER];
#pragma unroll
  for (int i = 0; i < C::PER; ++i) {
    const int slot = (wave * C::PER + i) * 64 + lane;
    const int row = slot / C::CPR;
    const int c = C::swz(row, slot % C::CPR) - row * C::CPR;
    voff[i] = (row < C::BN ? row : row - C::BN) * 64 + 16 * c;
  }
  const char* Wt = reinterpret_cast<const char*>(a.W) + (size_t)n0 * 64;
  const char* Xt = reinterpret_cast<const char*>(a.X) + tiled_off(m0, 0, a.K) * 2;
  const size_t w_stage = (size_t)a.w_rows * 64;
  const int nk = a.K / C::BK;
  const uint32_t ring_base = lds_address(ring);

  // stages past the end get an empty range: no memory moves, same DMA count
  auto rsrc_w = [&](int kt) {
    const bool live = kt < nk;
    return make_rsrc(Wt + (live ? kt * w_stage : 0), live ? (uint32_t)STAGE_BYTES : 0u);
  };
  auto rsrc_x = [&](int kt) {
    const bool live = kt < nk;
    return make_rsrc(Xt + (live ? kt * STAGE_BYTES : 0), live ? (uint32_t)(C::BM * 64) : 0u);
  };
  auto dma = [&](int i, const i32x4& rW, const i32x4& rX, uint32_t slot_base) {
    const int q = wave * C::PER + i;  // DMA group: W rows while q * 64 < BN * CPR
    buf_dma16_to(q * 64 < C::BN * C::CPR ? rW : rX, slot_base + (uint32_t)(q * 1024), voff[i]);
  };

  f32x4 acc[FI][TJ];

  const int l16 = lane & 15, lg = lane >> 4;
  bf16x8 fr0[NF], fr1[NF];
  // fragment f of a stage, in the order the MFMAs first use them:
  // A0, B0 .. B(TJ-1), A1 .. A7 (MFMAs run (i, j) i-major)
  auto frag_addr = [&](int f) {
    if (f == 0) return C::swz(wn * 128 + l16, lg);
    if (f <= TJ) return C::swz(C::BN + wm * C::TW + 16 * (f - 1) + l16, lg);
    return C::swz(wn * 128 + 16 * (f - TJ) + l16, lg);
  };
  auto fa = [](bf16x8 (&f)[NF], int i) -> bf16x8& { return i == 0 ? f[0] : f[TJ + i]; };
  auto fb = [](bf16x8 (&f)[NF], int j) -> bf16x8& { return f[1 + j]; };
  constexpr int RPS = (NF + NSL - 1) / NSL;  // fragment reads per slice
  auto kstep = [&](bf16x8 (&cur)[NF], bf16x8 (&nxt)[NF], const u32x4* L, const i32x4& rW, const i32x4& rX,
                   uint32_t dma_base, auto first_) {
#pragma unroll
    for (int r = 0; r < NSL; ++r) {
      const int i = r / (TJ / 4), j0 = 4 * (r % (TJ / 4));
#pragma unroll
      for (int u = 0; u < 4; ++u)
        acc[i][j0 + u] = mfma16_chunk(decltype(first_)::value ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[i][j0 + u], fa(cur, i),
                                      fb(cur, j0 + u));
#pragma unroll
      for (int f = r * RPS; f < (r + 1) * RPS && f < NF; ++f) nxt[f] = __builtin_bit_cast(bf16x8, L[frag_addr(f)]);
#pragma unroll
      for (int u = r; u < C::PER; u += NSL) dma(u, rW, rX, dma_base);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto stage = [&](int kt, bf16x8 (&cur)[NF], bf16x8 (&nxt)[NF], auto first_) {
    const int S = kt & (NS - 1);
    // stage kt+1 has landed once at most this wave's DMAs of stage kt+2 are
    // outstanding; after the barrier that holds for every wave, and every
    // wave has finished stage kt-1 (its fragment reads completed before its
    // MFMAs ran), so that slot takes stage kt+NS-1.
    wait_vmcnt<(NS - 3) * C::PER>();
    barrier_only();
    kstep(cur, nxt, ring + ((S + 1) % NS) * C::SLOT, rsrc_w(kt + NS - 1), rsrc_x(kt + NS - 1),
          ring_base + (uint32_t)(((S + NS - 1) % NS) * C::SLOT * 16), first_);
  };

#pragma unroll
  for (int st = 0; st < NS - 1; ++st) {
    const i32x4 rW = rsrc_w(st), rX = rsrc_x(st);
#pragma unroll
    for (int i = 0; i < C::PER; ++i) dma(i, rW, rX, ring_base + (uint32_t)(st * C::SLOT * 16));
  }
  wait_vmcnt<(NS - 2) * C::PER>();
  lds_barrier();
#pragma unroll
  for (int f = 0; f < NF; ++f) fr0[f] = __builtin_bit_cast(bf16x8, ring[frag_addr(f)]);
  using Yes = std::true_type;
  using No = std::false_type;
  static_assert(NS == 4, "ring of four slots");
  // The first stage starts every accumulator from zero inside its MFMAs, so
  // the loop begins with distinct values (accumulators set to one shared zero
  // beforehand make the register allocator shuffle them on every trip).
  stage(0, fr0, fr1, Yes{});
  int kt = 1;
  for (; kt + 2 <= nk; kt += 2) {
    stage(kt, fr1, fr0, No{});
    stage(kt + 1, fr0, fr1, No{});
  }
  stage(kt, fr1, fr0, No{});  // nk is even: one stage remains
  wait_vmcnt<0>();

  if constexpr (EPI == (int)Epi::SWIGLU) {
    // The tile's s = SiLU(r g) * (r u) is BM tokens x 128 columns of the down
    // GEMM's tiled operand (rows of a 32-column block 64 bytes apart).  In
    // block (i, j) lane l holds columns 8i + 2(l >> 4) + {0, 1} of token
    // 16j + (l & 15).  A 4 x 4 transpose across the wave's four 16-lane rows
    // (lane swaps at distance 32, then 16) over blocks i0 .. i0+3 leaves lane l
    // with the 8 consecutive columns 8(i0 + (l >> 4)) + {0..7} of its token:
    // one 16-byte store per lane, and 16 tokens x 64 bytes = 1 KB contiguous
    // per store instruction, with no trip through LDS.
    // m0 may be the second half of a 256-row tile (BM 128): tiled_off places
    // the tile's first row.
    bf16* ob = reinterpret_cast<bf16*>(a.out) + tiled_off(m0, n0 / 2, a.ldo);
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int tl = wm * C::TW + 16 * j + l16;
      const bool live = m0 + tl < a.M;
      const float r = live ? a.rowscale[m0 + tl] : 0.f;
#pragma unroll
      for (int i0 = 0; i0 < FI; i0 += 4) {
        unsigned w[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const f32x4 v = acc[i0 + u][j] * r;
          w[u] = __builtin_bit_cast(unsigned, bf16x2{from_f32<bf16>(silu(v[0]) * v[1]), from_f32<bf16>(silu(v[2]) * v[3])});
        }
        const auto p02 = __builtin_amdgcn_permlane32_swap(w[0], w[2], false, false);
        const auto p13 = __builtin_amdgcn_permlane32_swap(w[1], w[3], false, false);
        const auto p01 = __builtin_amdgcn_permlane16_swap(p02[0], p13[0], false, false);
        const auto p23 = __builtin_amdgcn_permlane16_swap(p02[1], p13[1], false, false);
        const int cl = wn * 64 + 8 * (i0 + lg);  // first s column of this lane's 16 bytes
        if (live)
          *reinterpret_cast<u32x4*>(ob + (cl >> 5) * kTileElems + tl * 32 + (cl & 31)) =
              u32x4{p01[0], p01[1], p23[0], p23[1]};
      }
    }
    return;
  }

  if constexpr (EPI == (int)Epi::QKV) {
    // QKV epilogue through LDS, one half of the tile (128 tokens, fp32) at a
    // time (same layout as the residual epilogues below), with the row scale
    // r1 applied as the accumulators are staged.  Pass 1 takes the q and k
    // features a token row per wave instruction: RoPE with the cos/sin table
    // rows read whole, q -> its [M][H*D] row, k -> its cache row.  Pass 2 takes the v features column-wise: the
    // eight keys of a V^T cache row half (vperm_pos order) are gathered from
    // LDS and stored as one 16-byte piece, with the cache block of each
    // 16-row group looked up once per half; blocks the half does not cover
    // whole (ragged batch or sequence edges, continuation prefill) are stored
    // key by key.
    f32x4* st = reinterpret_cast<f32x4*>(ring);
    float* stf = reinterpret_cast<float*>(ring);
    __shared__ int vgrp[8];  // per 16-row group of the half: its cache block when whole, else -1
    const int D = a.cache.D, G = a.cache.G, HD = a.H * D, KD = G * D;
    const int S = a.batch.seq_len;
    const float qs = q_scale(D);
    const bool has_v = n0 + C::BN > HD + KD && n0 < HD + 2 * KD;
    __syncthreads();  // every wave is done with the ring
#pragma unroll 1
    for (int hh = 0; hh < C::HALVES; ++hh) {
      if (C::in_pass(wm, hh)) {
        float rsj[TJ];
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          const int t = m0 + hh * 128 + C::pass_row(wm, hh) + 16 * j + l16;
          rsj[j] = t < a.M ? a.rowscale[t] : 0.f;
        }
#pragma unroll
        for (int i = 0; i < FI; ++i)
#pragma unroll
          for (int j = 0; j < TJ; ++j) {
            const int r = C::pass_row(wm, hh) + 16 * j + l16, c = (wn * 128 + 16 * i + 4 * lg) >> 2;
            st[r * 64 + (c ^ (r & 63))] = acc[i][j] * rsj[j];
          }
      }
      if (has_v && tid < 8) {
        const int t0 = m0 + hh * 128 + 16 * tid;
        int blk = -1;
        if (t0 + 15 < a.M) {
          const int b0 = t0 / S;
          const int pos0 = a.batch.desc[2 * b0 + 1] + (t0 - b0 * S);
          if ((pos0 & 15) == 0 && (t0 + 15) / S == b0)
            blk = a.cache.block_table[(size_t)a.batch.desc[2 * b0] * a.cache.max_blocks + (pos0 >> 4)];
        }
        vgrp[tid] = blk;
      }
      __syncthreads();
      // ---- pass 1: q and k ----
      const int f = n0 + 4 * lane;
      if (n0 < HD + KD) {
        // token of row p of this wave: tb + 4p; per-row data one row per
        // lane, broadcast with readlane
        const int tb = m0 + hh * 128 + wave;
        int pos_l = 0, blk_l = 0;
        {
          const int t = tb + 4 * (lane & 31);
          if (t < a.M) {
            const int b = t / S;
            pos_l = a.batch.desc[2 * b + 1] + (t - b * S);
            blk_l = a.cache.block_table[(size_t)a.batch.desc[2 * b] * a.cache.max_blocks + (pos_l >> 4)];
          }
        }
        const bool qk = f < HD + KD;  // lanes past the k features hold v (pass 2)
        const int kf = f - HD, g = kf / D;
        const int dd = (f < HD ? f : kf) % D;
        const float* cs_col = a.rope_cos + dd / 2;
        const float* sn_col = a.rope_sin + dd / 2;
        const int nrow = min(32, max(0, (a.M - tb + 3) >> 2));  // rows with t < M
        // the RoPE table rows of 16 token rows are loaded before any of them is
        // used (8, 16 and 32 rows measured within noise of each other; one
        // row at a time, as a loop whose early exits sat before the loads,
        // cost about 45 us per QKV launch at the LLaMA-3-8B shape and 8192 tokens)
        constexpr int NB = 16;
        // A tile of q features only (or k only) with all 32 rows and adjacent
        // RoPE pairs (every tile of the 8B-shaped layer at 8192 tokens): the
        // rows take no branches, so a batch's LDS reads issue together
        // instead of one LDS round trip per row (the same values and stores
        // as the general loop below)
        auto rows_fast = [&](auto is_k_) {
          constexpr bool IS_K = decltype(is_k_)::value;
#pragma unroll 1
          for (int p0 = 0; p0 < 32; p0 += NB) {
            f32x2 cs[NB], sn[NB];
            f32x4 xr[NB];
#pragma unroll
            for (int u = 0; u < NB; ++u) {
              const size_t o = (size_t)__builtin_amdgcn_readlane(pos_l, p0 + u) * (D / 2);
              cs[u] = *reinterpret_cast<const f32x2*>(cs_col + o);
              sn[u] = *reinterpret_cast<const f32x2*>(sn_col + o);
            }
#pragma unroll
            for (int u = 0; u < NB; ++u) {
              const int r = (p0 + u) * 4 + wave;
              xr[u] = st[r * 64 + (lane ^ (r & 63))];
            }
#pragma unroll
            for (int u = 0; u < NB; ++u) {
              const int p = p0 + u, t = tb + 4 * p;
              const f32x4 v = rotate4(xr[u], cs[u], sn[u]);
              if constexpr (IS_K) {
                const int pos = __builtin_amdgcn_readlane(pos_l, p);
                const size_t blk = (size_t)__builtin_amdgcn_readlane(blk_l, p);
                store4(reinterpret_cast<bf16*>(a.cache.k_pool) + ((blk * G + g) * 16 + (pos & 15)) * D + dd, v[0],
                       v[1], v[2], v[3]);
              } else {
                const f32x4 w = v * qs;
                store4(reinterpret_cast<bf16*>(a.q_out) + (size_t)t * HD + f, w[0], w[1], w[2], w[3]);
              }
            }
          }
        };
        const bool all_q = n0 + C::BN <= HD, all_k = n0 >= HD && n0 + C::BN <= HD + KD;
        if (nrow == 32 && !a.rope_half && all_q) {
          rows_fast(std::false_type{});
        } else if (nrow == 32 && !a.rope_half && all_k) {
          rows_fast(std::true_type{});
        } else {
#pragma unroll 1
          for (int p0 = 0; p0 < nrow; p0 += NB) {
            f32x2 cs[NB], sn[NB];
#pragma unroll
            for (int u = 0; u < NB; ++u) {
              const size_t o = (size_t)__builtin_amdgcn_readlane(pos_l, p0 + u) * (D / 2);
              cs[u] = *reinterpret_cast<const f32x2*>(cs_col + o);
              sn[u] = *reinterpret_cast<const f32x2*>(sn_col + o);
            }
#pragma unroll
            for (int u = 0; u < NB; ++u) {
              const int p = p0 + u, r = p * 4 + wave, t = tb + 4 * p;
              if (p >= nrow || !qk) continue;
              const f32x4 v = rotate4(st[r * 64 + (lane ^ (r & 63))], cs[u], sn[u]);
              if (f < HD) {
                store_head4(reinterpret_cast<bf16*>(a.q_out) + (size_t)t * HD + (f - dd), dd, v * qs, a.rope_half, D);
              } else {
                const int pos = __builtin_amdgcn_readlane(pos_l, p);
                const size_t blk = (size_t)__builtin_amdgcn_readlane(blk_l, p);
                store_head4(reinterpret_cast<bf16*>(a.cache.k_pool) + ((blk * G + g) * 16 + (pos & 15)) * D, dd, v,
                            a.rope_half, D);
              }
            }
          }
        }
      }
      // ---- pass 2: v (cache rows of V^T: 16 keys of one feature per 32 bytes) ----
      if (has_v) {
        const int vf0 = max(n0, HD + KD), vf1 = min(n0 + C::BN, HD + 2 * KD);
        const int nvf = vf1 - vf0;
        const int units = 8 * nvf * 2;  // 16-row groups x features x row halves
        for (int u = tid; u < units; u += 256) {
          const int rg = u / (nvf * 2), rem = u - rg * (nvf * 2);
          const int fl = vf0 + (rem >> 1) - n0, ch = rem & 1;  // feature within the tile, V^T row half
          const int vfeat = n0 + fl - HD - KD, g = vfeat / D, d = vfeat - g * D;
          const int r0 = 16 * rg, t0 = m0 + hh * 128 + r0;
          if (t0 >= a.M) continue;
          const int cidx = fl >> 2, e = fl & 3;
          // row r (0..127) of the half held in LDS
          auto lds_val = [&](int r) { return stf[(r * 64 + (cidx ^ (r & 63))) * 4 + e]; };
          const int blk = vgrp[rg];
          if (blk >= 0) {  // keys 4ch..4ch+3 and 8+4ch..8+4ch+3 of the group's block
            bf16x8 w;
#pragma unroll
            for (int k = 0; k < 8; ++k) w[k] = from_f32<bf16>(lds_val(r0 + 4 * ch + (k & 3) + 2 * (k & 4)));
            *reinterpret_cast<bf16x8*>(reinterpret_cast<bf16*>(a.cache.v_pool) + (((size_t)blk * G + g) * D + d) * 16 +
                                       8 * ch) = w;
          } else {  // key by key: this unit takes rows r0 + 4ch + {0..3} and r0 + 8 + 4ch + {0..3}
#pragma unroll
            for (int k = 0; k < 8; ++k) {
              const int rr = 4 * ch + (k & 3) + 2 * (k & 4);
              const int t = t0 + rr;
              if (t >= a.M) continue;
              const int b = t / S, pos = a.batch.desc[2 * b + 1] + (t - b * S), seq = a.batch.desc[2 * b];
              const size_t kb = (size_t)a.cache.block_table[(size_t)seq * a.cache.max_blocks + (pos >> 4)];
              reinterpret_cast<bf16*>(a.cache.v_pool)[((kb * G + g) * D + d) * 16 + vperm_pos(pos & 15)] =
                  from_f32<bf16>(lds_val(r0 + rr));
            }
          }
        }
      }
      __syncthreads();
    }
    return;
  }

  if constexpr (EPI == (int)Epi::RESID_H || EPI == (int)Epi::RESID_OUT) {
    // Residual epilogues: each token row of the tile is 256 contiguous
    // features of a row-major [M][N] output.  The accumulators go through LDS
    // one half of the tile (128 tokens, fp32, 128 KB) at a time, so that the
    // residual loads and the output stores cover whole rows: a wave moves one
    // token's 1 KB (fp32) per instruction.  16-byte chunk c of LDS row r sits
    // at chunk c ^ (r & 63), which keeps both the per-lane writes (32 rows,
    // one chunk) and the row reads free of bank conflicts.
    f32x4* st = reinterpret_cast<f32x4*>(ring);
    __syncthreads();  // every wave is done with the ring
#pragma unroll
    for (int hh = 0; hh < C::HALVES; ++hh) {
      // the half's residual rows are loaded first, so that their latency
      // overlaps the LDS writes and the barrier
      f32x4 res[32];
#pragma unroll
      for (int p = 0; p < 32; ++p) {
        const int t = m0 + hh * 128 + p * 4 + wave;
        const size_t o = (size_t)min(t, a.M - 1) * a.ldo + n0 + 4 * lane;
        if constexpr (EPI == (int)Epi::RESID_H)
          res[p] = load4(reinterpret_cast<const T*>(a.resid) + o);
        else
          res[p] = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(a.resid) + o);
      }
      if (C::in_pass(wm, hh)) {
#pragma unroll
        for (int i = 0; i < FI; ++i)
#pragma unroll
          for (int j = 0; j < TJ; ++j) {
            const int r = C::pass_row(wm, hh) + 16 * j + l16, c = (wn * 128 + 16 * i + 4 * lg) >> 2;
            st[r * 64 + (c ^ (r & 63))] = acc[i][j];
          }
      }
      __syncthreads();
      // A half whose 128 rows all lie before M takes a copy without the
      // per-row test, so that the LDS reads of 8 rows issue together instead
      // of one LDS round trip per row (the same sums and stores as below).
      auto rows_full = [&](auto out_f32_) {
        constexpr bool OUT_F32 = decltype(out_f32_)::value;
#pragma unroll
        for (int p0 = 0; p0 < 32; p0 += 8) {
          f32x4 vv[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int r = (p0 + u) * 4 + wave;
            vv[u] = st[r * 64 + (lane ^ (r & 63))];
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int p = p0 + u, r = p * 4 + wave, t = m0 + hh * 128 + r;
            const size_t o = (size_t)t * a.ldo + n0 + 4 * lane;
            const f32x4 hv = res[p] + vv[u];
            if constexpr (OUT_F32)
              *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + o) = hv;
            else
              store4(reinterpret_cast<bf16*>(a.out) + o, hv[0], hv[1], hv[2], hv[3]);
          }
        }
      };
      const bool out_f32 = EPI == (int)Epi::RESID_H || a.out_dtype == DType::F32;
      if (m0 + hh * 128 + 128 <= a.M && out_f32) {
        rows_full(std::true_type{});
      } else if (m0 + hh * 128 + 128 <= a.M) {
        rows_full(std::false_type{});
      } else {
#pragma unroll
        for (int p = 0; p < 32; ++p) {
          const int r = p * 4 + wave, c = lane;  // wave-uniform row, lane = 16-byte chunk
          const int t = m0 + hh * 128 + r;
          if (t < a.M) {
            const f32x4 v = st[r * 64 + (c ^ (r & 63))];
            const size_t o = (size_t)t * a.ldo + n0 + 4 * c;
            if constexpr (EPI == (int)Epi::RESID_H) {  // h = x + attn W_o^T, fp32
              *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + o) = res[p] + v;
            } else {  // out = h + s W_down^T
              const f32x4 hv = res[p] + v;
              if (a.out_dtype == DType::F32)
                *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + o) = hv;
              else
                store4(reinterpret_cast<bf16*>(a.out) + o, hv[0], hv[1], hv[2], hv[3]);
            }
          }
        }
      }
      __syncthreads();
    }
    return;
  }

#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int t = m0 + wm * C::TW + 16 * j + l16;
      if (t < a.M) epilogue<T, EPI>(a, t, n0 + wn * 128 + 16 * i + 4 * lg, acc[i][j]);
    }
}

// ---------------------------------------------------------------------------
// Skinny bf16 GEMM for few tokens (decode): the weights are streamed once from
// HBM and the work is bound by that stream, so the shape is chosen for memory
// parallelism, not reuse.  Workgroups of 64 features x 64 tokens and one of
// KS slices of K, two resident per CU (a 64 KB ring each), so that a launch
// of more workgroups than CUs (448 for the 8B gate/up) has them all in flight
// at once.  K is split into the largest power of two of slices that keeps the
// workgroups within 256 (more, shorter slices measured slower: each pays the
// pipeline ramp-up, and the partial sums grow), with at least two 64-deep
// stages per slice.  With KS = 1 the epilogue runs directly, otherwise the
// fp32 partial goes to [ks][M][N] and a second pass adds the KS partials in a
// fixed order and runs the epilogue.
// ---------------------------------------------------------------------------
int skinny_ks(int M, int N, int K) {
  const int groups = (N / 64) * ((M + 63) / 64);
  int ks = 1;
  while (ks < 16 && groups * ks * 2 <= 256 && K / (128 * ks * 2) >= 1) ks *= 2;
  return ks;
}

template <int EPI>
__global__ __launch_bounds__(256) void gemm_split_reduce_kernel(GemmArgs a, int KS) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;  // f32x4 index in [M][N / 4]
  const int n4 = a.N / 4;
  if (i >= (size_t)a.M * n4) return;
  const int t = (int)(i / n4), f = (int)(i % n4) * 4;
  const f32x4* p = reinterpret_cast<const f32x4*>(a.split_ws) + (size_t)t * n4 + f / 4;
  f32x4 v = p[0];
  for (int k = 1; k < KS; ++k) v += p[(size_t)k * a.M * n4];
  epilogue<bf16, EPI>(a, t, f, v);
}

// RESID_H pass that also runs the second RMSNorm (bf16): workgroup (segment,
// token) adds the K partials of 1024 features in slice order, writes
// h = x + sum, h * gamma_2 rounded to bf16 in the gate/up GEMM's tiled order,
// and the segment's sum of h^2 (lanes, then waves, in a fixed order); the
// gate/up epilogue adds the row's segments in order, so the result does not
// depend on timing.
__global__ __launch_bounds__(256) void gemm_split_reduce_norm_kernel(GemmArgs a, int KS) {
  const int seg = blockIdx.x, t = blockIdx.y;
  const int f = seg * kNormSeg + threadIdx.x * 4;
  float ss = 0.f;
  if (f < a.N) {
    const f32x4* p = reinterpret_cast<const f32x4*>(a.split_ws + (size_t)t * a.N + f);
    const size_t slice = (size_t)a.M * a.N / 4;
    f32x4 v = p[0];
    for (int k = 1; k < KS; ++k) v += p[k * slice];
    const size_t o = (size_t)t * a.ldo + f;
    const f32x4 h = load4(reinterpret_cast<const bf16*>(a.resid) + o) + v;
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + o) = h;
    ss = h[0] * h[0] + h[1] * h[1] + h[2] * h[2] + h[3] * h[3];
    const f32x4 g = h * *reinterpret_cast<const f32x4*>(a.norm_gamma + f);
    *reinterpret_cast<bf16x4*>(reinterpret_cast<bf16*>(a.norm_out) + tiled_off(t, f, a.N)) =
        bf16x4{from_f32<bf16>(g[0]), from_f32<bf16>(g[1]), from_f32<bf16>(g[2]), from_f32<bf16>(g[3])};
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) ss += shfl_xor(ss, m);
  __shared__ float wsum[4];
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = ss;
  __syncthreads();
  if (threadIdx.x == 0) a.ss_part[(size_t)t * a.ss_nseg + seg] = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
}

// ---------------------------------------------------------------------------
// Weight-streaming bf16 GEMM for few tokens, staged through LDS.  A workgroup
// owns 64 features x 64 tokens and one of KS slices of K.  Stages of 64
// K-elements (W: 64 rows x 128 B, X: 64 rows x 128 B) are moved by LDS DMA
// into a ring of NSL slots, NSL - 1 stages ahead (8 slots and one workgroup
// per CU measured 2-7% slower on the 8B decode shapes, also for launches of
// at most one workgroup per CU), each DMA instruction
// fetching whole 128-byte row segments.  Wave w computes features 16w..16w+15
// for all 64 tokens, so no cross-wave reduction is needed.
// ---------------------------------------------------------------------------
struct StreamCfg {
  static constexpr int NSL = 4;                 // ring slots (64 KB: two workgroups per CU)
  static constexpr int CPR = 8;                 // 16-byte chunks per row per stage (64 bf16)
  static constexpr int ROWS = 128;              // 64 W rows, then 64 X rows
  static constexpr int SLOT = ROWS * CPR;       // chunks per slot (16 KB)
  static constexpr int PER = SLOT / 256;        // DMAs per thread per stage
  // chunk position of logical chunk c in row r: XOR with the row spreads a
  // quarter-wave's 16 rows over all 16-byte bank groups
  static DEVI int swz(int r, int c) { return r * CPR + (c ^ (r & 7)); }
};

template <int EPI>
__global__ __launch_bounds__(256, 2) void gemm_stream_kernel(GemmArgs a, int KS) {
  using C = StreamCfg;
  __shared__ u32x4 ring[C::NSL * C::SLOT];
  const int n0 = blockIdx.x * 64, m0 = blockIdx.y * 64, ks = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15, g4 = lane >> 4;

  const int nk = a.K / 64;
  const int s_beg = nk * ks / KS, s_end = nk * (ks + 1) / KS;
  const int ns = s_end - s_beg;

  // A 64-deep stage of 64 rows is two contiguous 4 KB pieces per operand, one
  // in each of two consecutive 32-column K blocks: w_rows * 64 bytes apart for
  // W (K-block-major), 16 KB apart for X (256 x 32 tiles).  X rows past M are
  // padding rows of the tile (never stored).
  // DMA i of this thread: chunk slot (wave * PER + i) * 64 + lane of a stage
  const int wkb = a.w_rows * 64;  // bytes between W K blocks
  const char* Wt = reinterpret_cast<const char*>(a.W) + (size_t)s_beg * 2 * wkb + (size_t)n0 * 64;
  const char* Xt = reinterpret_cast<const char*>(a.X) + tiled_off(m0, s_beg * 64, a.K) * 2;
  constexpr int X_STAGE = 2 * kTileElems * 2;
  const uint32_t W_RANGE = (uint32_t)wkb + 64 * 64;             // both 4 KB pieces
  constexpr uint32_t X_RANGE = kTileElems * 2 + 64 * 64;
  // DMA group q = wave * PER + i covers rows 8q .. 8q + 7: W rows for q < 8,
  // X rows after (wave-uniform, so the descriptor choice stays scalar)
  int voff[C::PER];
#pragma unroll
  for (int i = 0; i < C::PER; ++i) {
    const int slot = (wave * C::PER + i) * 64 + lane;
    const int row = slot / C::CPR, c = (slot % C::CPR) ^ (row & 7);
    const bool is_x = wave * C::PER + i >= 8;
    voff[i] = (c >> 2) * (is_x ? kTileElems * 2 : wkb) + (row & 63) * 64 + (c & 3) * 16;
  }
  const uint32_t ring_base = lds_address(ring);
  auto issue = [&](int st) {
    const bool live = st < ns;
    const i32x4 rW = make_rsrc(Wt + (live ? (size_t)st * 2 * wkb : 0), live ? W_RANGE : 0u);
    const i32x4 rX = make_rsrc(Xt + (live ? st * X_STAGE : 0), live ? X_RANGE : 0u);
    const uint32_t slot_base = ring_base + (uint32_t)((st % C::NSL) * C::SLOT * 16);
#pragma unroll
    for (int i = 0; i < C::PER; ++i)
      buf_dma16_to(wave * C::PER + i >= 8 ? rX : rW, slot_base + (uint32_t)((wave * C::PER + i) * 1024), voff[i]);
  };

  f32x4 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int st = 0; st < C::NSL - 1; ++st) issue(st);
#pragma unroll 1
  for (int st = 0; st < ns; ++st) {
    wait_vmcnt<(C::NSL - 2) * C::PER>();  // stage st landed (later stages may still be in flight)
    lds_barrier();                         // ... for every wave; and every wave is done with st - 1
    issue(st + C::NSL - 1);
    const u32x4* L = ring + (st % C::NSL) * C::SLOT;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int c = 4 * kk + g4;
      const bf16x8 fa = __builtin_bit_cast(bf16x8, L[C::swz(16 * wave + c16, c)]);
      bf16x8 fb[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) fb[j] = __builtin_bit_cast(bf16x8, L[C::swz(64 + 16 * j + c16, c)]);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = mfma16_chunk(acc[j], fa, fb[j]);
    }
  }
  wait_vmcnt<0>();  // the empty DMAs issued past the end have retired

  const int f = n0 + 16 * wave + 4 * g4;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int t = m0 + 16 * j + c16;
    if (t >= a.M) continue;
    if (KS == 1)
      epilogue<bf16, EPI>(a, t, f, acc[j]);
    else
      *reinterpret_cast<f32x4*>(a.split_ws + ((size_t)ks * a.M + t) * a.N + f) = acc[j];
  }
}

template <int EPI>
hipError_t launch_skinny_epi(const GemmArgs& a, int KS, hipStream_t s) {
  dim3 grid(a.N / 64, (a.M + 63) / 64, KS);
  gemm_stream_kernel<EPI><<<grid, 256, 0, s>>>(a, KS);
  if (EPI == 1 && a.norm_gamma) {
    gemm_split_reduce_norm_kernel<<<dim3(a.ss_nseg, a.M), 256, 0, s>>>(a, KS);
  } else if (KS > 1) {
    const size_t n = (size_t)a.M * (a.N / 4);
    gemm_split_reduce_kernel<EPI><<<(unsigned)((n + 255) / 256), 256, 0, s>>>(a, KS);
  }
  return hipGetLastError();
}

hipError_t launch_skinny(const GemmArgs& a, hipStream_t s) {
  if (a.N % 64 != 0 || a.K % 64 != 0 || a.M <= 0 || a.M > 256) return hipErrorInvalidValue;
  const int KS = skinny_ks(a.M, a.N, a.K);
  if (KS > 1 && (a.split_ws == nullptr || a.split_ws_bytes < (size_t)KS * a.M * a.N * sizeof(float)))
    return hipErrorInvalidValue;
  // the folded norm needs the split pass and whole 1024-feature segments
  if (a.norm_gamma && (a.epi != Epi::RESID_H || KS == 1 || !a.norm_out || !a.ss_part ||
                       a.ss_nseg != (a.N + kNormSeg - 1) / kNormSeg || a.ldo != a.N))
    return hipErrorInvalidValue;
  switch (a.epi) {
    case Epi::QKV: return launch_skinny_epi<0>(a, KS, s);
    case Epi::RESID_H: return launch_skinny_epi<1>(a, KS, s);
    case Epi::SWIGLU: return launch_skinny_epi<2>(a, KS, s);
    case Epi::RESID_OUT: return launch_skinny_epi<3>(a, KS, s);
  }
  return hipErrorInvalidValue;
}

template <typename T, typename C>
hipError_t launch_cfg(const GemmArgs& a, hipStream_t s) {
  if (a.N % C::BN != 0 || a.K % (2 * C::BK) != 0 || a.M <= 0) return hipErrorInvalidValue;
  // row-major (fp32) operands: 32-bit buffer offsets, so a tile's rows times
  // the row pitch must stay below 2^31 (tiled bf16 stages are 16 KB pieces)
  if (sizeof(T) == 4 && ((int64_t)C::BN * a.K * (int64_t)sizeof(T) >= (1ll << 31) ||
                         (int64_t)C::BM * a.ldx * (int64_t)sizeof(T) >= (1ll << 31)))
    return hipErrorInvalidValue;
  const int grid = (a.N / C::BN) * ((a.M + C::BM - 1) / C::BM);
  switch (a.epi) {
    case Epi::QKV: gemm_kernel<T, C, 0><<<grid, C::NT, 0, s>>>(a); break;
    case Epi::RESID_H: gemm_kernel<T, C, 1><<<grid, C::NT, 0, s>>>(a); break;
    case Epi::SWIGLU: gemm_kernel<T, C, 2><<<grid, C::NT, 0, s>>>(a); break;
    case Epi::RESID_OUT: gemm_kernel<T, C, 3><<<grid, C::NT, 0, s>>>(a); break;
  }
  return hipGetLastError();
}

template <int BM>
hipError_t launch_big_bm(const GemmArgs& a, hipStream_t s) {
  using C = BigCfg<BM>;
  if (a.N % C::BN != 0 || a.K % (2 * C::BK) != 0 || a.M <= 0) return hipErrorInvalidValue;
  const int grid = (a.N / C::BN) * ((a.M + C::BM - 1) / C::BM);
  switch (a.epi) {
    case Epi::QKV: gemm_big_kernel<0, BM><<<grid, C::NT, 0, s>>>(a); break;
    case Epi::RESID_H: gemm_big_kernel<1, BM><<<grid, C::NT, 0, s>>>(a); break;
    case Epi::SWIGLU: gemm_big_kernel<2, BM><<<grid, C::NT, 0, s>>>(a); break;
    case Epi::RESID_OUT: gemm_big_kernel<3, BM><<<grid, C::NT, 0, s>>>(a); break;
  }
  return hipGetLastError();
}

// 256 x 256 tiles, or 256 x 128 when 256 x 256 would fill fewer than two
// rounds of the 256 CUs (the half-height tile has two thirds of the
// arithmetic intensity, so it pays only where it fills idle CUs)
int big_tile_m(int M, int N) {
  const long tiles256 = (long)(N / 256) * ((M + 255) / 256);
  return tiles256 < 2 * 256 ? 128 : 256;
}

hipError_t launch_big(const GemmArgs& a, hipStream_t s) {
  return big_tile_m(a.M, a.N) == 128 ? launch_big_bm<128>(a, s) : launch_big_bm<256>(a, s);
}

using SmallBF = Cfg<bf16, 64, 64, 2, 2>;
using LargeF = Cfg<float, 256, 256, 2, 4>;
using SmallF = Cfg<float, 64, 64, 2, 2>;

}  // namespace

int gemm_tile_n(GemmTile t) { return t == GemmTile::LARGE ? 256 : 64; }

int skinny_ksplit(int M, int N, int K) { return skinny_ks(M, N, K); }
size_t skinny_partial_bytes(int M, int N, int K) {
  const int ks = skinny_ks(M, N, K);
  return ks > 1 ? (size_t)ks * M * N * sizeof(float) : 0;
}

hipError_t launch_gemm(DType t, GemmTile tile, const GemmArgs& a, hipStream_t s) {
  if (t == DType::BF16) {
    if (a.w_rows < a.N || a.w_rows % kTileRows != 0) return hipErrorInvalidValue;  // K-block stride of W
    if (tile == GemmTile::SKINNY) return launch_skinny(a, s);
    return tile == GemmTile::LARGE ? launch_big(a, s) : launch_cfg<bf16, SmallBF>(a, s);
  }
  if (tile == GemmTile::SKINNY) return hipErrorInvalidValue;
  return tile == GemmTile::LARGE ? launch_cfg<float, LargeF>(a, s) : launch_cfg<float, SmallF>(a, s);
}

}  // namespace llk
