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
#include "common.h"
#include "kernels.h"
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
  int vW[C::LW], vX[C::LX];
#pragma unroll
  for (int i = 0; i < C::LW; ++i) {
    const int slot = (wave * C::LW + i) * 64 + lane;
    const int row = slot >> 2, c = (slot & 3) ^ ((row >> 2) & 3);
    vW[i] = (row * a.K + c * Chunk<T>::N) * ES;
  }
#pragma unroll
  for (int i = 0; i < C::LX; ++i) {
    const int slot = (wave * C::LX + i) * 64 + lane;
    const int row = slot >> 2, c = (slot & 3) ^ ((row >> 2) & 3);
    vX[i] = (row * a.ldx + c * Chunk<T>::N) * ES;
  }
  const char* Wt = reinterpret_cast<const char*>(a.W) + (size_t)n0 * a.K * ES;
  const char* Xt = reinterpret_cast<const char*>(a.X) + (size_t)m0 * a.ldx * ES;
  // bytes of X from the tile's first row to the end of the matrix (< 2^31 for
  // every supported shape), kept wave-uniform so the descriptor lives in SGPRs
  const uint64_t xb = (uint64_t)(a.M - m0) * (uint64_t)a.ldx * ES;
  const int x_bytes = __builtin_amdgcn_readfirstlane((int)(xb < 0x7fffffffull ? xb : 0x7fffffffull));
  const int nk = a.K / C::BK;

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
    const int kb = live ? kt * C::BK * ES : 0;
    const i32x4 rW = make_rsrc(Wt + kb, live ? 0x7fffffffu : 0u);
    const i32x4 rX = make_rsrc(Xt + kb, live ? (uint32_t)(x_bytes - kb) : 0u);
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
// Large bf16 tiles: 256 features x 256 tokens, four waves (one per SIMD), each
// wave 128 x 128 as 4 x 4 blocks of v_mfma_f32_32x32x16_bf16 whose
// accumulators (256 registers) stay in the matrix core's register file.
// A stage is 32 elements of K (two k-steps of 16) held in one slot of a
// four-slot LDS ring.  Each k-step is 8 slices of two MFMAs plus one LDS read
// of the next k-step's fragments (read in the order the MFMAs consume them),
// so with a single wave per SIMD the matrix core does not wait for LDS:
//   k-step 0 of stage kt: MFMAs || reads of k-step 1;
//   wait for this wave's DMAs of stage kt+1, barrier (every wave now holds
//   all of stage kt in registers);
//   k-step 1: MFMAs || reads of k-step 0 of stage kt+1 || one DMA per slice
//   of stage kt+4 into stage kt's slot.
// 32x32 result layout: lane l holds token (l & 31) and, in registers
// 4g..4g+3, features 8g + 4(l >> 5) + {0..3}: four lane-local groups of four
// consecutive features, so the same epilogues apply.
// ---------------------------------------------------------------------------
struct BigCfg {
  static constexpr int BN = 256, BM = 256, NT = 256, CPR = 4, BK = 32, NS = 4;
  static constexpr int LW = BN * CPR / NT, LX = BM * CPR / NT;  // 16-byte DMAs per thread per stage
  static constexpr int SLOT = (BN + BM) * CPR;                    // 16-byte chunks per slot
};

template <int EPI>
__global__ __launch_bounds__(256) void gemm_big_kernel(GemmArgs a) {
  using C = BigCfg;
  using T = bf16;
  __shared__ u32x4 L0[C::SLOT];
  __shared__ u32x4 L1[C::SLOT];
  __shared__ u32x4 L2[C::SLOT];
  __shared__ u32x4 L3[C::SLOT];

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
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave & 1, wm = wave >> 1;

  // DMA i of this lane: W rows for i < LW, X rows after; slot s of a stage
  // holds logical chunk (s % 4) ^ swizzle(row) of row s / 4
  constexpr int ES = 2, PER = C::LW + C::LX;
  int voff[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int slot = ((i < C::LW ? wave * C::LW + i : wave * C::LX + i - C::LW)) * 64 + lane;
    const int row = slot >> 2, c = (slot & 3) ^ ((row >> 2) & 3);
    voff[i] = (row * (i < C::LW ? a.K : a.ldx) + c * 8) * ES;
  }
  // LDS byte address (wave-uniform) where DMA i of this wave lands, relative to its slot
  auto dma_lds = [&](int i) {
    return (i < C::LW ? (wave * C::LW + i) * 1024 : C::BN * C::CPR * 16 + (wave * C::LX + i - C::LW) * 1024);
  };
  const char* Wt = reinterpret_cast<const char*>(a.W) + (size_t)n0 * a.K * ES;
  const char* Xt = reinterpret_cast<const char*>(a.X) + (size_t)m0 * a.ldx * ES;
  const uint64_t xb = (uint64_t)(a.M - m0) * (uint64_t)a.ldx * ES;
  const int x_bytes = __builtin_amdgcn_readfirstlane((int)(xb < 0x7fffffffull ? xb : 0x7fffffffull));
  const int nk = a.K / C::BK;
  const uint32_t base[4] = {lds_address(L0), lds_address(L1), lds_address(L2), lds_address(L3)};

  // buffer descriptors of stage kt; stages past the end get empty buffers
  // (no memory moves, but every stage has the same DMA count to wait on)
  auto rsrc_w = [&](int kt) {
    const bool live = kt < nk;
    return make_rsrc(Wt + (live ? kt * C::BK * ES : 0), live ? 0x7fffffffu : 0u);
  };
  auto rsrc_x = [&](int kt) {
    const bool live = kt < nk;
    const int kb = live ? kt * C::BK * ES : 0;
    return make_rsrc(Xt + kb, live ? (uint32_t)(x_bytes - kb) : 0u);
  };
  auto dma = [&](int i, const i32x4& rW, const i32x4& rX, uint32_t slot_base) {
    buf_dma16_to(i < C::LW ? rW : rX, slot_base + dma_lds(i), voff[i]);
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int l32 = lane & 31, lh = lane >> 5;
  // fragment r of a k-step, in the order the MFMAs first use them:
  // A0, B0, B1, B2, B3, A1, A2, A3 (MFMAs run (i, j) i-major)
  bf16x8 fr0[8], fr1[8];
  auto frag_addr = [&](int r, int ks) {
    const int c = 2 * ks + lh;
    if (r == 0) return C::BN * 0 + swz(wn * 128 + l32, c);
    if (r <= 4) return C::BN * C::CPR + swz(wm * 128 + 32 * (r - 1) + l32, c);
    return swz(wn * 128 + 32 * (r - 4) + l32, c);
  };
  auto fa = [](bf16x8 (&f)[8], int i) -> bf16x8& { return i == 0 ? f[0] : f[4 + i]; };
  auto fb = [](bf16x8 (&f)[8], int j) -> bf16x8& { return f[1 + j]; };
  // one k-step: 8 slices of {2 MFMAs from cur, read fragment r of the next
  // k-step into nxt (from slot L, k-step nks), DMA r if requested}
  auto kstep = [&](bf16x8 (&cur)[8], bf16x8 (&nxt)[8], const u32x4* L, int nks, bool with_dma, const i32x4& rW,
                   const i32x4& rX, uint32_t dma_base) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int i = r >> 1, j0 = 2 * (r & 1);
      acc[i][j0] = mfma32_chunk(acc[i][j0], fa(cur, i), fb(cur, j0));
      acc[i][j0 + 1] = mfma32_chunk(acc[i][j0 + 1], fa(cur, i), fb(cur, j0 + 1));
      nxt[r] = __builtin_bit_cast(bf16x8, L[frag_addr(r, nks)]);
      if (with_dma) dma(r, rW, rX, dma_base);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto slot_of = [&](auto s_) -> const u32x4* {
    constexpr int S = decltype(s_)::value & 3;
    if constexpr (S == 0) return L0;
    else if constexpr (S == 1) return L1;
    else if constexpr (S == 2) return L2;
    else return L3;
  };
  const i32x4 none{0, 0, 0, 0};
  auto stage = [&](int kt, auto s_) {
    using S = decltype(s_);
    const u32x4* cur = slot_of(s_);
    kstep(fr0, fr1, cur, 1, false, none, none, 0);
    wait_vmcnt<2 * PER>();  // stage kt+1 landed (kt+2, kt+3 may still be in flight)
    lds_barrier();
    kstep(fr1, fr0, slot_of(std::integral_constant<int, S::value + 1>{}), 0, true, rsrc_w(kt + 4), rsrc_x(kt + 4),
          base[S::value & 3]);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;

#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const i32x4 rW = rsrc_w(s), rX = rsrc_x(s);
#pragma unroll
    for (int i = 0; i < PER; ++i) dma(i, rW, rX, base[s]);
  }
  wait_vmcnt<3 * PER>();
  lds_barrier();
#pragma unroll
  for (int r = 0; r < 8; ++r) fr0[r] = __builtin_bit_cast(bf16x8, L0[frag_addr(r, 0)]);
  int kt = 0;
  for (; kt + 4 <= nk; kt += 4) {
    stage(kt, I0{});
    stage(kt + 1, I1{});
    stage(kt + 2, I2{});
    stage(kt + 3, I3{});
  }
  if (kt < nk) {  // K is a multiple of 64: at most two stages remain (slots 0, 1)
    stage(kt, I0{});
    stage(kt + 1, I1{});
  }
  wait_vmcnt<0>();  // the empty DMAs issued past the end have retired

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = m0 + wm * 128 + 32 * j + l32;
      if (t < a.M) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int f = n0 + wn * 128 + 32 * i + 8 * g + 4 * lh;
          epilogue<T, EPI>(a, t, f, f32x4{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]});
        }
      }
    }
}

template <typename T, typename C>
hipError_t launch_cfg(const GemmArgs& a, hipStream_t s) {
  if (a.N % C::BN != 0 || a.K % (2 * C::BK) != 0 || a.M <= 0) return hipErrorInvalidValue;
  // 32-bit buffer offsets: a tile's rows times the row pitch must stay below 2^31
  if ((int64_t)C::BN * a.K * (int64_t)sizeof(T) >= (1ll << 31) ||
      (int64_t)C::BM * a.ldx * (int64_t)sizeof(T) >= (1ll << 31))
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

hipError_t launch_big(const GemmArgs& a, hipStream_t s) {
  using C = BigCfg;
  if (a.N % C::BN != 0 || a.K % (2 * C::BK) != 0 || a.M <= 0) return hipErrorInvalidValue;
  if ((int64_t)C::BN * a.K * 2 >= (1ll << 31) || (int64_t)C::BM * a.ldx * 2 >= (1ll << 31)) return hipErrorInvalidValue;
  const int grid = (a.N / C::BN) * ((a.M + C::BM - 1) / C::BM);
  switch (a.epi) {
    case Epi::QKV: gemm_big_kernel<0><<<grid, C::NT, 0, s>>>(a); break;
    case Epi::RESID_H: gemm_big_kernel<1><<<grid, C::NT, 0, s>>>(a); break;
    case Epi::SWIGLU: gemm_big_kernel<2><<<grid, C::NT, 0, s>>>(a); break;
    case Epi::RESID_OUT: gemm_big_kernel<3><<<grid, C::NT, 0, s>>>(a); break;
  }
  return hipGetLastError();
}

using SmallBF = Cfg<bf16, 64, 64, 2, 2>;
using LargeF = Cfg<float, 256, 256, 2, 4>;
using SmallF = Cfg<float, 64, 64, 2, 2>;

}  // namespace

int gemm_tile_n(GemmTile t) { return t == GemmTile::LARGE ? 256 : 64; }

hipError_t launch_gemm(DType t, GemmTile tile, const GemmArgs& a, hipStream_t s) {
  if (t == DType::BF16)
    return tile == GemmTile::LARGE ? launch_big(a, s) : launch_cfg<bf16, SmallBF>(a, s);
  return tile == GemmTile::LARGE ? launch_cfg<float, LargeF>(a, s) : launch_cfg<float, SmallF>(a, s);
}

}  // namespace llk
