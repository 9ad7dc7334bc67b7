// Host-only check of the library's runtime (validation, block manager, packing
// plan, RoPE table, uploads, paged K/V copies) under ASan/UBSan.  The kernel
// launch interface is replaced by stubs that run on host memory: "device"
// buffers are plain host allocations, uploads and K/V copies are executed, and
// compute launches are only recorded.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "llama_layer.h"
#include "../../decoder_block_amd/csrc/kernels.h"

static int g_fail = 0;
#define CHECK(c)                                                        \
  do {                                                                  \
    if (!(c)) {                                                         \
      std::fprintf(stderr, "CHECK failed %s:%d: %s\n", __FILE__, __LINE__, #c); \
      ++g_fail;                                                         \
    }                                                                   \
  } while (0)

static std::vector<std::string> g_log;
static int g_events = 0;
static int g_uploads = 0;
struct PackCall { int rows, cols, ldd, drows, row_mul, row_add, head_pairs; bool gamma; };
static std::vector<PackCall> g_packs;
static int g_attn_units = -1;  // work units of the last decode-attention launch
static std::vector<const void*> g_ins;   // x of each first-norm / final-norm launch
static std::vector<void*> g_outs;        // out of each down-projection launch
struct FinalCall { const void* gamma; void* y; };
static FinalCall g_final = {nullptr, nullptr};
// name of a stubbed launch that fails (empty: none), to test the rollback of a failed call
static std::string g_fail_launch;
// the static scratch buffer: a host allocation here, looked up on every call
static void* g_scratch = nullptr;
static int g_scratch_lookups = 0;
static bool fails(const char* what) { return g_fail_launch == what; }
static const float* g_ss_part = nullptr;  // partial sums the last folded norm wrote

namespace llk {
int gemm_tile_n(GemmTile t) { return t == GemmTile::LARGE ? 256 : 64; }
int skinny_ksplit(int, int N, int) { return N <= 8192 ? 4 : 1; }
size_t skinny_partial_bytes(int M, int N, int K) {
  const int ks = skinny_ksplit(M, N, K);
  return ks > 1 ? (size_t)ks * M * N * sizeof(float) : 0;
}
hipError_t launch_gemm(DType, GemmTile t, const GemmArgs& a, hipStream_t) {
  const char* tag = t == GemmTile::LARGE ? "L" : (t == GemmTile::SKINNY ? "K" : "S");
  g_log.push_back("gemm" + std::to_string((int)a.epi) + tag);
  if (fails(g_log.back().c_str())) return hipErrorLaunchFailure;
  // RMSNorm_2 folded into the o_proj split pass: the operand copy and the
  // partial sums come out of it, and the gate/up GEMM reads the same sums
  if (a.norm_gamma) {
    g_log.back() += "+norm2";
    if (a.epi != Epi::RESID_H || !a.norm_out || !a.ss_part || a.ss_nseg != (a.N + kNormSeg - 1) / kNormSeg)
      g_log.push_back("norm2-args-bad");
    g_ss_part = a.ss_part;
  }
  if (a.epi == Epi::SWIGLU && a.ss_part != nullptr && (a.ss_part != g_ss_part || a.ss_d != a.K || !(a.eps > 0.f)))
    g_log.push_back("norm2-sums-bad");
  if (a.epi == Epi::RESID_OUT) g_outs.push_back(a.out);
  if (t == GemmTile::SKINNY && a.split_ws_bytes < skinny_partial_bytes(a.M, a.N, a.K)) g_log.push_back("gemm-ws-short");
  return hipSuccess;
}
hipError_t launch_upload(const Upload& u, hipStream_t);
hipError_t launch_rms_rowscale(DType t, const void* x, float*, void* xt, int, int, float, const Upload* up,
                               hipStream_t s) {
  g_log.push_back("rms1");
  g_ins.push_back(x);
  // bf16 layers get the tiled operand copy of x; fp32 layers read x directly
  if ((t == DType::BF16) != (xt != nullptr)) g_log.push_back("rms1-xt-mismatch");
  if (up) {  // the batch riding on this launch is applied like a standalone upload
    if (launch_upload(*up, s) != hipSuccess) return hipErrorUnknown;
    --g_uploads;  // not a launch of its own
  }
  return hipSuccess;
}
hipError_t launch_rms_convert(DType, const float*, const float*, void*, float*, int, int, float, hipStream_t) {
  g_log.push_back("rms2");
  return hipSuccess;
}
hipError_t launch_rms_norm_out(DType, const void* x, const void* gamma, void* y, DType, int, int, float,
                               hipStream_t) {
  g_log.push_back("rms_final");
  g_ins.push_back(x);
  g_final = {gamma, y};
  return fails("rms_final") ? hipErrorLaunchFailure : hipSuccess;
}
hipError_t launch_attn_prefill(DType, const void*, void*, int, const CacheView&, const BatchView&, hipStream_t) {
  g_log.push_back("attn_prefill");
  return fails("attn_prefill") ? hipErrorLaunchFailure : hipSuccess;
}
int decode_split_keys() { return 1024; }
hipError_t launch_attn_decode(DType, const void*, float*, int, int, const CacheView&, const BatchView&, int units,
                              hipStream_t) {
  g_attn_units = units;
  g_log.push_back("attn_decode");
  return fails("attn_decode") ? hipErrorLaunchFailure : hipSuccess;
}
hipError_t launch_attn_decode_combine(DType, const float*, void*, int, int, int, const BatchView&, hipStream_t) {
  g_log.push_back("attn_combine");
  return hipSuccess;
}
hipError_t event_create(void** ev) {
  *ev = std::malloc(8);
  ++g_events;
  return hipSuccess;
}
hipError_t event_destroy(void* ev) {
  std::free(ev);
  --g_events;
  return hipSuccess;
}
hipError_t event_record(void*, hipStream_t) { return hipSuccess; }
hipError_t event_elapsed_ms(float* ms, void*, void*) {
  *ms = 0.5f;
  return hipSuccess;
}
hipError_t launch_pack(DType, const void*, const void* gamma, void*, int rows, int cols, int ldd, int drows,
                       int row_mul, int row_add, int head_pairs, hipStream_t) {
  g_packs.push_back({rows, cols, ldd, drows, row_mul, row_add, head_pairs, gamma != nullptr});
  return hipSuccess;
}
hipError_t launch_to_f32(DType, const void*, float* dst, int n, hipStream_t) {
  for (int i = 0; i < n; ++i) dst[i] = 1.0f;
  return hipSuccess;
}
hipError_t launch_fill(void* dst, size_t bytes, uint8_t byte, hipStream_t) {
  std::memset(dst, byte, bytes);
  g_log.push_back("fill");
  return hipSuccess;
}
hipError_t launch_zero(void* dst, size_t bytes, hipStream_t) {
  std::memset(dst, 0, bytes);
  return hipSuccess;
}
hipError_t launch_upload(const Upload& u, hipStream_t) {
  for (int i = 0; i < u.n; ++i) u.base[(u.idx[i] >> 31) & 1][u.idx[i] & 0x7fffffff] = u.val[i];
  ++g_uploads;
  return hipSuccess;
}
hipError_t scratch_region(void** ptr, size_t* bytes) {
  if (!g_scratch && posix_memalign(&g_scratch, 256, LLAMA_SCRATCH_BYTES) != 0) return hipErrorOutOfMemory;
  ++g_scratch_lookups;
  *ptr = g_scratch;
  *bytes = LLAMA_SCRATCH_BYTES;
  return hipSuccess;
}
hipError_t copy_to_device(void* dst, const void* src, size_t bytes, hipStream_t) {
  std::memcpy(dst, src, bytes);
  return hipSuccess;
}
hipError_t stream_sync(hipStream_t) { return hipSuccess; }
hipError_t launch_kv_copy(DType t, const CacheView& c, int seq, int start, int n, void* k, void* v, bool to_cache,
                          hipStream_t) {
  if (fails("kv_copy")) return hipErrorLaunchFailure;
  const size_t es = t == DType::F32 ? 4 : 2;
  char* kp = (char*)c.k_pool;
  char* vp = (char*)c.v_pool;
  for (int i = 0; i < n; ++i)
    for (int g = 0; g < c.G; ++g)
      for (int d = 0; d < c.D; ++d) {
        const int pos = start + i;
        const size_t blk = (size_t)c.block_table[(size_t)seq * c.max_blocks + pos / 16];
        const size_t ko = ((blk * c.G + g) * 16 + pos % 16) * c.D + d;
        const size_t vo = ((blk * c.G + g) * c.D + d) * 16 + pos % 16;
        const size_t lo = ((size_t)i * c.G + g) * c.D + d;
        if (to_cache) {
          std::memcpy(kp + ko * es, (char*)k + lo * es, es);
          std::memcpy(vp + vo * es, (char*)v + lo * es, es);
        } else {
          std::memcpy((char*)k + lo * es, kp + ko * es, es);
          std::memcpy((char*)v + lo * es, vp + vo * es, es);
        }
      }
  return hipSuccess;
}
}  // namespace llk

static void* aligned_buf(size_t n) {
  void* p = nullptr;
  if (posix_memalign(&p, 256, n ? n : 256) != 0) std::abort();
  std::memset(p, 0, n);
  return p;
}

static llama_layer_config tiny(llama_dtype dt = LLAMA_DTYPE_F32) {
  llama_layer_config c;
  c.hidden_size = 256;
  c.intermediate_size = 688;
  c.num_attention_heads = 4;
  c.num_key_value_heads = 2;
  c.rms_norm_eps = 1e-5f;
  c.rope_theta = 10000.f;
  c.max_position = 80;
  c.dtype = dt;
  c.rope_style = LLAMA_ROPE_INTERLEAVED;
  return c;
}

int main() {
  size_t bytes = 0;
  // ---- config validation ----
  llama_layer_config c = tiny();
  CHECK(llama_layer_packed_bytes(&c, &bytes) == LLAMA_OK && bytes > 0);
  c.num_key_value_heads = 3;
  CHECK(llama_layer_packed_bytes(&c, &bytes) == LLAMA_ERR_SHAPE);  // H % G != 0
  c = tiny();
  c.hidden_size = 260;
  CHECK(llama_layer_packed_bytes(&c, &bytes) == LLAMA_ERR_SHAPE);  // d % H != 0
  c = tiny();
  c.dtype = 7;
  CHECK(llama_layer_packed_bytes(&c, &bytes) == LLAMA_ERR_DTYPE);
  c = tiny();
  c.rms_norm_eps = 0.f;
  CHECK(llama_layer_packed_bytes(&c, &bytes) == LLAMA_ERR_INVALID_ARG);
  c = tiny();
  c.hidden_size = 4 * 96;  // D = 96
  CHECK(llama_layer_packed_bytes(&c, &bytes) == LLAMA_ERR_UNSUPPORTED);
  c = tiny();
  CHECK(llama_layer_packed_bytes(nullptr, &bytes) == LLAMA_ERR_INVALID_ARG);
  CHECK(llama_kv_cache_bytes(&c, 8, 32, 2, &bytes) == LLAMA_ERR_UNSUPPORTED);

  // ---- create: packing plan and RoPE table ----
  c = tiny();
  CHECK(llama_layer_packed_bytes(&c, &bytes) == LLAMA_OK);
  void* packed = aligned_buf(bytes);
  std::vector<void*> wbufs;
  llama_layer_weights w;
  const void** wp = reinterpret_cast<const void**>(&w);
  for (int i = 0; i < 9; ++i) {
    wbufs.push_back(aligned_buf(256 * 1024 * 4));
    wp[i] = wbufs.back();
  }
  llama_layer* L = nullptr;
  llama_layer_weights wnull = w;
  wnull.up_proj = nullptr;
  CHECK(llama_layer_create(&c, &wnull, packed, nullptr, &L) == LLAMA_ERR_INVALID_ARG && L == nullptr);
  CHECK(llama_layer_create(&c, &w, packed, nullptr, &L) == LLAMA_OK && L != nullptr);
  CHECK(g_packs.size() == 7);
  if (g_packs.size() == 7) {
    // q, k, v rows stacked; gate/up interleaved; down padded to a multiple of 128 columns
    CHECK(g_packs[0].rows == 256 && g_packs[0].row_add == 0 && g_packs[0].gamma);
    CHECK(g_packs[1].rows == 128 && g_packs[1].row_add == 256 && g_packs[1].gamma);
    CHECK(g_packs[2].rows == 128 && g_packs[2].row_add == 384 && g_packs[2].gamma);
    CHECK(!g_packs[3].gamma && g_packs[3].rows == 256);
    CHECK(g_packs[4].row_mul == 2 && g_packs[4].row_add == 0 && !g_packs[4].gamma);
    CHECK(g_packs[5].row_mul == 2 && g_packs[5].row_add == 1 && !g_packs[5].gamma);
    CHECK(g_packs[6].cols == 688 && g_packs[6].ldd == 768 && !g_packs[6].gamma);
    // destination rows of each packed matrix: qkv 512, o 256, gate/up 2 x 768, down 256
    CHECK(g_packs[0].drows == 512 && g_packs[1].drows == 512 && g_packs[2].drows == 512);
    CHECK(g_packs[3].drows == 256 && g_packs[4].drows == 1536 && g_packs[5].drows == 1536);
    CHECK(g_packs[6].drows == 256);
    for (const PackCall& pc : g_packs) CHECK(pc.head_pairs == 0);  // interleaved RoPE: rows in order
  }
  // half-split RoPE: the q and k rows of each head are reordered, nothing else
  {
    llama_layer_config ch = c;
    ch.rope_style = 7;
    CHECK(llama_layer_packed_bytes(&ch, &bytes) == LLAMA_ERR_INVALID_ARG);
    ch.rope_style = LLAMA_ROPE_HALF_SPLIT;
    g_packs.clear();
    llama_layer* Lh = nullptr;
    CHECK(llama_layer_create(&ch, &w, packed, nullptr, &Lh) == LLAMA_OK && Lh != nullptr);
    CHECK(g_packs.size() == 7);
    if (g_packs.size() == 7) {
      CHECK(g_packs[0].head_pairs == 64 && g_packs[1].head_pairs == 64);
      for (int i = 2; i < 7; ++i) CHECK(g_packs[i].head_pairs == 0);
    }
    CHECK(llama_layer_destroy(Lh) == LLAMA_OK);
  }
  // the RoPE tables are the last two sections of the packed buffer
  {
    const int half = 32, P = 80;
    const size_t tbl = (size_t)P * half * sizeof(float);
    const size_t sin_off = bytes - ((tbl + 255) & ~size_t(255));
    const size_t cos_off = sin_off - ((tbl + 255) & ~size_t(255));
    const float* cs = (const float*)((char*)packed + cos_off);
    const float* sn = (const float*)((char*)packed + sin_off);
    for (int p : {0, 1, 37, 79})
      for (int i : {0, 1, 17, 31}) {
        const double a = p * std::pow(10000.0, -2.0 * i / 64);
        CHECK(std::fabs(cs[p * half + i] - (float)std::cos(a)) < 1e-7);
        CHECK(std::fabs(sn[p * half + i] - (float)std::sin(a)) < 1e-7);
      }
  }
  size_t wsb = 0;
  CHECK(llama_layer_workspace_bytes(L, 64, 1, &wsb) == LLAMA_OK && wsb > 0);
  CHECK(llama_layer_workspace_bytes(L, 4, 8, &wsb) == LLAMA_ERR_INVALID_ARG);

  // ---- cache ----
  const int NB = 9;
  CHECK(llama_kv_cache_bytes(&c, NB, 16, 3, &bytes) == LLAMA_OK);
  void* pool = aligned_buf(bytes);
  llama_kv_cache* C = nullptr;
  int32_t bad_order[NB];
  for (int i = 0; i < NB; ++i) bad_order[i] = i % 6;
  CHECK(llama_kv_cache_create(&c, NB, 16, 3, bad_order, pool, &C) == LLAMA_ERR_INVALID_ARG);
  int32_t order[NB] = {5, 8, 2, 7, 0, 3, 1, 6, 4};
  CHECK(llama_kv_cache_create(&c, NB, 16, 3, order, pool, &C) == LLAMA_OK);
  int32_t s0 = -1, s1 = -1, s2 = -1, s3 = -1, n = 0;
  CHECK(llama_kv_cache_add_seq(C, &s0) == LLAMA_OK && s0 == 0);
  CHECK(llama_kv_cache_add_seq(C, &s1) == LLAMA_OK && s1 == 1);
  CHECK(llama_kv_cache_add_seq(C, &s2) == LLAMA_OK && s2 == 2);
  CHECK(llama_kv_cache_add_seq(C, &s3) == LLAMA_ERR_CACHE_FULL);
  CHECK(llama_kv_cache_free_seq(C, s2) == LLAMA_OK);
  CHECK(llama_kv_cache_free_seq(C, s2) == LLAMA_ERR_BAD_SEQ);

  // prefill 2 x 20 tokens: 2 blocks each, handed out in `order`
  const size_t kWsBytes = 1 << 22;
  void* ws = aligned_buf(kWsBytes);
  void* x = aligned_buf(2 * 20 * 256 * 4);
  void* out = aligned_buf(2 * 20 * 256 * 4);
  int32_t ids[2] = {s0, s1};
  g_log.clear();
  CHECK(llama_layer_prefill(L, C, 2, 20, ids, x, out, LLAMA_DTYPE_BF16, ws, kWsBytes, nullptr) == LLAMA_ERR_DTYPE);
  CHECK(llama_layer_prefill(L, C, 2, 20, ids, x, out, LLAMA_DTYPE_F32, ws, kWsBytes, nullptr) == LLAMA_OK);
  {
    const std::vector<std::string> want = {"rms1", "gemm0S", "attn_prefill", "gemm1S", "rms2", "gemm2S", "gemm3S"};
    CHECK(g_log == want);
  }
  CHECK(llama_kv_cache_seq_len(C, s0, &n) == LLAMA_OK && n == 20);
  CHECK(llama_kv_cache_free_blocks(C, &n) == LLAMA_OK && n == NB - 4);
  // block table rows: seq 0 got order[0], order[1]; seq 1 got order[2], order[3]
  size_t tab_off = 0;
  {
    size_t kvb = (size_t)NB * 2 * 16 * 64 * 4;
    tab_off = 2 * ((kvb + 255) & ~size_t(255));
  }
  const int32_t* tab = (const int32_t*)((char*)pool + tab_off);
  const int maxb = 5;  // ceil(80 / 16)
  CHECK(tab[0 * maxb + 0] == 5 && tab[0 * maxb + 1] == 8);
  CHECK(tab[1 * maxb + 0] == 2 && tab[1 * maxb + 1] == 7);
  const int32_t* desc = (const int32_t*)ws;
  CHECK(desc[0] == s0 && desc[1] == 0 && desc[2] == s1 && desc[3] == 0);

  // errors leave the state unchanged
  int32_t dup[2] = {s0, s0};
  CHECK(llama_layer_prefill(L, C, 2, 4, dup, x, out, LLAMA_DTYPE_F32, ws, kWsBytes, nullptr) == LLAMA_ERR_BAD_SEQ);
  int32_t unk[1] = {2};
  CHECK(llama_layer_decode(L, C, 1, unk, x, out, LLAMA_DTYPE_F32, ws, kWsBytes, nullptr) == LLAMA_ERR_BAD_SEQ);
  CHECK(llama_layer_prefill(L, C, 1, 61, ids, x, out, LLAMA_DTYPE_F32, ws, kWsBytes, nullptr) == LLAMA_ERR_POSITION);
  CHECK(llama_layer_prefill(L, C, 2, 60, ids, x, out, LLAMA_DTYPE_F32, ws, kWsBytes, nullptr) == LLAMA_ERR_CACHE_FULL);
  CHECK(llama_kv_cache_seq_len(C, s0, &n) == LLAMA_OK && n == 20);
  CHECK(llama_kv_cache_free_blocks(C, &n) == LLAMA_OK && n == NB - 4);
  CHECK(llama_layer_prefill(L, C, 1, 4, ids, (char*)x + 4, out, LLAMA_DTYPE_F32, ws, kWsBytes, nullptr) ==
        LLAMA_ERR_INVALID_ARG);

  // a workspace smaller than the call needs is refused before any device work
  {
    size_t need = 0;
    CHECK(llama_layer_workspace_bytes(L, 2 * 4, 2, &need) == LLAMA_OK && need <= kWsBytes);
    g_log.clear();
    CHECK(llama_layer_prefill(L, C, 2, 4, ids, x, out, LLAMA_DTYPE_F32, ws, need - 1, nullptr) ==
          LLAMA_ERR_INVALID_ARG);
    CHECK(llama_layer_decode(L, C, 2, ids, x, out, LLAMA_DTYPE_F32, ws, 0, nullptr) == LLAMA_ERR_INVALID_ARG);
    CHECK(g_log.empty());
    CHECK(llama_kv_cache_seq_len(C, s0, &n) == LLAMA_OK && n == 20);
    CHECK(llama_kv_cache_free_blocks(C, &n) == LLAMA_OK && n == NB - 4);
  }
  // a launch that fails part-way leaves lengths, blocks and the free list as they were
  {
    const std::vector<int32_t> tab_before(tab, tab + 3 * maxb);
    for (const char* k : {"attn_prefill", "gemm3S"}) {
      g_fail_launch = k;
      CHECK(llama_layer_prefill(L, C, 2, 13, ids, x, out, LLAMA_DTYPE_F32, ws, kWsBytes, nullptr) == LLAMA_ERR_HIP);
      g_fail_launch.clear();
      CHECK(llama_kv_cache_seq_len(C, s0, &n) == LLAMA_OK && n == 20);
      CHECK(llama_kv_cache_seq_len(C, s1, &n) == LLAMA_OK && n == 20);
      CHECK(llama_kv_cache_free_blocks(C, &n) == LLAMA_OK && n == NB - 4);
    }
    CHECK(tab_before[0] == tab[0] && tab_before[1] == tab[1] && tab_before[maxb + 1] == tab[maxb + 1]);
    // the decode below takes order[4] for seq 0's third block: the free list
    // came back in its original order
  }

  // decode: 12 steps on seq 0 (20 -> 32 crosses into a third block only at 32)
  g_log.clear();
  for (int t = 0; t < 12; ++t)
    CHECK(llama_layer_decode(L, C, 1, ids, x, out, LLAMA_DTYPE_F32, ws, kWsBytes, nullptr) == LLAMA_OK);
  CHECK(llama_kv_cache_seq_len(C, s0, &n) == LLAMA_OK && n == 32);
  CHECK(llama_kv_cache_free_blocks(C, &n) == LLAMA_OK && n == NB - 4);
  CHECK(llama_layer_decode(L, C, 1, ids, x, out, LLAMA_DTYPE_F32, ws, kWsBytes, nullptr) == LLAMA_OK);
  CHECK(llama_kv_cache_free_blocks(C, &n) == LLAMA_OK && n == NB - 5);
  CHECK(tab[0 * maxb + 2] == 0);  // order[4]
  CHECK(desc[0] == s0 && desc[1] == 32);
  CHECK(g_attn_units == 1);  // one sequence, 33 keys: one chunk
  CHECK(g_log.size() == 13 * 8 && g_log[2] == "attn_decode" && g_log[3] == "attn_combine");

  // LLAMA_LAYER_POISON: the workspace is filled before the call's uploads and kernels
  {
    setenv("LLAMA_LAYER_POISON", "1", 1);
    g_log.clear();
    CHECK(llama_layer_decode(L, C, 1, ids, x, out, LLAMA_DTYPE_F32, ws, kWsBytes, nullptr) == LLAMA_OK);
    CHECK(!g_log.empty() && g_log[0] == "fill" && g_log.size() == 9);
    CHECK(desc[0] == s0 && desc[1] == 33);  // descriptors written after the fill
    unsetenv("LLAMA_LAYER_POISON");
    g_log.clear();
    CHECK(llama_layer_decode(L, C, 1, ids, x, out, LLAMA_DTYPE_F32, ws, kWsBytes, nullptr) == LLAMA_OK);
    CHECK(g_log.size() == 8 && g_log[0] == "rms1");
    CHECK(desc[1] == 34);
  }

  // decode without allocation: the workspace is the static scratch buffer
  {
    g_log.clear();
    const int lookups = g_scratch_lookups;
    CHECK(llama_layer_decode_noalloc(L, C, 1, ids, x, out, LLAMA_DTYPE_F32, nullptr) == LLAMA_OK);
    CHECK(g_scratch_lookups == lookups + 1 && g_scratch != nullptr);
    CHECK(g_log.size() == 8 && g_log[2] == "attn_decode");
    const int32_t* sdesc = (const int32_t*)g_scratch;
    CHECK(sdesc[0] == s0 && sdesc[1] == 35);
    CHECK(llama_kv_cache_seq_len(C, s0, &n) == LLAMA_OK && n == 36);
    // validation comes first: nothing is looked up or launched for a bad call
    g_log.clear();
    CHECK(llama_layer_decode_noalloc(L, C, 1, ids, nullptr, out, LLAMA_DTYPE_F32, nullptr) == LLAMA_ERR_INVALID_ARG);
    CHECK(llama_layer_decode_noalloc(L, C, 1, ids, x, out, LLAMA_DTYPE_BF16, nullptr) == LLAMA_ERR_DTYPE);
    CHECK(llama_layer_decode_noalloc(nullptr, C, 1, ids, x, out, LLAMA_DTYPE_F32, nullptr) == LLAMA_ERR_INVALID_ARG);
    // a batch whose workspace exceeds the buffer is refused before any HIP call
    size_t big = 0;
    int32_t bigb = 1;
    while (llama_layer_workspace_bytes(L, bigb, bigb, &big) == LLAMA_OK && big <= LLAMA_SCRATCH_BYTES) bigb *= 2;
    CHECK(big > LLAMA_SCRATCH_BYTES);
    std::vector<int32_t> many(bigb, s0);
    void* xb = aligned_buf((size_t)bigb * 256 * 4);
    CHECK(llama_layer_decode_noalloc(L, C, bigb, many.data(), xb, xb, LLAMA_DTYPE_F32, nullptr) == LLAMA_ERR_SCRATCH);
    std::free(xb);
    CHECK(g_log.empty() && g_scratch_lookups == lookups + 1);
    CHECK(llama_kv_cache_seq_len(C, s0, &n) == LLAMA_OK && n == 36);
    CHECK(std::string(llama_status_string(LLAMA_ERR_SCRATCH)).find("scratch") != std::string::npos);
  }

  // per-kernel timing: two events per launch, totals per kernel family
  {
    CHECK(llama_layer_profile_enable(L, 1) == LLAMA_OK);
    CHECK(llama_layer_decode(L, C, 1, ids, x, out, LLAMA_DTYPE_F32, ws, kWsBytes, nullptr) == LLAMA_OK);
    CHECK(llama_layer_decode(L, C, 1, ids, x, out, LLAMA_DTYPE_F32, ws, kWsBytes, nullptr) == LLAMA_OK);
    llama_kernel_time kt[16];
    int32_t nk = 0;
    CHECK(llama_layer_profile_read(L, kt, 16, &nk, 1) == LLAMA_OK && nk == 8);
    bool seen = false;
    for (int i = 0; i < nk; ++i) {
      CHECK(kt[i].launches == 2 && std::fabs(kt[i].total_ms - 1.0) < 1e-9);
      if (std::string(kt[i].name) == "attn_decode_split") seen = true;
    }
    CHECK(seen);
    CHECK(llama_layer_profile_read(L, kt, 16, &nk, 0) == LLAMA_OK && nk == 0);
    CHECK(llama_layer_profile_enable(L, 0) == LLAMA_OK);
    CHECK(g_events == 0);
  }

  // K/V write then read back through the paged layout
  {
    int32_t s = -1;
    CHECK(llama_kv_cache_free_seq(C, s1) == LLAMA_OK);
    CHECK(llama_kv_cache_add_seq(C, &s) == LLAMA_OK);
    const int ntok = 37, G = 2, D = 64;
    std::vector<float> k(ntok * G * D), v(ntok * G * D), k2(ntok * G * D), v2(ntok * G * D);
    for (size_t i = 0; i < k.size(); ++i) {
      k[i] = (float)i;
      v[i] = -(float)i;
    }
    int32_t fb0 = 0, fb1 = 0;
    CHECK(llama_kv_cache_free_blocks(C, &fb0) == LLAMA_OK);
    g_fail_launch = "kv_copy";
    CHECK(llama_kv_cache_write(C, s, 30, k.data(), v.data(), nullptr) == LLAMA_ERR_HIP);
    g_fail_launch.clear();
    CHECK(llama_kv_cache_free_blocks(C, &fb1) == LLAMA_OK && fb1 == fb0);
    CHECK(llama_kv_cache_seq_len(C, s, &n) == LLAMA_OK && n == 0);
    CHECK(llama_kv_cache_write(C, s, 30, k.data(), v.data(), nullptr) == LLAMA_OK);
    CHECK(llama_kv_cache_write(C, s, 7, k.data() + 30 * G * D, v.data() + 30 * G * D, nullptr) == LLAMA_OK);
    CHECK(llama_kv_cache_read(C, s, 0, ntok, k2.data(), v2.data(), nullptr) == LLAMA_OK);
    CHECK(k == k2 && v == v2);
    CHECK(llama_kv_cache_read(C, s, 30, 8, k2.data(), v2.data(), nullptr) == LLAMA_ERR_POSITION);
  }
  CHECK(llama_kv_cache_free_seq(C, s0) == LLAMA_OK);
  CHECK(llama_kv_cache_destroy(C) == LLAMA_OK);
  CHECK(llama_layer_destroy(L) == LLAMA_OK);

  // bf16 layer: few tokens take the split-K skinny GEMMs, whose partial sums
  // fit a workspace sized for any larger token count
  {
    llama_layer_config cb = tiny();
    cb.dtype = LLAMA_DTYPE_BF16;
    cb.max_position = 512;
    size_t pb = 0;
    CHECK(llama_layer_packed_bytes(&cb, &pb) == LLAMA_OK);
    void* packed_b = aligned_buf(pb);
    llama_layer* Lb = nullptr;
    CHECK(llama_layer_create(&cb, &w, packed_b, nullptr, &Lb) == LLAMA_OK);
    size_t w1 = 0, w64 = 0, w100 = 0, w128 = 0, w1000 = 0;
    CHECK(llama_layer_workspace_bytes(Lb, 1, 1, &w1) == LLAMA_OK);
    CHECK(llama_layer_workspace_bytes(Lb, 64, 1, &w64) == LLAMA_OK);
    CHECK(llama_layer_workspace_bytes(Lb, 100, 1, &w100) == LLAMA_OK);
    CHECK(llama_layer_workspace_bytes(Lb, 128, 1, &w128) == LLAMA_OK);
    CHECK(llama_layer_workspace_bytes(Lb, 1000, 1, &w1000) == LLAMA_OK);
    CHECK(w1 <= w64 && w64 <= w100 && w100 <= w128 && w128 <= w1000);
    size_t cbytes = 0;
    CHECK(llama_kv_cache_bytes(&cb, 40, 16, 2, &cbytes) == LLAMA_OK);
    void* pool_b = aligned_buf(cbytes);
    llama_kv_cache* Cb = nullptr;
    CHECK(llama_kv_cache_create(&cb, 40, 16, 2, nullptr, pool_b, &Cb) == LLAMA_OK);
    int32_t sa = -1, sb = -1;
    CHECK(llama_kv_cache_add_seq(Cb, &sa) == LLAMA_OK && llama_kv_cache_add_seq(Cb, &sb) == LLAMA_OK);
    void* wsb2 = aligned_buf(w1000);
    void* xb = aligned_buf(2 * 300 * 256 * 2);
    void* ob = aligned_buf(2 * 300 * 256 * 4);
    int32_t ids2[2] = {sa, sb};
    g_log.clear();
    CHECK(llama_layer_prefill(Lb, Cb, 2, 50, ids2, xb, ob, LLAMA_DTYPE_F32, wsb2, w1000, nullptr) == LLAMA_OK);
    {
      // split-K o_proj: RMSNorm_2 rides on its split pass
      const std::vector<std::string> want = {"rms1", "gemm0K", "attn_prefill", "gemm1K+norm2", "gemm2K", "gemm3K"};
      CHECK(g_log == want);
    }
    g_log.clear();
    const int uploads_before = g_uploads;
    CHECK(llama_layer_decode(Lb, Cb, 2, ids2, xb, ob, LLAMA_DTYPE_BF16, wsb2, w1000, nullptr) == LLAMA_OK);
    CHECK(g_uploads == uploads_before);  // block table + descriptors ride on the first norm launch
    CHECK(g_log.size() == 7 && g_log[1] == "gemm0K" && g_log[4] == "gemm1K+norm2" && g_log[5] == "gemm2K" &&
          g_log[6] == "gemm3K");
    g_log.clear();
    CHECK(llama_layer_prefill(Lb, Cb, 1, 300, ids2, xb, ob, LLAMA_DTYPE_F32, wsb2, w1000, nullptr) == LLAMA_OK);
    {
      const std::vector<std::string> want = {"rms1", "gemm0L", "attn_prefill", "gemm1L", "rms2", "gemm2L", "gemm3L"};
      CHECK(g_log == want);
    }
    CHECK(llama_kv_cache_destroy(Cb) == LLAMA_OK);
    CHECK(llama_layer_destroy(Lb) == LLAMA_OK);
    std::free(pool_b);
    std::free(wsb2);
    std::free(xb);
    std::free(ob);
    std::free(packed_b);
  }
  // ---- stack of 3 layers over one 3-layer cache ----
  {
    const int NL = 3;
    std::vector<void*> packs;
    std::vector<llama_layer*> Ls;
    llama_layer_config cs = tiny();
    for (int l = 0; l < NL; ++l) {
      size_t pb = 0;
      CHECK(llama_layer_packed_bytes(&cs, &pb) == LLAMA_OK);
      packs.push_back(aligned_buf(pb));
      llama_layer* Ll = nullptr;
      CHECK(llama_layer_create(&cs, &w, packs.back(), nullptr, &Ll) == LLAMA_OK);
      Ls.push_back(Ll);
    }
    void* gamma_f = aligned_buf(256 * 4);
    llama_stack* S = nullptr;
    CHECK(llama_stack_create(Ls.data(), 0, gamma_f, &S) == LLAMA_ERR_INVALID_ARG);
    CHECK(llama_stack_create(Ls.data(), NL, nullptr, &S) == LLAMA_ERR_INVALID_ARG);
    {
      // a layer with another config does not join the stack
      llama_layer_config co = cs;
      co.rope_theta = 500000.f;
      size_t pb = 0;
      CHECK(llama_layer_packed_bytes(&co, &pb) == LLAMA_OK);
      void* po = aligned_buf(pb);
      llama_layer* Lo = nullptr;
      CHECK(llama_layer_create(&co, &w, po, nullptr, &Lo) == LLAMA_OK);
      llama_layer* mixed[2] = {Ls[0], Lo};
      CHECK(llama_stack_create(mixed, 2, gamma_f, &S) == LLAMA_ERR_SHAPE && S == nullptr);
      CHECK(llama_layer_destroy(Lo) == LLAMA_OK);
      std::free(po);
    }
    CHECK(llama_stack_create(Ls.data(), NL, gamma_f, &S) == LLAMA_OK && S != nullptr);
    size_t b1 = 0, b3 = 0;
    CHECK(llama_kv_cache_bytes_layers(&cs, 1, 6, 16, 2, &b1) == LLAMA_OK);
    CHECK(llama_kv_cache_bytes(&cs, 6, 16, 2, &bytes) == LLAMA_OK && bytes == b1);
    CHECK(llama_kv_cache_bytes_layers(&cs, NL, 6, 16, 2, &b3) == LLAMA_OK);
    const size_t layer_pool = (size_t)6 * 2 * 16 * 64 * 4;  // blocks x G x 16 x D x 4 bytes
    CHECK(b3 == b1 + 2 * (NL - 1) * layer_pool);
    CHECK(llama_kv_cache_bytes_layers(&cs, 0, 6, 16, 2, &b3) == LLAMA_ERR_INVALID_ARG);
    void* pool3 = aligned_buf(b3);
    llama_kv_cache* C3 = nullptr;
    CHECK(llama_kv_cache_create_layers(&cs, NL, 6, 16, 2, nullptr, pool3, &C3) == LLAMA_OK);
    int32_t nl = 0;
    CHECK(llama_kv_cache_num_layers(C3, &nl) == LLAMA_OK && nl == NL);
    int32_t sa = -1, sb = -1;
    CHECK(llama_kv_cache_add_seq(C3, &sa) == LLAMA_OK && llama_kv_cache_add_seq(C3, &sb) == LLAMA_OK);
    int32_t sids[2] = {sa, sb};
    size_t wsz = 0, lwsz = 0;
    CHECK(llama_stack_workspace_bytes(S, 40, 2, &wsz) == LLAMA_OK);
    CHECK(llama_layer_workspace_bytes(Ls[0], 40, 2, &lwsz) == LLAMA_OK);
    CHECK(wsz >= lwsz + 2 * 40 * 256 * 4);
    void* ws3 = aligned_buf(wsz);
    void* x3 = aligned_buf(40 * 256 * 4);
    void* y3 = aligned_buf(40 * 256 * 4);
    // a multi-layer cache is the stack's; a single-layer cache is the layer's
    CHECK(llama_layer_prefill(Ls[0], C3, 2, 20, sids, x3, y3, LLAMA_DTYPE_F32, ws3, wsz, nullptr) == LLAMA_ERR_SHAPE);
    llama_kv_cache* C1 = nullptr;
    void* pool1 = aligned_buf(b1);
    CHECK(llama_kv_cache_create(&cs, 6, 16, 2, nullptr, pool1, &C1) == LLAMA_OK);
    int32_t s1a = -1;
    CHECK(llama_kv_cache_add_seq(C1, &s1a) == LLAMA_OK);
    CHECK(llama_stack_prefill(S, C1, 1, 20, &s1a, x3, y3, LLAMA_DTYPE_F32, ws3, wsz, nullptr) == LLAMA_ERR_SHAPE);
    CHECK(llama_kv_cache_destroy(C1) == LLAMA_OK);
    std::free(pool1);
    CHECK(llama_stack_prefill(S, C3, 2, 20, sids, x3, y3, LLAMA_DTYPE_BF16, ws3, wsz, nullptr) == LLAMA_ERR_DTYPE);

    g_log.clear();
    g_ins.clear();
    g_outs.clear();
    CHECK(llama_stack_prefill(S, C3, 2, 20, sids, x3, y3, LLAMA_DTYPE_F32, ws3, wsz, nullptr) == LLAMA_OK);
    {
      std::vector<std::string> want;
      for (int l = 0; l < NL; ++l)
        for (const char* k : {"rms1", "gemm0S", "attn_prefill", "gemm1S", "rms2", "gemm2S", "gemm3S"}) want.push_back(k);
      want.push_back("rms_final");
      CHECK(g_log == want);
    }
    // layer l + 1 reads what layer l wrote, the final norm reads the last layer's output
    CHECK(g_ins.size() == NL + 1 && g_outs.size() == NL);
    if (g_ins.size() == NL + 1 && g_outs.size() == NL) {
      CHECK(g_ins[0] == x3);
      for (int l = 0; l < NL; ++l) CHECK(g_ins[l + 1] == g_outs[l] && g_outs[l] != y3);
      CHECK(g_outs[0] != g_outs[1] && g_outs[1] != g_outs[2] && g_outs[0] == g_outs[2]);
    }
    CHECK(g_final.gamma == gamma_f && g_final.y == y3);
    CHECK(llama_kv_cache_seq_len(C3, sa, &n) == LLAMA_OK && n == 20);  // advanced once
    CHECK(llama_kv_cache_free_blocks(C3, &n) == LLAMA_OK && n == 2);
    g_log.clear();
    CHECK(llama_stack_decode(S, C3, 2, sids, x3, y3, LLAMA_DTYPE_F32, ws3, wsz, nullptr) == LLAMA_OK);
    CHECK(g_log.size() == NL * 8 + 1 && g_log.back() == "rms_final" && g_log[2] == "attn_decode");
    CHECK(g_attn_units == 2);  // two sequences of 21 keys
    CHECK(llama_kv_cache_seq_len(C3, sb, &n) == LLAMA_OK && n == 21);
    // per-layer pools: K/V written as [NL, n, G, D] come back per layer, unaliased
    {
      int32_t sc = -1;
      CHECK(llama_kv_cache_free_seq(C3, sb) == LLAMA_OK && llama_kv_cache_add_seq(C3, &sc) == LLAMA_OK);
      const int ntok = 19, G = 2, D = 64;
      const size_t per = (size_t)ntok * G * D;
      std::vector<float> k(NL * per), v(NL * per), k2(NL * per), v2(NL * per);
      for (size_t i = 0; i < k.size(); ++i) {
        k[i] = (float)i;
        v[i] = 0.5f - (float)i;
      }
      CHECK(llama_kv_cache_write(C3, sc, ntok, k.data(), v.data(), nullptr) == LLAMA_OK);
      CHECK(llama_kv_cache_read(C3, sc, 0, ntok, k2.data(), v2.data(), nullptr) == LLAMA_OK);
      CHECK(k == k2 && v == v2);
      // layer 1's K pool starts one layer's pool after layer 0's
      const float* kp = (const float*)pool3;
      int32_t blk0 = -1;
      {
        // first block of sc is the block at the table slot of sc
        const size_t tabo = 2 * ((NL * layer_pool + 255) & ~size_t(255));
        blk0 = ((const int32_t*)((char*)pool3 + tabo))[sc * 5 + 0];
      }
      const size_t lp = layer_pool / 4;
      CHECK(kp[lp + ((size_t)blk0 * G * 16) * D] == (float)per);  // layer 1, position 0, head 0, d 0
      CHECK(kp[2 * lp + ((size_t)blk0 * G * 16) * D + 5] == (float)(2 * per + 5));
    }
    {
      CHECK(llama_layer_profile_enable(Ls[NL - 1], 1) == LLAMA_OK);
      CHECK(llama_stack_decode(S, C3, 1, sids, x3, y3, LLAMA_DTYPE_F32, ws3, wsz, nullptr) == LLAMA_OK);
      llama_kernel_time kt[16];
      int32_t nk = 0;
      CHECK(llama_layer_profile_read(Ls[NL - 1], kt, 16, &nk, 1) == LLAMA_OK && nk == 9);
      bool seen = false;
      for (int i = 0; i < nk; ++i) seen |= std::string(kt[i].name) == "rms_final_norm";
      CHECK(seen);
      CHECK(llama_layer_profile_enable(Ls[NL - 1], 0) == LLAMA_OK);
    }
    CHECK(llama_stack_destroy(S) == LLAMA_OK);
    CHECK(llama_kv_cache_destroy(C3) == LLAMA_OK);
    for (llama_layer* Ll : Ls) CHECK(llama_layer_destroy(Ll) == LLAMA_OK);
    for (void* p : packs) std::free(p);
    std::free(gamma_f);
    std::free(pool3);
    std::free(ws3);
    std::free(x3);
    std::free(y3);
  }
  std::free(pool);
  std::free(ws);
  std::free(x);
  std::free(out);
  std::free(packed);
  for (void* p : wbufs) std::free(p);
  std::free(g_scratch);
  if (g_fail) {
    std::fprintf(stderr, "%d checks failed\n", g_fail);
    return 1;
  }
  std::printf("host_check: all checks passed\n");
  return 0;
}
