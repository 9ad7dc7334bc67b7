// Host runtime of the decoder-layer library: C ABI, argument validation, the
// paged-KV block manager, weight packing, workspace carving and the launch
// sequence of one prefill or decode call.
//
// The launch sequence follows the layer as the pages state it ("LLaMA3
// Block: from parts to engine", 4.2; "Chapter 10: the modern LLaMA
// architecture", section 9):
//   r1 = rowscale(x)                                  RMSNorm_1 statistics
//   [q | k | v] = r1 * x W'qkv^T, RoPE(q, k), k/v -> cache    (W' = W diag(gamma_1))
//   attn = causal GQA attention(q, cache)             prefill: flash; decode: split-K
//   h = x + attn Wo^T                                  fp32 residual stream
//   r2 = rowscale(h), hb = h * gamma_2 in the layer dtype   RMSNorm_2
//     (decode-sized calls: in the o_proj GEMM's split-K pass, with r2 finished
//     in the gate/up epilogue from per-segment sums of h^2)
//   s = SiLU(r2 * hb Wg^T) * (r2 * hb Wu^T)
//   out = h + s Wd^T
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <unordered_set>
#include <vector>

#include "../../include/llama_layer.h"
#include "kernels.h"

using llk::DType;

namespace {

constexpr int kBlock = 16;

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }
bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Shape {
  int d, I, I_pad, H, G, D, HD, KD, NQKV, NQKV_pad, max_pos;
  bool rope_half;  // RoPE pairs (i, i + D/2) instead of (2i, 2i+1)
  int d_rows;  // stored rows of W_o and W_down: d, rounded up to 256 for tiled bf16
  DType dt;
  size_t es;
};

// bf16 GEMM operands are stored in 256-row tiles: activation buffers hold the
// token count rounded up to 256 rows
size_t op_rows(const Shape& s, size_t T) { return s.dt == DType::BF16 ? (T + 255) / 256 * 256 : T; }

llama_status check_config(const llama_layer_config* c, Shape* s) {
  if (!c) return LLAMA_ERR_INVALID_ARG;
  if (c->dtype != LLAMA_DTYPE_F32 && c->dtype != LLAMA_DTYPE_BF16) return LLAMA_ERR_DTYPE;
  if (c->rope_style != LLAMA_ROPE_INTERLEAVED && c->rope_style != LLAMA_ROPE_HALF_SPLIT) return LLAMA_ERR_INVALID_ARG;
  if (c->hidden_size <= 0 || c->intermediate_size <= 0 || c->num_attention_heads <= 0 ||
      c->num_key_value_heads <= 0 || c->max_position <= 0)
    return LLAMA_ERR_INVALID_ARG;
  if (!(c->rms_norm_eps > 0.f) || !std::isfinite(c->rms_norm_eps) || !(c->rope_theta > 1.f) ||
      !std::isfinite(c->rope_theta))
    return LLAMA_ERR_INVALID_ARG;
  // "From Transformer to the LLaMA series", section 8: heads must split evenly
  if (c->num_attention_heads % c->num_key_value_heads != 0) return LLAMA_ERR_SHAPE;
  if (c->hidden_size % c->num_attention_heads != 0) return LLAMA_ERR_SHAPE;
  const int D = c->hidden_size / c->num_attention_heads;
  if (D % 2 != 0) return LLAMA_ERR_SHAPE;  // RoPE pairs need an even head_dim ("Chapter 10", section 3)
  if (D != 64 && D != 128) return LLAMA_ERR_UNSUPPORTED;
  if (c->dtype == LLAMA_DTYPE_F32 && D != 64) return LLAMA_ERR_UNSUPPORTED;
  const int R = c->num_attention_heads / c->num_key_value_heads;
  if (R > 32 || (R & (R - 1)) != 0) return LLAMA_ERR_UNSUPPORTED;
  if (c->hidden_size % 64 != 0 || c->intermediate_size % 8 != 0) return LLAMA_ERR_SHAPE;
  if ((int64_t)c->hidden_size > (1 << 16) || (int64_t)c->intermediate_size > (1 << 18) ||
      c->max_position > (1 << 22))
    return LLAMA_ERR_SHAPE;
  s->d = c->hidden_size;
  s->I = c->intermediate_size;
  s->I_pad = (c->intermediate_size + 127) / 128 * 128;
  s->H = c->num_attention_heads;
  s->G = c->num_key_value_heads;
  s->D = D;
  s->HD = s->H * D;
  s->KD = s->G * D;
  s->NQKV = s->HD + 2 * s->KD;
  s->NQKV_pad = (s->NQKV + 255) / 256 * 256;
  s->max_pos = c->max_position;
  s->dt = c->dtype == LLAMA_DTYPE_BF16 ? DType::BF16 : DType::F32;
  s->es = llk::dsize(s->dt);
  s->d_rows = s->dt == DType::BF16 ? (s->d + 255) / 256 * 256 : s->d;
  s->rope_half = c->rope_style == LLAMA_ROPE_HALF_SPLIT;
  return LLAMA_OK;
}

struct PackedLayout {
  size_t qkv, o, gu, down, gamma2, cos, sin, total;
};

PackedLayout packed_layout(const Shape& s) {
  PackedLayout p;
  size_t off = 0;
  p.qkv = off;
  off = align256(off + (size_t)s.NQKV_pad * s.d * s.es);
  p.o = off;
  off = align256(off + (size_t)s.d_rows * s.HD * s.es);
  p.gu = off;
  off = align256(off + (size_t)2 * s.I_pad * s.d * s.es);
  p.down = off;
  off = align256(off + (size_t)s.d_rows * s.I_pad * s.es);
  p.gamma2 = off;
  off = align256(off + (size_t)s.d * sizeof(float));
  p.cos = off;
  off = align256(off + (size_t)s.max_pos * (s.D / 2) * sizeof(float));
  p.sin = off;
  off = align256(off + (size_t)s.max_pos * (s.D / 2) * sizeof(float));
  p.total = off;
  return p;
}

int max_splits_for(const Shape& s) { return (s.max_pos + llk::decode_split_keys() - 1) / llk::decode_split_keys(); }

struct WsLayout {
  size_t desc, r1, r2, ss, xt, q, attn, h, hb, s, part, gpart, gpart_bytes, total;
};

bool use_skinny(const Shape& sh, long M) { return sh.dt == DType::BF16 && M <= 128; }

// RMSNorm_2 rides on the o_proj GEMM's split-K pass (no norm launch) when that
// GEMM streams its weights with K split over workgroups.
bool fold_norm2(const Shape& sh, long M) {
  return use_skinny(sh, M) && llk::skinny_ksplit((int)M, sh.d, sh.HD) > 1;
}
int norm_segments(const Shape& sh) { return (sh.d + llk::kNormSeg - 1) / llk::kNormSeg; }

// Split-K partial sums of the skinny GEMMs, for every token count up to T (the
// size is non-decreasing in T, so a workspace sized for T serves every call
// with fewer tokens).
size_t skinny_ws_bytes(const Shape& sh, size_t T) {
  if (sh.dt != DType::BF16) return 0;
  const int shapes[4][2] = {{sh.NQKV_pad, sh.d}, {sh.d, sh.HD}, {2 * sh.I_pad, sh.d}, {sh.d, sh.I_pad}};
  size_t best = 0;
  for (const int m : {64, 128}) {
    const int M = (int)std::min<size_t>(T, (size_t)m);
    for (const auto& nk : shapes) best = std::max(best, llk::skinny_partial_bytes(M, nk[0], nk[1]));
  }
  return best;
}

WsLayout ws_layout(const Shape& sh, size_t T, size_t B) {
  WsLayout w;
  size_t off = 0;
  w.desc = off;
  off = align256(off + B * 2 * sizeof(int32_t));
  w.r1 = off;
  off = align256(off + T * sizeof(float));
  w.r2 = off;
  off = align256(off + T * sizeof(float));
  w.ss = off;  // folded RMSNorm_2 partial sums (skinny calls only)
  off = align256(off + (sh.dt == DType::BF16 ? std::min<size_t>(T, 128) * norm_segments(sh) * sizeof(float) : 0));
  const size_t Tp = op_rows(sh, T);  // GEMM operands: whole 256-row tiles (bf16)
  w.xt = off;
  off = align256(off + (sh.dt == DType::BF16 ? Tp * sh.d * sh.es : 0));
  w.q = off;
  off = align256(off + T * sh.HD * sh.es);
  w.attn = off;
  off = align256(off + Tp * sh.HD * sh.es);
  w.h = off;
  off = align256(off + T * sh.d * sizeof(float));
  w.hb = off;
  off = align256(off + Tp * sh.d * sh.es);
  w.s = off;
  off = align256(off + Tp * sh.I_pad * sh.es);
  w.part = off;
  off = align256(off + B * sh.H * (size_t)max_splits_for(sh) * (sh.D + 2) * sizeof(float));
  w.gpart = off;
  w.gpart_bytes = skinny_ws_bytes(sh, T);
  off = align256(off + w.gpart_bytes);
  w.total = off;
  return w;
}

bool trace_on() {
  static int v = -1;
  if (v < 0) {
    const char* e = std::getenv("LLAMA_LAYER_TRACE");
    v = (e && *e && *e != '0') ? 1 : 0;
  }
  return v == 1;
}

// LLAMA_LAYER_POISON=1: fill each call's workspace with 0xFF bytes (NaN in
// fp32 and bf16) before any of its kernels run, so that a kernel reading
// workspace memory the same call has not written shows up as NaN or changed
// bits in the outputs (a device-side check for missing writes and races).
// Read at every call.
bool poison_on() {
  const char* e = std::getenv("LLAMA_LAYER_POISON");
  return e && *e && *e != '0';
}

#define HIP_TRY(expr)                                                                   \
  do {                                                                                  \
    hipError_t _e = (expr);                                                             \
    if (_e != hipSuccess) {                                                             \
      if (trace_on()) std::fprintf(stderr, "[llama_layer] %s -> %s\n", #expr, hipGetErrorString(_e)); \
      return LLAMA_ERR_HIP;                                                             \
    }                                                                                   \
  } while (0)

}  // namespace

// ---------------------------------------------------------------------------
// handles
// ---------------------------------------------------------------------------

namespace {
enum Kern {
  K_RMS1, K_QKV, K_ATTN_PREFILL, K_ATTN_DECODE, K_ATTN_COMBINE, K_OPROJ, K_RMS2, K_GATEUP, K_DOWN, K_FINAL_NORM,
  K_COUNT
};
const char* const kKernNames[K_COUNT] = {"rms_rowscale",   "gemm_qkv_rope",     "attn_prefill",
                                         "attn_decode_split", "attn_decode_combine", "gemm_o_resid",
                                         "rms_convert",    "gemm_gate_up_swiglu", "gemm_down_resid",
                                         "rms_final_norm"};
struct Pending {
  int kind;
  void* start;
  void* stop;
};
}  // namespace

struct llama_layer {
  llama_layer_config cfg;
  Shape s;
  PackedLayout pl;
  char* packed;
  // per-kernel timing
  bool profiling = false;
  std::vector<void*> free_events;
  std::vector<Pending> pending;
  int launches[K_COUNT] = {};
  double total_ms[K_COUNT] = {};
};

namespace {

void drop_events(llama_layer* L) {
  for (auto& p : L->pending) {
    (void)llk::event_destroy(p.start);
    (void)llk::event_destroy(p.stop);
  }
  L->pending.clear();
  for (void* e : L->free_events) (void)llk::event_destroy(e);
  L->free_events.clear();
}

hipError_t take_event(llama_layer* L, void** ev) {
  if (!L->free_events.empty()) {
    *ev = L->free_events.back();
    L->free_events.pop_back();
    return hipSuccess;
  }
  return llk::event_create(ev);
}

// Launch `fn` on stream s, bracketed by timing events when profiling.
template <typename F>
hipError_t timed(llama_layer* L, int kind, hipStream_t s, F&& fn) {
  if (!L->profiling) return fn();
  void *a = nullptr, *b = nullptr;
  hipError_t e = take_event(L, &a);
  if (e == hipSuccess) e = take_event(L, &b);
  if (e == hipSuccess) e = llk::event_record(a, s);
  if (e != hipSuccess) return e;
  e = fn();
  if (e != hipSuccess) return e;
  e = llk::event_record(b, s);
  if (e != hipSuccess) return e;
  L->pending.push_back({kind, a, b});
  return hipSuccess;
}

}  // namespace

struct SeqState {
  bool open = false;
  int len = 0;
  std::vector<int32_t> blocks;
};

struct llama_kv_cache {
  Shape s;
  int num_blocks, max_seqs, max_blocks;
  int n_layers;        // layers sharing the block tables; pools are [n_layers][num_blocks] blocks
  size_t layer_bytes;  // bytes of one layer's K (or V) pool
  void* k_pool;
  void* v_pool;
  int32_t* table;
  std::vector<int32_t> free_blocks;  // handed out from the back
  std::vector<SeqState> seqs;
};

namespace {

size_t pool_bytes(const Shape& s, int num_blocks) { return (size_t)num_blocks * s.G * kBlock * s.D * s.es; }

struct CacheLayout {
  size_t k, v, table, total;
};
CacheLayout cache_layout(const Shape& s, int num_blocks, int max_seqs, int n_layers) {
  CacheLayout c;
  const int max_blocks = (s.max_pos + kBlock - 1) / kBlock;
  size_t off = 0;
  c.k = off;
  off = align256(off + (size_t)n_layers * pool_bytes(s, num_blocks));
  c.v = off;
  off = align256(off + (size_t)n_layers * pool_bytes(s, num_blocks));
  c.table = off;
  off = align256(off + (size_t)max_seqs * max_blocks * sizeof(int32_t));
  c.total = off;
  return c;
}

// The cache as the kernels of layer `layer` see it: that layer's pools, the
// shared block tables.
llk::CacheView cache_view(const llama_kv_cache* c, int layer = 0) {
  llk::CacheView v;
  v.k_pool = reinterpret_cast<char*>(c->k_pool) + (size_t)layer * c->layer_bytes;
  v.v_pool = reinterpret_cast<char*>(c->v_pool) + (size_t)layer * c->layer_bytes;
  v.block_table = c->table;
  v.max_blocks = c->max_blocks;
  v.G = c->s.G;
  v.D = c->s.D;
  return v;
}

// Flush (index, value) pairs to device int32 memory through kernel arguments.
// Host-side int32 stores for the device (block tables, batch descriptors),
// batched into kernel arguments: a batch holds up to kUploadMax stores to at
// most two arrays.
struct Uploader {
  std::vector<llk::Upload> batches;
  void add(int32_t* base, int32_t idx, int32_t val) {
    int slot = -1;
    if (!batches.empty() && batches.back().n < llk::kUploadMax) {
      llk::Upload& u = batches.back();
      if (u.base[0] == base) slot = 0;
      else if (u.base[1] == base || u.base[1] == nullptr) slot = 1;
    }
    if (slot < 0) {
      batches.emplace_back();
      std::memset(&batches.back(), 0, sizeof(llk::Upload));
      slot = 0;
    }
    llk::Upload& u = batches.back();
    u.base[slot] = base;
    u.idx[u.n] = idx | (slot ? (int32_t)0x80000000u : 0);
    u.val[u.n] = val;
    ++u.n;
  }
  // launch every batch but the last, which is returned for the caller's first
  // kernel to apply (null if there is none)
  hipError_t flush_all_but_last(hipStream_t s, const llk::Upload** last) {
    *last = nullptr;
    for (size_t i = 0; i + 1 < batches.size(); ++i) {
      hipError_t e = llk::launch_upload(batches[i], s);
      if (e != hipSuccess) return e;
    }
    if (!batches.empty()) *last = &batches.back();
    return hipSuccess;
  }
  hipError_t flush(hipStream_t s) {
    for (auto& u : batches) {
      hipError_t e = llk::launch_upload(u, s);
      if (e != hipSuccess) return e;
    }
    batches.clear();
    return hipSuccess;
  }
};

bool same_shape(const Shape& a, const Shape& b) {
  return a.G == b.G && a.D == b.D && a.dt == b.dt && a.max_pos == b.max_pos;
}

// Validate a batch of sequences about to grow by n tokens each; on success
// append the block-table updates to `up` and commit the allocation.
llama_status reserve(llama_kv_cache* c, int batch, const int32_t* seq_ids, int n, Uploader* up) {
  std::unordered_set<int32_t> seen;
  long need = 0;
  for (int b = 0; b < batch; ++b) {
    const int32_t id = seq_ids[b];
    if (id < 0 || id >= c->max_seqs || !c->seqs[id].open) return LLAMA_ERR_BAD_SEQ;
    if (!seen.insert(id).second) return LLAMA_ERR_BAD_SEQ;
    const long new_len = (long)c->seqs[id].len + n;
    if (new_len > c->s.max_pos) return LLAMA_ERR_POSITION;
    need += (new_len + kBlock - 1) / kBlock - (long)c->seqs[id].blocks.size();
  }
  if (need > (long)c->free_blocks.size()) return LLAMA_ERR_CACHE_FULL;
  for (int b = 0; b < batch; ++b) {
    SeqState& st = c->seqs[seq_ids[b]];
    const int want = (st.len + n + kBlock - 1) / kBlock;
    while ((int)st.blocks.size() < want) {
      const int32_t blk = c->free_blocks.back();
      c->free_blocks.pop_back();
      up->add(c->table, seq_ids[b] * c->max_blocks + (int32_t)st.blocks.size(), blk);
      st.blocks.push_back(blk);
    }
  }
  return LLAMA_OK;
}

}  // namespace

extern "C" {

const char* llama_status_string(llama_status s) {
  switch (s) {
    case LLAMA_OK: return "ok";
    case LLAMA_ERR_INVALID_ARG: return "invalid argument";
    case LLAMA_ERR_SHAPE: return "invalid shape";
    case LLAMA_ERR_DTYPE: return "invalid dtype";
    case LLAMA_ERR_CACHE_FULL: return "KV cache full";
    case LLAMA_ERR_BAD_SEQ: return "bad sequence id";
    case LLAMA_ERR_POSITION: return "position beyond max_position";
    case LLAMA_ERR_HIP: return "HIP error";
    case LLAMA_ERR_UNSUPPORTED: return "unsupported configuration";
    case LLAMA_ERR_SCRATCH: return "workspace larger than the static scratch buffer";
  }
  return "unknown status";
}

llama_status llama_layer_packed_bytes(const llama_layer_config* cfg, size_t* bytes) {
  if (!bytes) return LLAMA_ERR_INVALID_ARG;
  Shape s;
  llama_status st = check_config(cfg, &s);
  if (st != LLAMA_OK) return st;
  *bytes = packed_layout(s).total;
  return LLAMA_OK;
}

llama_status llama_layer_create(const llama_layer_config* cfg, const llama_layer_weights* w, void* packed_dev,
                                void* stream, llama_layer** out) {
  if (!out || !w || !packed_dev) return LLAMA_ERR_INVALID_ARG;
  Shape s;
  llama_status st = check_config(cfg, &s);
  if (st != LLAMA_OK) return st;
  const void* ptrs[] = {w->q_proj, w->k_proj, w->v_proj, w->o_proj, w->gate_proj,
                        w->up_proj, w->down_proj, w->input_layernorm, w->post_attention_layernorm};
  for (const void* p : ptrs)
    if (!p || !aligned(p, 16)) return LLAMA_ERR_INVALID_ARG;
  if (!aligned(packed_dev, 256)) return LLAMA_ERR_INVALID_ARG;

  llama_layer* L = new (std::nothrow) llama_layer;
  if (!L) return LLAMA_ERR_INVALID_ARG;
  L->cfg = *cfg;
  L->s = s;
  L->pl = packed_layout(s);
  L->packed = reinterpret_cast<char*>(packed_dev);
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  auto fail = [&](hipError_t e) {
    if (trace_on()) std::fprintf(stderr, "[llama_layer] create: %s\n", hipGetErrorString(e));
    delete L;
    return LLAMA_ERR_HIP;
  };
  char* P = L->packed;
  hipError_t e = llk::launch_zero(P, L->pl.cos, hs);  // padding rows and columns stay zero
  // fused QKV weight with gamma_1 folded in: rows [q | k | v].  With half-split
  // RoPE the q and k rows of each head are reordered (0, D/2, 1, D/2+1, ...)
  // so that every rotated pair sits in adjacent rows, as in the interleaved
  // form; the QKV epilogue writes each result back to its own position.
  const int rp = s.rope_half ? s.D : 0;
  if (e == hipSuccess)
    e = llk::launch_pack(s.dt, w->q_proj, w->input_layernorm, P + L->pl.qkv, s.HD, s.d, s.d, s.NQKV_pad, 1, 0, rp, hs);
  if (e == hipSuccess)
    e = llk::launch_pack(s.dt, w->k_proj, w->input_layernorm, P + L->pl.qkv, s.KD, s.d, s.d, s.NQKV_pad, 1, s.HD, rp, hs);
  if (e == hipSuccess)
    e = llk::launch_pack(s.dt, w->v_proj, w->input_layernorm, P + L->pl.qkv, s.KD, s.d, s.d, s.NQKV_pad, 1, s.HD + s.KD, 0, hs);
  if (e == hipSuccess) e = llk::launch_pack(s.dt, w->o_proj, nullptr, P + L->pl.o, s.d, s.HD, s.HD, s.d_rows, 1, 0, 0, hs);
  // gate/up interleaved row by row; gamma_2 scales the activation instead
  // (h * gamma_2 is rounded once, the weights stay exact)
  if (e == hipSuccess) e = llk::launch_pack(s.dt, w->gate_proj, nullptr, P + L->pl.gu, s.I, s.d, s.d, 2 * s.I_pad, 2, 0, 0, hs);
  if (e == hipSuccess) e = llk::launch_pack(s.dt, w->up_proj, nullptr, P + L->pl.gu, s.I, s.d, s.d, 2 * s.I_pad, 2, 1, 0, hs);
  if (e == hipSuccess)
    e = llk::launch_to_f32(s.dt, w->post_attention_layernorm, reinterpret_cast<float*>(P + L->pl.gamma2), s.d, hs);
  if (e == hipSuccess)
    e = llk::launch_pack(s.dt, w->down_proj, nullptr, P + L->pl.down, s.d, s.I, s.I_pad, s.d_rows, 1, 0, 0, hs);
  if (e != hipSuccess) return fail(e);

  // RoPE table, angle pos * theta^(-2i/D) evaluated in double, stored fp32
  // ("Chapter 10", section 3; "From Transformer to LLaMA: an overview", 4.2)
  const int half = s.D / 2;
  std::vector<float> cs((size_t)s.max_pos * half), sn((size_t)s.max_pos * half);
  for (int i = 0; i < half; ++i) {
    const double inv = std::pow((double)cfg->rope_theta, -2.0 * i / s.D);
    for (int p = 0; p < s.max_pos; ++p) {
      const double a = (double)p * inv;
      cs[(size_t)p * half + i] = (float)std::cos(a);
      sn[(size_t)p * half + i] = (float)std::sin(a);
    }
  }
  e = llk::copy_to_device(P + L->pl.cos, cs.data(), cs.size() * sizeof(float), hs);
  if (e == hipSuccess) e = llk::copy_to_device(P + L->pl.sin, sn.data(), sn.size() * sizeof(float), hs);
  if (e == hipSuccess) e = llk::stream_sync(hs);
  if (e != hipSuccess) return fail(e);
  *out = L;
  return LLAMA_OK;
}

llama_status llama_layer_workspace_bytes(const llama_layer* layer, int32_t max_tokens, int32_t max_batch,
                                         size_t* bytes) {
  if (!layer || !bytes || max_tokens <= 0 || max_batch <= 0 || max_batch > max_tokens) return LLAMA_ERR_INVALID_ARG;
  *bytes = ws_layout(layer->s, (size_t)max_tokens, (size_t)max_batch).total;
  return LLAMA_OK;
}

llama_status llama_layer_destroy(llama_layer* layer) {
  if (!layer) return LLAMA_ERR_INVALID_ARG;
  drop_events(layer);
  delete layer;
  return LLAMA_OK;
}

llama_status llama_layer_profile_enable(llama_layer* layer, int32_t enable) {
  if (!layer) return LLAMA_ERR_INVALID_ARG;
  layer->profiling = enable != 0;
  if (!layer->profiling) {
    drop_events(layer);
    for (int k = 0; k < K_COUNT; ++k) {
      layer->launches[k] = 0;
      layer->total_ms[k] = 0.0;
    }
  }
  return LLAMA_OK;
}

llama_status llama_layer_profile_read(llama_layer* layer, llama_kernel_time* out, int32_t max, int32_t* n,
                                      int32_t reset) {
  if (!layer || !n || max < 0 || (max > 0 && !out)) return LLAMA_ERR_INVALID_ARG;
  for (auto& p : layer->pending) {
    float ms = 0.f;
    HIP_TRY(llk::event_elapsed_ms(&ms, p.start, p.stop));
    layer->launches[p.kind] += 1;
    layer->total_ms[p.kind] += ms;
    layer->free_events.push_back(p.start);
    layer->free_events.push_back(p.stop);
  }
  layer->pending.clear();
  int cnt = 0;
  for (int k = 0; k < K_COUNT; ++k) {
    if (layer->launches[k] == 0) continue;
    if (cnt < max) {
      std::memset(&out[cnt], 0, sizeof(llama_kernel_time));
      std::snprintf(out[cnt].name, sizeof(out[cnt].name), "%s", kKernNames[k]);
      out[cnt].launches = layer->launches[k];
      out[cnt].total_ms = layer->total_ms[k];
    }
    ++cnt;
  }
  *n = cnt < max ? cnt : max;
  if (reset) {
    for (int k = 0; k < K_COUNT; ++k) {
      layer->launches[k] = 0;
      layer->total_ms[k] = 0.0;
    }
  }
  return LLAMA_OK;
}

// ---- cache ----------------------------------------------------------------

llama_status llama_kv_cache_bytes_layers(const llama_layer_config* cfg, int32_t n_layers, int32_t num_blocks,
                                         int32_t block_size, int32_t max_seqs, size_t* bytes) {
  if (!bytes || n_layers <= 0 || num_blocks <= 0 || max_seqs <= 0) return LLAMA_ERR_INVALID_ARG;
  Shape s;
  llama_status st = check_config(cfg, &s);
  if (st != LLAMA_OK) return st;
  if (block_size != kBlock) return LLAMA_ERR_UNSUPPORTED;
  *bytes = cache_layout(s, num_blocks, max_seqs, n_layers).total;
  return LLAMA_OK;
}

llama_status llama_kv_cache_bytes(const llama_layer_config* cfg, int32_t num_blocks, int32_t block_size,
                                  int32_t max_seqs, size_t* bytes) {
  return llama_kv_cache_bytes_layers(cfg, 1, num_blocks, block_size, max_seqs, bytes);
}

llama_status llama_kv_cache_create_layers(const llama_layer_config* cfg, int32_t n_layers, int32_t num_blocks,
                                          int32_t block_size, int32_t max_seqs, const int32_t* block_order,
                                          void* pool_dev, llama_kv_cache** out) {
  if (!out || !pool_dev || n_layers <= 0 || num_blocks <= 0 || max_seqs <= 0) return LLAMA_ERR_INVALID_ARG;
  if (!aligned(pool_dev, 256)) return LLAMA_ERR_INVALID_ARG;
  Shape s;
  llama_status st = check_config(cfg, &s);
  if (st != LLAMA_OK) return st;
  if (block_size != kBlock) return LLAMA_ERR_UNSUPPORTED;
  std::vector<int32_t> order(num_blocks);
  if (block_order) {
    std::vector<char> hit(num_blocks, 0);
    for (int i = 0; i < num_blocks; ++i) {
      const int32_t b = block_order[i];
      if (b < 0 || b >= num_blocks || hit[b]) return LLAMA_ERR_INVALID_ARG;
      hit[b] = 1;
      order[i] = b;
    }
  } else {
    for (int i = 0; i < num_blocks; ++i) order[i] = i;
  }
  llama_kv_cache* c = new (std::nothrow) llama_kv_cache;
  if (!c) return LLAMA_ERR_INVALID_ARG;
  const CacheLayout cl = cache_layout(s, num_blocks, max_seqs, n_layers);
  c->s = s;
  c->num_blocks = num_blocks;
  c->max_seqs = max_seqs;
  c->max_blocks = (s.max_pos + kBlock - 1) / kBlock;
  c->n_layers = n_layers;
  c->layer_bytes = pool_bytes(s, num_blocks);
  c->k_pool = reinterpret_cast<char*>(pool_dev) + cl.k;
  c->v_pool = reinterpret_cast<char*>(pool_dev) + cl.v;
  c->table = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(pool_dev) + cl.table);
  c->free_blocks.assign(order.rbegin(), order.rend());
  c->seqs.resize(max_seqs);
  *out = c;
  return LLAMA_OK;
}

llama_status llama_kv_cache_create(const llama_layer_config* cfg, int32_t num_blocks, int32_t block_size,
                                   int32_t max_seqs, const int32_t* block_order, void* pool_dev,
                                   llama_kv_cache** out) {
  return llama_kv_cache_create_layers(cfg, 1, num_blocks, block_size, max_seqs, block_order, pool_dev, out);
}

llama_status llama_kv_cache_num_layers(const llama_kv_cache* c, int32_t* n) {
  if (!c || !n) return LLAMA_ERR_INVALID_ARG;
  *n = c->n_layers;
  return LLAMA_OK;
}

llama_status llama_kv_cache_destroy(llama_kv_cache* cache) {
  if (!cache) return LLAMA_ERR_INVALID_ARG;
  delete cache;
  return LLAMA_OK;
}

llama_status llama_kv_cache_add_seq(llama_kv_cache* c, int32_t* seq_id_out) {
  if (!c || !seq_id_out) return LLAMA_ERR_INVALID_ARG;
  for (int i = 0; i < c->max_seqs; ++i) {
    if (!c->seqs[i].open) {
      c->seqs[i].open = true;
      c->seqs[i].len = 0;
      c->seqs[i].blocks.clear();
      *seq_id_out = i;
      return LLAMA_OK;
    }
  }
  return LLAMA_ERR_CACHE_FULL;
}

llama_status llama_kv_cache_free_seq(llama_kv_cache* c, int32_t seq_id) {
  if (!c) return LLAMA_ERR_INVALID_ARG;
  if (seq_id < 0 || seq_id >= c->max_seqs || !c->seqs[seq_id].open) return LLAMA_ERR_BAD_SEQ;
  SeqState& st = c->seqs[seq_id];
  for (auto it = st.blocks.rbegin(); it != st.blocks.rend(); ++it) c->free_blocks.push_back(*it);
  st = SeqState();
  return LLAMA_OK;
}

llama_status llama_kv_cache_seq_len(const llama_kv_cache* c, int32_t seq_id, int32_t* len) {
  if (!c || !len) return LLAMA_ERR_INVALID_ARG;
  if (seq_id < 0 || seq_id >= c->max_seqs || !c->seqs[seq_id].open) return LLAMA_ERR_BAD_SEQ;
  *len = c->seqs[seq_id].len;
  return LLAMA_OK;
}

llama_status llama_kv_cache_free_blocks(const llama_kv_cache* c, int32_t* n) {
  if (!c || !n) return LLAMA_ERR_INVALID_ARG;
  *n = (int32_t)c->free_blocks.size();
  return LLAMA_OK;
}

llama_status llama_kv_cache_write(llama_kv_cache* c, int32_t seq_id, int32_t n_tokens, const void* k_dev,
                                  const void* v_dev, void* stream) {
  if (!c || !k_dev || !v_dev || n_tokens <= 0) return LLAMA_ERR_INVALID_ARG;
  Uploader up;
  const bool known = seq_id >= 0 && seq_id < c->max_seqs;
  const int start = known ? c->seqs[seq_id].len : 0;
  const size_t nblk = known ? c->seqs[seq_id].blocks.size() : 0;
  llama_status st = reserve(c, 1, &seq_id, n_tokens, &up);
  if (st != LLAMA_OK) return st;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = up.flush(hs);
  const size_t per_layer = (size_t)n_tokens * c->s.KD * c->s.es;  // bytes of one layer's [n, G, D]
  for (int l = 0; l < c->n_layers && e == hipSuccess; ++l)
    e = llk::launch_kv_copy(c->s.dt, cache_view(c, l), seq_id, start, n_tokens,
                            const_cast<char*>(reinterpret_cast<const char*>(k_dev)) + l * per_layer,
                            const_cast<char*>(reinterpret_cast<const char*>(v_dev)) + l * per_layer, true, hs);
  SeqState& sq = c->seqs[seq_id];
  if (e != hipSuccess) {  // give the reserved blocks back, newest first: the cache is as before the call
    while (sq.blocks.size() > nblk) {
      c->free_blocks.push_back(sq.blocks.back());
      sq.blocks.pop_back();
    }
    if (trace_on()) std::fprintf(stderr, "[llama_layer] kv_cache_write: %s\n", hipGetErrorString(e));
    return LLAMA_ERR_HIP;
  }
  sq.len += n_tokens;
  return LLAMA_OK;
}

llama_status llama_kv_cache_read(const llama_kv_cache* c, int32_t seq_id, int32_t start, int32_t n, void* k_dev,
                                 void* v_dev, void* stream) {
  if (!c || !k_dev || !v_dev || n <= 0 || start < 0) return LLAMA_ERR_INVALID_ARG;
  if (seq_id < 0 || seq_id >= c->max_seqs || !c->seqs[seq_id].open) return LLAMA_ERR_BAD_SEQ;
  if ((long)start + n > c->seqs[seq_id].len) return LLAMA_ERR_POSITION;
  const size_t per_layer = (size_t)n * c->s.KD * c->s.es;
  for (int l = 0; l < c->n_layers; ++l)
    HIP_TRY(llk::launch_kv_copy(c->s.dt, cache_view(c, l), seq_id, start, n,
                                reinterpret_cast<char*>(k_dev) + l * per_layer,
                                reinterpret_cast<char*>(v_dev) + l * per_layer, false,
                                reinterpret_cast<hipStream_t>(stream)));
  return LLAMA_OK;
}

// ---- forward ----------------------------------------------------------------

}  // extern "C"

namespace {

// Argument checks common to a layer call and a stack call (the workspace size
// is checked by the caller, once the call's layout is known).
llama_status check_call(const Shape& s, const llama_kv_cache* c, int32_t batch, int32_t seq_len,
                        const int32_t* seq_ids, const void* x, const void* out, int32_t out_dtype,
                        const void* workspace) {
  if (!c || !seq_ids || !x || !out || !workspace) return LLAMA_ERR_INVALID_ARG;
  if (batch <= 0 || seq_len <= 0) return LLAMA_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(out, 16) || !aligned(workspace, 256)) return LLAMA_ERR_INVALID_ARG;
  if (out_dtype != LLAMA_DTYPE_F32 && out_dtype != LLAMA_DTYPE_BF16) return LLAMA_ERR_DTYPE;
  if (s.dt == DType::F32 && out_dtype != LLAMA_DTYPE_F32) return LLAMA_ERR_DTYPE;
  if (!same_shape(s, c->s)) return LLAMA_ERR_SHAPE;
  if ((long)batch * seq_len > (1L << 24)) return LLAMA_ERR_SHAPE;
  return LLAMA_OK;
}

// Host bookkeeping of one forward call, shared by every layer it runs.
// begin() reserves the sequences' new blocks and queues the block-table and
// batch-descriptor stores (all but the last batch of them launched here; the
// last rides on the first kernel).  commit() advances the sequence lengths
// once every kernel of the call has been enqueued; abort() instead returns
// the blocks reserved by begin() to the pool, in the order they were taken,
// so a failed call leaves the cache as it found it.
struct CallBook {
  llama_kv_cache* c = nullptr;
  int batch = 0, seq_len = 0;
  const int32_t* seq_ids = nullptr;
  std::vector<int> nblocks;  // blocks of each sequence before the call
  bool reserved = false;

  llama_status begin(llama_kv_cache* cache, int32_t b_, int32_t s_, const int32_t* ids, int32_t* desc, hipStream_t hs,
                     const llk::Upload** last_upload, Uploader* up, int* attn_units) {
    c = cache;
    batch = b_;
    seq_len = s_;
    seq_ids = ids;
    std::vector<int32_t> start(batch);
    nblocks.assign(batch, 0);
    for (int b = 0; b < batch; ++b) {
      const bool known = seq_ids[b] >= 0 && seq_ids[b] < c->max_seqs;
      start[b] = known ? c->seqs[seq_ids[b]].len : 0;
      nblocks[b] = known ? (int)c->seqs[seq_ids[b]].blocks.size() : 0;
    }
    llama_status st = reserve(c, batch, seq_ids, seq_len, up);
    if (st != LLAMA_OK) return st;  // reserve changes nothing when it fails
    reserved = true;
    // (sequence, key chunk) work units of the decode attention after this call
    const int ck = llk::decode_split_keys();
    *attn_units = 0;
    for (int b = 0; b < batch; ++b) *attn_units += (start[b] + seq_len + ck - 1) / ck;
    for (int b = 0; b < batch; ++b) {
      up->add(desc, 2 * b, seq_ids[b]);
      up->add(desc, 2 * b + 1, start[b]);
    }
    HIP_TRY(up->flush_all_but_last(hs, last_upload));
    return LLAMA_OK;
  }
  void commit() {
    for (int b = 0; b < batch; ++b) c->seqs[seq_ids[b]].len += seq_len;
    reserved = false;
  }
  void abort() {
    if (!reserved) return;
    // reserve() took blocks from the back of the free list, sequence by
    // sequence; putting them back in reverse restores the list exactly
    for (int b = batch - 1; b >= 0; --b) {
      SeqState& st = c->seqs[seq_ids[b]];
      while ((int)st.blocks.size() > nblocks[b]) {
        c->free_blocks.push_back(st.blocks.back());
        st.blocks.pop_back();
      }
    }
    reserved = false;
  }
};

// The kernels of one layer over the tokens of a call (begin_call done):
// x [M][d] in the layer dtype -> out [M][d] in out_t; K/V of the new tokens
// go to the pools of `cv`.
llama_status run_layer(llama_layer* L, const llk::CacheView& cv, const llk::BatchView& bv, int M, const void* x,
                       void* out, DType out_t, char* W, const WsLayout& wl, const llk::Upload* last_upload,
                       hipStream_t hs, bool decode, int attn_units) {
  const Shape& s = L->s;
  float* r1 = reinterpret_cast<float*>(W + wl.r1);
  float* r2 = reinterpret_cast<float*>(W + wl.r2);
  void* xt = s.dt == DType::BF16 ? W + wl.xt : nullptr;  // tiled copy of x (QKV operand)
  void* qb = W + wl.q;
  void* attn = W + wl.attn;
  float* h = reinterpret_cast<float*>(W + wl.h);
  void* hb = W + wl.hb;
  void* sb = W + wl.s;
  float* part = reinterpret_cast<float*>(W + wl.part);
  const char* P = L->packed;
  const float eps = L->cfg.rms_norm_eps;
  float* gpart = reinterpret_cast<float*>(W + wl.gpart);
  auto tile_for = [&](int N) {
    if (use_skinny(s, M)) return llk::GemmTile::SKINNY;
    return (M >= 256 && N % llk::gemm_tile_n(llk::GemmTile::LARGE) == 0) ? llk::GemmTile::LARGE
                                                                          : llk::GemmTile::SMALL;
  };
  if (trace_on())
    std::fprintf(stderr, "[llama_layer] %s B=%d S=%d T=%d d=%d H=%d G=%d D=%d I=%d\n", decode ? "decode" : "prefill",
                 bv.batch, bv.seq_len, M, s.d, s.H, s.G, s.D, s.I);

  // RMSNorm_1 statistics
  HIP_TRY(timed(L, K_RMS1, hs,
                [&] { return llk::launch_rms_rowscale(s.dt, x, r1, xt, M, s.d, eps, last_upload, hs); }));

  // QKV + RoPE + cache append
  llk::GemmArgs a{};
  a.split_ws = gpart;
  a.split_ws_bytes = wl.gpart_bytes;
  a.W = P + L->pl.qkv;
  a.X = xt ? xt : x;
  a.M = M;
  a.N = s.NQKV_pad;
  a.w_rows = s.NQKV_pad;
  a.K = s.d;
  a.ldx = s.d;
  a.epi = llk::Epi::QKV;
  a.rowscale = r1;
  a.q_out = qb;
  a.cache = cv;
  a.batch = bv;
  a.rope_cos = reinterpret_cast<const float*>(P + L->pl.cos);
  a.rope_sin = reinterpret_cast<const float*>(P + L->pl.sin);
  a.rope_half = s.rope_half ? 1 : 0;
  a.H = s.H;
  HIP_TRY(timed(L, K_QKV, hs, [&] { return llk::launch_gemm(s.dt, tile_for(a.N), a, hs); }));

  // attention
  if (decode) {
    const int ms = max_splits_for(s);
    HIP_TRY(timed(L, K_ATTN_DECODE, hs, [&] { return llk::launch_attn_decode(s.dt, qb, part, ms, s.H, cv, bv, attn_units, hs); }));
    HIP_TRY(timed(L, K_ATTN_COMBINE, hs,
                  [&] { return llk::launch_attn_decode_combine(s.dt, part, attn, ms, s.H, s.D, bv, hs); }));
  } else {
    HIP_TRY(timed(L, K_ATTN_PREFILL, hs, [&] { return llk::launch_attn_prefill(s.dt, qb, attn, s.H, cv, bv, hs); }));
  }

  // o_proj + residual -> h (fp32)
  llk::GemmArgs o{};
  o.split_ws = gpart;
  o.split_ws_bytes = wl.gpart_bytes;
  o.W = P + L->pl.o;
  o.X = attn;
  o.M = M;
  o.N = s.d;
  o.w_rows = s.d_rows;
  o.K = s.HD;
  o.ldx = s.HD;
  o.epi = llk::Epi::RESID_H;
  o.resid = x;
  o.out = h;
  o.ldo = s.d;
  const float* gamma2 = reinterpret_cast<const float*>(P + L->pl.gamma2);
  const bool fold2 = fold_norm2(s, M);
  float* ss = reinterpret_cast<float*>(W + wl.ss);
  if (fold2) {  // RMSNorm_2 statistics + operand copy in the split-K pass
    o.norm_gamma = gamma2;
    o.norm_out = hb;
    o.ss_part = ss;
    o.ss_nseg = norm_segments(s);
  }
  HIP_TRY(timed(L, K_OPROJ, hs, [&] { return llk::launch_gemm(s.dt, tile_for(o.N), o, hs); }));

  // RMSNorm_2 statistics + operand copy
  if (!fold2)
    HIP_TRY(timed(L, K_RMS2, hs, [&] { return llk::launch_rms_convert(s.dt, h, gamma2, hb, r2, M, s.d, eps, hs); }));

  // gate/up + SiLU * up
  llk::GemmArgs g{};
  g.split_ws = gpart;
  g.split_ws_bytes = wl.gpart_bytes;
  g.W = P + L->pl.gu;
  g.X = hb;
  g.M = M;
  g.N = 2 * s.I_pad;
  g.w_rows = 2 * s.I_pad;
  g.K = s.d;
  g.ldx = s.d;
  g.epi = llk::Epi::SWIGLU;
  g.rowscale = r2;
  if (fold2) {
    g.ss_part = ss;
    g.ss_nseg = norm_segments(s);
    g.ss_d = s.d;
    g.eps = eps;
  }
  g.out = sb;
  g.ldo = s.I_pad;
  HIP_TRY(timed(L, K_GATEUP, hs, [&] { return llk::launch_gemm(s.dt, tile_for(g.N), g, hs); }));

  // down + residual -> out
  llk::GemmArgs dn{};
  dn.split_ws = gpart;
  dn.split_ws_bytes = wl.gpart_bytes;
  dn.W = P + L->pl.down;
  dn.X = sb;
  dn.M = M;
  dn.N = s.d;
  dn.w_rows = s.d_rows;
  dn.K = s.I_pad;
  dn.ldx = s.I_pad;
  dn.epi = llk::Epi::RESID_OUT;
  dn.resid = h;
  dn.out = out;
  dn.ldo = s.d;
  dn.out_dtype = out_t;
  HIP_TRY(timed(L, K_DOWN, hs, [&] { return llk::launch_gemm(s.dt, tile_for(dn.N), dn, hs); }));
  return LLAMA_OK;
}

llama_status forward(llama_layer* L, llama_kv_cache* c, int32_t batch, int32_t seq_len, const int32_t* seq_ids,
                     const void* x, void* out, int32_t out_dtype, void* workspace, size_t ws_bytes, void* stream,
                     bool decode) {
  if (!L) return LLAMA_ERR_INVALID_ARG;
  llama_status st = check_call(L->s, c, batch, seq_len, seq_ids, x, out, out_dtype, workspace);
  if (st != LLAMA_OK) return st;
  if (c->n_layers != 1) return LLAMA_ERR_SHAPE;  // a multi-layer cache belongs to a stack
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  const int M = batch * seq_len;
  const WsLayout wl = ws_layout(L->s, (size_t)M, (size_t)batch);
  if (ws_bytes < wl.total) return LLAMA_ERR_INVALID_ARG;
  char* W = reinterpret_cast<char*>(workspace);
  int32_t* desc = reinterpret_cast<int32_t*>(W + wl.desc);
  if (poison_on()) HIP_TRY(llk::launch_fill(W, wl.total, 0xFF, hs));  // before the uploads into it
  Uploader up;
  const llk::Upload* last_upload = nullptr;
  int units = 0;
  CallBook book;
  st = book.begin(c, batch, seq_len, seq_ids, desc, hs, &last_upload, &up, &units);
  if (st == LLAMA_OK) {
    const llk::BatchView bv{desc, batch, seq_len};
    st = run_layer(L, cache_view(c), bv, M, x, out, out_dtype == LLAMA_DTYPE_F32 ? DType::F32 : DType::BF16, W, wl,
                   last_upload, hs, decode, units);
  }
  if (st == LLAMA_OK) book.commit();
  else book.abort();
  return st;
}

}  // namespace

extern "C" {

// ---- stack ------------------------------------------------------------------

}  // extern "C"

struct llama_stack {
  std::vector<llama_layer*> layers;
  const void* final_norm;  // [d] in the layer dtype, caller-owned
};

namespace {

bool same_config(const llama_layer_config& a, const llama_layer_config& b) {
  return a.hidden_size == b.hidden_size && a.intermediate_size == b.intermediate_size &&
         a.num_attention_heads == b.num_attention_heads && a.num_key_value_heads == b.num_key_value_heads &&
         a.rms_norm_eps == b.rms_norm_eps && a.rope_theta == b.rope_theta && a.max_position == b.max_position &&
         a.dtype == b.dtype && a.rope_style == b.rope_style;
}

// Workspace of a stack call: one layer's workspace (reused by every layer in
// turn), then two [T][d] hidden-state buffers in the layer dtype that the
// layers write in alternation.
struct StackWs {
  WsLayout layer;
  size_t act[2], total;
};
StackWs stack_ws(const Shape& s, size_t T, size_t B) {
  StackWs w;
  w.layer = ws_layout(s, T, B);
  size_t off = w.layer.total;
  for (int i = 0; i < 2; ++i) {
    w.act[i] = off;
    off = align256(off + T * s.d * s.es);
  }
  w.total = off;
  return w;
}

llama_status stack_forward(llama_stack* S, llama_kv_cache* c, int32_t batch, int32_t seq_len,
                           const int32_t* seq_ids, const void* x, void* out, int32_t out_dtype, void* workspace,
                           size_t ws_bytes, void* stream, bool decode) {
  if (!S) return LLAMA_ERR_INVALID_ARG;
  llama_layer* L0 = S->layers[0];
  llama_status st = check_call(L0->s, c, batch, seq_len, seq_ids, x, out, out_dtype, workspace);
  if (st != LLAMA_OK) return st;
  const int nl = (int)S->layers.size();
  if (c->n_layers != nl) return LLAMA_ERR_SHAPE;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  const int M = batch * seq_len;
  const StackWs sw = stack_ws(L0->s, (size_t)M, (size_t)batch);
  if (ws_bytes < sw.total) return LLAMA_ERR_INVALID_ARG;
  char* W = reinterpret_cast<char*>(workspace);
  int32_t* desc = reinterpret_cast<int32_t*>(W + sw.layer.desc);
  if (poison_on()) HIP_TRY(llk::launch_fill(W, sw.total, 0xFF, hs));  // before the uploads into it
  Uploader up;
  const llk::Upload* last_upload = nullptr;
  int units = 0;
  CallBook book;
  st = book.begin(c, batch, seq_len, seq_ids, desc, hs, &last_upload, &up, &units);
  const llk::BatchView bv{desc, batch, seq_len};
  // x_{l+1} = layer_l(x_l), held in the layer dtype between layers
  const void* cur = x;
  for (int l = 0; l < nl && st == LLAMA_OK; ++l) {
    void* nxt = W + sw.act[l & 1];
    st = run_layer(S->layers[l], cache_view(c, l), bv, M, cur, nxt, L0->s.dt, W, sw.layer,
                   l == 0 ? last_upload : nullptr, hs, decode, units);
    cur = nxt;
  }
  // y = RMSNorm_final(x_L), timed with the last layer's kernels
  if (st == LLAMA_OK) {
    llama_layer* Ll = S->layers[nl - 1];
    const DType out_t = out_dtype == LLAMA_DTYPE_F32 ? DType::F32 : DType::BF16;
    const hipError_t e = timed(Ll, K_FINAL_NORM, hs, [&] {
      return llk::launch_rms_norm_out(L0->s.dt, cur, S->final_norm, out, out_t, M, L0->s.d, L0->cfg.rms_norm_eps, hs);
    });
    if (e != hipSuccess) st = LLAMA_ERR_HIP;
  }
  if (st == LLAMA_OK) book.commit();
  else book.abort();
  return st;
}

}  // namespace

extern "C" {

llama_status llama_stack_create(llama_layer* const* layers, int32_t n_layers, const void* final_norm,
                                llama_stack** out) {
  if (!layers || n_layers <= 0 || !final_norm || !out) return LLAMA_ERR_INVALID_ARG;
  if (!aligned(final_norm, 16)) return LLAMA_ERR_INVALID_ARG;
  for (int l = 0; l < n_layers; ++l) {
    if (!layers[l]) return LLAMA_ERR_INVALID_ARG;
    if (!same_config(layers[l]->cfg, layers[0]->cfg)) return LLAMA_ERR_SHAPE;
  }
  llama_stack* S = new (std::nothrow) llama_stack;
  if (!S) return LLAMA_ERR_INVALID_ARG;
  S->layers.assign(layers, layers + n_layers);
  S->final_norm = final_norm;
  *out = S;
  return LLAMA_OK;
}

llama_status llama_stack_workspace_bytes(const llama_stack* S, int32_t max_tokens, int32_t max_batch,
                                         size_t* bytes) {
  if (!S || !bytes || max_tokens <= 0 || max_batch <= 0 || max_batch > max_tokens) return LLAMA_ERR_INVALID_ARG;
  *bytes = stack_ws(S->layers[0]->s, (size_t)max_tokens, (size_t)max_batch).total;
  return LLAMA_OK;
}

llama_status llama_stack_destroy(llama_stack* S) {
  if (!S) return LLAMA_ERR_INVALID_ARG;
  delete S;
  return LLAMA_OK;
}

llama_status llama_stack_prefill(llama_stack* stack, llama_kv_cache* cache, int32_t batch, int32_t seq_len,
                                 const int32_t* seq_ids, const void* x, void* out, int32_t out_dtype,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  return stack_forward(stack, cache, batch, seq_len, seq_ids, x, out, out_dtype, workspace, workspace_bytes, stream,
                       false);
}

llama_status llama_stack_decode(llama_stack* stack, llama_kv_cache* cache, int32_t batch, const int32_t* seq_ids,
                                const void* x, void* out, int32_t out_dtype, void* workspace, size_t workspace_bytes,
                                void* stream) {
  return stack_forward(stack, cache, batch, 1, seq_ids, x, out, out_dtype, workspace, workspace_bytes, stream, true);
}

llama_status llama_layer_prefill(llama_layer* layer, llama_kv_cache* cache, int32_t batch, int32_t seq_len,
                                 const int32_t* seq_ids, const void* x, void* out, int32_t out_dtype,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  return forward(layer, cache, batch, seq_len, seq_ids, x, out, out_dtype, workspace, workspace_bytes, stream, false);
}

llama_status llama_layer_decode(llama_layer* layer, llama_kv_cache* cache, int32_t batch, const int32_t* seq_ids,
                                const void* x, void* out, int32_t out_dtype, void* workspace, size_t workspace_bytes,
                                void* stream) {
  return forward(layer, cache, batch, 1, seq_ids, x, out, out_dtype, workspace, workspace_bytes, stream, true);
}

llama_status llama_layer_decode_noalloc(llama_layer* layer, llama_kv_cache* cache, int32_t batch,
                                        const int32_t* seq_ids, const void* x, void* out, int32_t out_dtype,
                                        void* stream) {
  if (!layer) return LLAMA_ERR_INVALID_ARG;
  // host validation first (a stand-in workspace address: only its presence
  // and alignment are checked here)
  llama_status st = check_call(layer->s, cache, batch, 1, seq_ids, x, out, out_dtype, reinterpret_cast<void*>(256));
  if (st != LLAMA_OK) return st;
  if (ws_layout(layer->s, (size_t)batch, (size_t)batch).total > LLAMA_SCRATCH_BYTES) return LLAMA_ERR_SCRATCH;
  void* scratch = nullptr;
  size_t scratch_bytes = 0;
  HIP_TRY(llk::scratch_region(&scratch, &scratch_bytes));
  // no timing events for this call: creating them may allocate
  const bool prof = layer->profiling;
  layer->profiling = false;
  st = forward(layer, cache, batch, 1, seq_ids, x, out, out_dtype, scratch, scratch_bytes, stream, true);
  layer->profiling = prof;
  return st;
}

}  // extern "C"
