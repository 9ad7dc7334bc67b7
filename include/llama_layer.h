/*
 * llama_layer.h - C ABI of an MI355X (gfx950) implementation of the forward
 * pass of one LLaMA-style pre-norm decoder layer, with a paged KV cache for
 * incremental decode.
 *
 * The layer (pages cited by title and section):
 *   h   = x + o_proj( causal_GQA_attention( RoPE(q), RoPE(k), v ) ),
 *         [q | k | v] = RMSNorm_1(x) W_{q,k,v}^T
 *   out = h + down( SiLU( gate(RMSNorm_2(h)) ) * up(RMSNorm_2(h)) )
 *   - "LLaMA3 Block: from parts to engine", 3.1 (the two residual sub-blocks)
 *     and 4.2 (save residual -> norm -> sub-layer -> add back, two separate
 *     RMSNorm gammas named input_layernorm / post_attention_layernorm);
 *   - "Chapter 10: the modern LLaMA architecture", section 9 (block
 *     pseudocode with position_ids and past_kv), section 1 (the config.json
 *     fields used below);
 *   - RMSNorm(x) = x * rsqrt(mean(x^2) + eps) * gamma, in fp32
 *     ("Chapter 10", section 4; "3.2 Core components, one by one", 3.2.1);
 *   - RoPE on q and k only, pair i rotated by pos * theta^(-2i/D) ("Chapter
 *     10", sections 2-3; "From Transformer to LLaMA: an overview", 4.2), the
 *     pairs being interleaved (x[2i], x[2i+1]) ("Chapter 10", section 3) or,
 *     as an option, the two halves of the head (x[i], x[i + D/2]) ("From
 *     Transformer to the LLaMA series", section 8, apply_rope);
 *   - grouped-query attention: query head h reads KV head h / (H/G); the
 *     cache stores only the G KV heads ("Chapter 10", section 6);
 *   - softmax(q k^T / sqrt(D)) v with a causal mask, diagonal included
 *     ("From Transformer to LLaMA: an overview", 1.1);
 *   - SwiGLU with SiLU on the gate branch ("3.2 Core components", 3.2.2;
 *     "LLaMA3 Block", 4.1 and the gate/up pitfall of section 6);
 *   - KV cache: prefill writes the K/V of all prompt tokens; decode computes
 *     one new token at position = current length, appends its K/V, and
 *     attends to the whole cache plus itself ("Chapter 10", section 7).
 *
 * Memory and ownership
 *   All device memory is owned by the caller: the source weights (free once
 *   llama_layer_create has returned), the packed-weight buffer, the KV pool,
 *   the workspace, and every activation.  The library owns only host-side
 *   handles and the host copy of the block tables.  Device pointers must be
 *   256-byte aligned; pointers to activations and weights must be 16-byte
 *   aligned.
 *
 * Layouts (row-major, no padding between rows)
 *   weights: nn.Linear layout [out_features, in_features] in cfg.dtype;
 *     q_proj [H*D, d], k_proj/v_proj [G*D, d], o_proj [d, H*D],
 *     gate_proj/up_proj [I, d], down_proj [d, I]; gammas [d] in cfg.dtype.
 *   activations: x and out are [B, S, d] (prefill) or [B, d] (decode).
 *   cache read/write buffers: [n, G, D] in cfg.dtype, K already rotated.
 *
 * Errors
 *   Every call returns llama_status; nothing else crosses the ABI.  Argument
 *   and shape validation happens on the host before any HIP call, and a call
 *   that fails validation leaves every handle unchanged.  Device work is
 *   enqueued on the caller's HIP stream (a hipStream_t passed as void*; NULL
 *   is the default stream); results are ready when that stream is
 *   synchronised.  A failed HIP launch returns LLAMA_ERR_HIP.
 *
 * Threads: handles are not thread-safe.  Host bookkeeping (sequence lengths,
 * block tables) changes at call time, so keep all calls on one handle in one
 * stream order.
 */
#ifndef LLAMA_LAYER_H
#define LLAMA_LAYER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LLAMA_OK = 0,
  LLAMA_ERR_INVALID_ARG = -1, /* null pointer, non-positive size, bad eps/theta, misaligned */
  LLAMA_ERR_SHAPE = -2,       /* H % G != 0, d != H*D, odd or unsupported D, sizes too large */
  LLAMA_ERR_DTYPE = -3,       /* unknown dtype, or bf16 output from an fp32 layer */
  LLAMA_ERR_CACHE_FULL = -4,  /* the batch needs more free blocks / sequence slots than remain */
  LLAMA_ERR_BAD_SEQ = -5,     /* unknown or duplicated seq_id */
  LLAMA_ERR_POSITION = -6,    /* a position would reach max_position */
  LLAMA_ERR_HIP = -7,         /* a HIP call or kernel launch failed */
  LLAMA_ERR_UNSUPPORTED = -8, /* valid but not supported by this build */
  LLAMA_ERR_SCRATCH = -9      /* the call needs more than the static scratch buffer holds */
} llama_status;

typedef enum { LLAMA_DTYPE_F32 = 0, LLAMA_DTYPE_BF16 = 1 } llama_dtype;

/* Which elements of a head RoPE rotates together (same angle pos * theta^(-2i/D)
 * for pair i in both). */
typedef enum {
  LLAMA_ROPE_INTERLEAVED = 0, /* (x[2i], x[2i+1]): "Chapter 10", section 3 */
  LLAMA_ROPE_HALF_SPLIT = 1   /* (x[i], x[i + D/2]): "From Transformer to the LLaMA series", section 8 */
} llama_rope_style;

/* The config.json fields of the layer ("Chapter 10", section 1) plus the
 * storage dtype and the RoPE table length.  Accumulation is always fp32.
 * Supported: head_dim D = hidden_size / num_attention_heads in {64, 128}
 * (fp32 layers: 64),
 * num_attention_heads / num_key_value_heads in {1, 2, 4, 8, 16, 32},
 * hidden_size a multiple of 64, intermediate_size a multiple of 8. */
typedef struct {
  int32_t hidden_size;
  int32_t intermediate_size;
  int32_t num_attention_heads;
  int32_t num_key_value_heads;
  float rms_norm_eps;
  float rope_theta;
  int32_t max_position; /* positions >= max_position are rejected (LLAMA_ERR_POSITION) */
  int32_t dtype;        /* a llama_dtype: weights, activations and cache */
  int32_t rope_style;   /* a llama_rope_style (other values: LLAMA_ERR_INVALID_ARG) */
} llama_layer_config;

/* Device pointers to the nine parameter tensors, nn.Linear layout. */
typedef struct {
  const void *q_proj, *k_proj, *v_proj, *o_proj;
  const void *gate_proj, *up_proj, *down_proj;
  const void *input_layernorm, *post_attention_layernorm;
} llama_layer_weights;

typedef struct llama_layer llama_layer;         /* opaque */
typedef struct llama_kv_cache llama_kv_cache;   /* opaque */
typedef struct llama_stack llama_stack;         /* opaque */

const char* llama_status_string(llama_status s);

/* ---- layer ------------------------------------------------------------- */

/* Bytes of the packed-weight buffer llama_layer_create needs for cfg. */
llama_status llama_layer_packed_bytes(const llama_layer_config* cfg, size_t* bytes);

/* Validate cfg, repack the weights into packed_dev (caller-owned, at least
 * llama_layer_packed_bytes, 256-byte aligned) on `stream`, build the RoPE
 * table, and return a handle.  gamma_1 is folded into the q/k/v weights (in
 * fp32, rounded once to cfg.dtype); gamma_2 scales the fp32 residual stream
 * when it is converted to the gate/up operand.
 * Synchronises `stream` before returning, so the source weights may be freed
 * afterwards.  packed_dev must outlive the handle. */
llama_status llama_layer_create(const llama_layer_config* cfg, const llama_layer_weights* w,
                                void* packed_dev, void* stream, llama_layer** out);

/* Workspace bytes for calls with at most max_tokens tokens (B*S in a
 * prefill, B in a decode) and at most max_batch sequences per call, with
 * positions below the layer's max_position. */
llama_status llama_layer_workspace_bytes(const llama_layer* layer, int32_t max_tokens,
                                         int32_t max_batch, size_t* bytes);

llama_status llama_layer_destroy(llama_layer* layer);

/* ---- paged KV cache ---------------------------------------------------- */

/* Device bytes of a pool holding num_blocks blocks of block_size tokens for
 * the G KV heads of one layer, plus the block tables of max_seqs sequences
 * of up to cfg.max_position tokens.  Only block_size 16 is supported. */
llama_status llama_kv_cache_bytes(const llama_layer_config* cfg, int32_t num_blocks,
                                  int32_t block_size, int32_t max_seqs, size_t* bytes);

/* Create a cache over pool_dev (caller-owned, llama_kv_cache_bytes, 256-byte
 * aligned).  block_order, if not NULL, is a permutation of [0, num_blocks)
 * giving the order in which physical blocks are handed out (NULL: 0, 1, ...). */
llama_status llama_kv_cache_create(const llama_layer_config* cfg, int32_t num_blocks,
                                   int32_t block_size, int32_t max_seqs,
                                   const int32_t* block_order, void* pool_dev,
                                   llama_kv_cache** out);

/* The same for a stack of n_layers layers of config cfg: one K and one V pool
 * per layer ("Chapter 10", section 8: the cache holds K and V for every
 * layer), laid out [n_layers][num_blocks][...], all indexed by one set of
 * block tables, so a sequence's block i holds the same 16 positions in every
 * layer.  n_layers = 1 is the single-layer cache above.  On a cache with
 * n_layers > 1, llama_kv_cache_write and llama_kv_cache_read move
 * [n_layers, n, G, D] buffers (layer-major); llama_layer_prefill/decode
 * reject it (LLAMA_ERR_SHAPE): it is used through llama_stack_*. */
llama_status llama_kv_cache_bytes_layers(const llama_layer_config* cfg, int32_t n_layers,
                                         int32_t num_blocks, int32_t block_size, int32_t max_seqs,
                                         size_t* bytes);
llama_status llama_kv_cache_create_layers(const llama_layer_config* cfg, int32_t n_layers,
                                          int32_t num_blocks, int32_t block_size, int32_t max_seqs,
                                          const int32_t* block_order, void* pool_dev,
                                          llama_kv_cache** out);
llama_status llama_kv_cache_num_layers(const llama_kv_cache* cache, int32_t* n_layers);
llama_status llama_kv_cache_destroy(llama_kv_cache* cache);

/* Open an empty sequence; its id is in [0, max_seqs). */
llama_status llama_kv_cache_add_seq(llama_kv_cache* cache, int32_t* seq_id_out);
/* Close a sequence and return its blocks to the pool. */
llama_status llama_kv_cache_free_seq(llama_kv_cache* cache, int32_t seq_id);
llama_status llama_kv_cache_seq_len(const llama_kv_cache* cache, int32_t seq_id, int32_t* len);
/* Free blocks remaining in the pool. */
llama_status llama_kv_cache_free_blocks(const llama_kv_cache* cache, int32_t* n);

/* Append n_tokens already-rotated keys and values ([n, G, D] each, device,
 * cfg.dtype; [n_layers, n, G, D] for a multi-layer cache) to a sequence
 * (positions len .. len+n-1).  Used to restore a saved cache or to pre-fill
 * one.  The length advances after the copies are enqueued; if a launch fails
 * (LLAMA_ERR_HIP) the blocks reserved for the call go back to the pool. */
llama_status llama_kv_cache_write(llama_kv_cache* cache, int32_t seq_id, int32_t n_tokens,
                                  const void* k_dev, const void* v_dev, void* stream);

/* Copy positions start .. start+n-1 of a sequence into [n, G, D] buffers
 * ([n_layers, n, G, D] for a multi-layer cache). */
llama_status llama_kv_cache_read(const llama_kv_cache* cache, int32_t seq_id, int32_t start,
                                 int32_t n, void* k_dev, void* v_dev, void* stream);

/* ---- forward ----------------------------------------------------------- */

/* Causal prefill of `batch` sequences of seq_len new tokens each.
 * x: [batch, seq_len, d] (cfg.dtype); out: [batch, seq_len, d] in out_dtype
 * (a llama_dtype; LLAMA_DTYPE_BF16 only for a bf16 layer).
 * seq_ids: host array of `batch` distinct open sequences.  Sequence b's new
 * tokens take positions len_b .. len_b+seq_len-1 and see every cached key
 * at or before their position; their K/V are appended to the cache.
 * workspace: device scratch of workspace_bytes bytes (caller-owned, 256-byte
 * aligned, contents need not be initialised and are not kept between calls);
 * a workspace_bytes below llama_layer_workspace_bytes(batch*seq_len, batch)
 * is rejected with LLAMA_ERR_INVALID_ARG before any device work.
 * Cache bookkeeping: the sequence lengths advance only once every kernel of
 * the call has been enqueued.  If a launch fails (LLAMA_ERR_HIP) the lengths
 * and the block allocation are restored to their state before the call (the
 * K/V the call already wrote sit past the restored lengths and are
 * overwritten by the next call). */
llama_status llama_layer_prefill(llama_layer* layer, llama_kv_cache* cache, int32_t batch,
                                 int32_t seq_len, const int32_t* seq_ids, const void* x,
                                 void* out, int32_t out_dtype, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* One decode step: token b sits at position len_b of sequence seq_ids[b],
 * is appended to the cache and attends to all len_b + 1 keys.
 * x: [batch, d]; out: [batch, d] in out_dtype.
 * workspace / workspace_bytes: as for prefill, with at least
 * llama_layer_workspace_bytes(batch, batch) bytes.  Bookkeeping and failure
 * behaviour as for prefill. */
llama_status llama_layer_decode(llama_layer* layer, llama_kv_cache* cache, int32_t batch,
                                const int32_t* seq_ids, const void* x, void* out,
                                int32_t out_dtype, void* workspace, size_t workspace_bytes,
                                void* stream);

/* ---- decode without allocation ---------------------------------------- */

/* Bytes of the static device scratch buffer behind llama_layer_decode_noalloc. */
#define LLAMA_SCRATCH_BYTES ((size_t)64 << 20)

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 * llama_layer_decode with the workspace taken from a static device array of
 * LLAMA_SCRATCH_BYTES bytes inside the library, of which every GPU the
 * library runs on holds one copy until the process ends.  Arguments,
 * results, bookkeeping and errors are those of llama_layer_decode; a call
 * whose workspace (llama_layer_workspace_bytes(batch, batch)) exceeds
 * LLAMA_SCRATCH_BYTES returns LLAMA_ERR_SCRATCH before any device work.  The
 * call allocates nothing (no hipMalloc, no events: per-kernel timing is not
 * recorded for it); on the first call on a device it looks up that device's
 * copy of the array.  Every call on a GPU shares that GPU's copy: calls that
 * overlap in time on one GPU (other streams, other threads) race and must be
 * serialised by the caller.  No kernel needs the buffer cleared: each call
 * writes every scratch byte it reads before reading it. */
llama_status llama_layer_decode_noalloc(llama_layer* layer, llama_kv_cache* cache, int32_t batch,
                                        const int32_t* seq_ids, const void* x, void* out,
                                        int32_t out_dtype, void* stream);

/* ---- stack of layers + final RMSNorm ---------------------------------- */

/* The model-level use of the layer ("From Transformer to the LLaMA series",
 * section 8, LlamaModel.forward; section 3.3 and self-test Q1: Pre-LN needs
 * one more RMSNorm after the last block; "From Transformer to LLaMA: an
 * overview", 4.1):
 *   x_{l+1} = layer_l(x_l), l = 0 .. n_layers-1;  y = RMSNorm_final(x_L)
 * The hidden state between layers (and into the final norm) is held in
 * cfg.dtype.  The final norm uses the layers' rms_norm_eps.
 *
 * layers: n_layers handles created with identical configs (else
 * LLAMA_ERR_SHAPE), run in array order; they must outlive the stack, and the
 * stack does not own them.  final_norm: device [d] gamma in cfg.dtype,
 * caller-owned, must outlive the stack. */
llama_status llama_stack_create(llama_layer* const* layers, int32_t n_layers, const void* final_norm,
                                llama_stack** out);

/* Workspace bytes for stack calls with at most max_tokens tokens and
 * max_batch sequences (one layer's workspace plus two [T, d] hidden-state
 * buffers). */
llama_status llama_stack_workspace_bytes(const llama_stack* stack, int32_t max_tokens, int32_t max_batch,
                                         size_t* bytes);
llama_status llama_stack_destroy(llama_stack* stack);

/* Prefill / decode through every layer and the final norm, with the
 * arguments and semantics of llama_layer_prefill / llama_layer_decode; cache
 * must have been created with n_layers equal to the stack's (else
 * LLAMA_ERR_SHAPE); workspace_bytes must be at least
 * llama_stack_workspace_bytes for the call (else LLAMA_ERR_INVALID_ARG).
 * Layer l reads and appends the K/V of its own pools; the sequence lengths
 * advance once per call, after the last launch (restored if a launch fails).
 * out holds y.  Per-kernel timing is recorded by each layer's handle; the
 * final norm ("rms_final_norm") is counted with the last layer. */
llama_status llama_stack_prefill(llama_stack* stack, llama_kv_cache* cache, int32_t batch,
                                 int32_t seq_len, const int32_t* seq_ids, const void* x,
                                 void* out, int32_t out_dtype, void* workspace,
                                 size_t workspace_bytes, void* stream);
llama_status llama_stack_decode(llama_stack* stack, llama_kv_cache* cache, int32_t batch,
                                const int32_t* seq_ids, const void* x, void* out,
                                int32_t out_dtype, void* workspace, size_t workspace_bytes,
                                void* stream);

/* ---- measurement ------------------------------------------------------ */

/* Per-kernel totals of a layer's forward calls while profiling is on. */
typedef struct {
  char name[32];     /* kernel family, e.g. "gemm_gate_up_swiglu" */
  int32_t launches;  /* kernels launched */
  double total_ms;   /* summed device time between the events around each launch */
} llama_kernel_time;

/* Turn per-kernel timing on (1) or off (0): while on, every kernel a forward
 * call launches is bracketed by two HIP events on the call's stream.  The
 * events add no device work.  Turning it off drops unread measurements. */
llama_status llama_layer_profile_enable(llama_layer* layer, int32_t enable);

/* Wait for the recorded events and fill out[0..*n) with the totals per kernel
 * family since the last reset (at most max entries).  reset != 0 clears the
 * totals afterwards.  Blocks the host until the recorded work has finished. */
llama_status llama_layer_profile_read(llama_layer* layer, llama_kernel_time* out, int32_t max,
                                      int32_t* n, int32_t reset);

#ifdef __cplusplus
}
#endif

#endif /* LLAMA_LAYER_H */
