"""ctypes binding of libllama_layer.so (include/llama_layer.h).

The functions below carry the C names and only marshal arguments: every step
of the layer runs inside the library's HIP kernels.  PyTorch is used for
device memory and streams only.  If the library has not been built, the
binding raises instead of falling back to anything else.

Two thin owners of device memory sit on top, DecoderLayer and PagedKVCache;
they allocate the caller-owned buffers the C API asks for as torch tensors.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libllama_layer.so")

LLAMA_DTYPE_F32 = 0
LLAMA_DTYPE_BF16 = 1

STATUS = {0: "LLAMA_OK", -1: "LLAMA_ERR_INVALID_ARG", -2: "LLAMA_ERR_SHAPE", -3: "LLAMA_ERR_DTYPE",
          -4: "LLAMA_ERR_CACHE_FULL", -5: "LLAMA_ERR_BAD_SEQ", -6: "LLAMA_ERR_POSITION",
          -7: "LLAMA_ERR_HIP", -8: "LLAMA_ERR_UNSUPPORTED", -9: "LLAMA_ERR_SCRATCH"}

EXPORTED = ("llama_status_string", "llama_layer_packed_bytes", "llama_layer_create",
            "llama_layer_workspace_bytes", "llama_layer_destroy", "llama_kv_cache_bytes",
            "llama_kv_cache_create", "llama_kv_cache_destroy", "llama_kv_cache_add_seq",
            "llama_kv_cache_free_seq", "llama_kv_cache_seq_len", "llama_kv_cache_free_blocks",
            "llama_kv_cache_write", "llama_kv_cache_read", "llama_layer_prefill", "llama_layer_decode",
            "llama_layer_profile_enable", "llama_layer_profile_read", "llama_kv_cache_bytes_layers",
            "llama_kv_cache_create_layers", "llama_kv_cache_num_layers", "llama_stack_create",
            "llama_stack_workspace_bytes", "llama_stack_destroy", "llama_stack_prefill", "llama_stack_decode",
            "llama_layer_decode_noalloc")

# bytes of the library's static scratch buffer (LLAMA_SCRATCH_BYTES in the header)
SCRATCH_BYTES = 64 << 20


class LlamaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}")


class LlamaLayerConfig(ctypes.Structure):
    _fields_ = [("hidden_size", ctypes.c_int32), ("intermediate_size", ctypes.c_int32),
                ("num_attention_heads", ctypes.c_int32), ("num_key_value_heads", ctypes.c_int32),
                ("rms_norm_eps", ctypes.c_float), ("rope_theta", ctypes.c_float),
                ("max_position", ctypes.c_int32), ("dtype", ctypes.c_int), ("rope_style", ctypes.c_int32)]


class LlamaLayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("q_proj", "k_proj", "v_proj", "o_proj", "gate_proj", "up_proj", "down_proj",
                 "input_layernorm", "post_attention_layernorm")]


class LlamaKernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", ctypes.c_int32), ("total_ms", ctypes.c_double)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load the library (after torch, so both share one HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m decoder_block_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    cfgp = ctypes.POINTER(LlamaLayerConfig)
    sig = {
        "llama_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "llama_layer_packed_bytes": (ctypes.c_int, [cfgp, ctypes.POINTER(SZ)]),
        "llama_layer_create": (ctypes.c_int, [cfgp, ctypes.POINTER(LlamaLayerWeights), P, P, ctypes.POINTER(P)]),
        "llama_layer_workspace_bytes": (ctypes.c_int, [P, I32, I32, ctypes.POINTER(SZ)]),
        "llama_layer_destroy": (ctypes.c_int, [P]),
        "llama_kv_cache_bytes": (ctypes.c_int, [cfgp, I32, I32, I32, ctypes.POINTER(SZ)]),
        "llama_kv_cache_create": (ctypes.c_int, [cfgp, I32, I32, I32, ctypes.POINTER(I32), P, ctypes.POINTER(P)]),
        "llama_kv_cache_destroy": (ctypes.c_int, [P]),
        "llama_kv_cache_add_seq": (ctypes.c_int, [P, ctypes.POINTER(I32)]),
        "llama_kv_cache_free_seq": (ctypes.c_int, [P, I32]),
        "llama_kv_cache_seq_len": (ctypes.c_int, [P, I32, ctypes.POINTER(I32)]),
        "llama_kv_cache_free_blocks": (ctypes.c_int, [P, ctypes.POINTER(I32)]),
        "llama_kv_cache_write": (ctypes.c_int, [P, I32, I32, P, P, P]),
        "llama_kv_cache_read": (ctypes.c_int, [P, I32, I32, I32, P, P, P]),
        "llama_layer_prefill": (ctypes.c_int, [P, P, I32, I32, ctypes.POINTER(I32), P, P, ctypes.c_int, P, SZ, P]),
        "llama_layer_decode": (ctypes.c_int, [P, P, I32, ctypes.POINTER(I32), P, P, ctypes.c_int, P, SZ, P]),
        "llama_layer_profile_enable": (ctypes.c_int, [P, I32]),
        "llama_layer_profile_read": (ctypes.c_int, [P, ctypes.POINTER(LlamaKernelTime), I32, ctypes.POINTER(I32), I32]),
        "llama_kv_cache_bytes_layers": (ctypes.c_int, [cfgp, I32, I32, I32, I32, ctypes.POINTER(SZ)]),
        "llama_kv_cache_create_layers": (ctypes.c_int, [cfgp, I32, I32, I32, I32, ctypes.POINTER(I32), P,
                                                        ctypes.POINTER(P)]),
        "llama_kv_cache_num_layers": (ctypes.c_int, [P, ctypes.POINTER(I32)]),
        "llama_stack_create": (ctypes.c_int, [ctypes.POINTER(P), I32, P, ctypes.POINTER(P)]),
        "llama_stack_workspace_bytes": (ctypes.c_int, [P, I32, I32, ctypes.POINTER(SZ)]),
        "llama_stack_destroy": (ctypes.c_int, [P]),
        "llama_stack_prefill": (ctypes.c_int, [P, P, I32, I32, ctypes.POINTER(I32), P, P, ctypes.c_int, P, SZ, P]),
        "llama_stack_decode": (ctypes.c_int, [P, P, I32, ctypes.POINTER(I32), P, P, ctypes.c_int, P, SZ, P]),
        "llama_layer_decode_noalloc": (ctypes.c_int, [P, P, I32, ctypes.POINTER(I32), P, P, ctypes.c_int, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def _check(status: int, where: str):
    if status != 0:
        raise LlamaError(status, where)


ROPE_STYLES = {"interleaved": 0, "half_split": 1}


def make_config(hidden_size, intermediate_size, num_attention_heads, num_key_value_heads,
                rms_norm_eps, rope_theta, max_position, dtype, rope_style="interleaved") -> LlamaLayerConfig:
    dt = {"f32": LLAMA_DTYPE_F32, "bf16": LLAMA_DTYPE_BF16}.get(dtype, dtype)
    rs = ROPE_STYLES.get(rope_style, rope_style)
    return LlamaLayerConfig(int(hidden_size), int(intermediate_size), int(num_attention_heads),
                            int(num_key_value_heads), float(rms_norm_eps), float(rope_theta),
                            int(max_position), int(dt), int(rs))


def _i32_array(vals):
    arr = (ctypes.c_int32 * len(vals))(*[int(v) for v in vals])
    return arr


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _ptr(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr() if isinstance(t, torch.Tensor) else int(t))


# ---------------------------------------------------------------------------
# same-name functions (status -> exception; outputs returned)
# ---------------------------------------------------------------------------

def llama_status_string(status: int) -> str:
    return lib().llama_status_string(status).decode()


def llama_layer_packed_bytes(cfg: LlamaLayerConfig) -> int:
    n = ctypes.c_size_t()
    _check(lib().llama_layer_packed_bytes(ctypes.byref(cfg), ctypes.byref(n)), "llama_layer_packed_bytes")
    return n.value


def llama_layer_create(cfg: LlamaLayerConfig, weights: LlamaLayerWeights, packed_dev, stream=None):
    h = ctypes.c_void_p()
    _check(lib().llama_layer_create(ctypes.byref(cfg), ctypes.byref(weights), _ptr(packed_dev), _stream(stream),
                                    ctypes.byref(h)), "llama_layer_create")
    return h


def llama_layer_workspace_bytes(layer, max_tokens: int, max_batch: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().llama_layer_workspace_bytes(layer, max_tokens, max_batch, ctypes.byref(n)),
           "llama_layer_workspace_bytes")
    return n.value


def llama_layer_destroy(layer):
    _check(lib().llama_layer_destroy(layer), "llama_layer_destroy")


def llama_kv_cache_bytes(cfg: LlamaLayerConfig, num_blocks: int, block_size: int, max_seqs: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().llama_kv_cache_bytes(ctypes.byref(cfg), num_blocks, block_size, max_seqs, ctypes.byref(n)),
           "llama_kv_cache_bytes")
    return n.value


def llama_kv_cache_create(cfg: LlamaLayerConfig, num_blocks: int, block_size: int, max_seqs: int,
                          pool_dev, block_order=None):
    h = ctypes.c_void_p()
    order = _i32_array(block_order) if block_order is not None else None
    _check(lib().llama_kv_cache_create(ctypes.byref(cfg), num_blocks, block_size, max_seqs, order,
                                       _ptr(pool_dev), ctypes.byref(h)), "llama_kv_cache_create")
    return h


def llama_kv_cache_bytes_layers(cfg: LlamaLayerConfig, n_layers: int, num_blocks: int, block_size: int,
                                max_seqs: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().llama_kv_cache_bytes_layers(ctypes.byref(cfg), n_layers, num_blocks, block_size, max_seqs,
                                             ctypes.byref(n)), "llama_kv_cache_bytes_layers")
    return n.value


def llama_kv_cache_create_layers(cfg: LlamaLayerConfig, n_layers: int, num_blocks: int, block_size: int,
                                 max_seqs: int, pool_dev, block_order=None):
    h = ctypes.c_void_p()
    order = _i32_array(block_order) if block_order is not None else None
    _check(lib().llama_kv_cache_create_layers(ctypes.byref(cfg), n_layers, num_blocks, block_size, max_seqs, order,
                                              _ptr(pool_dev), ctypes.byref(h)), "llama_kv_cache_create_layers")
    return h


def llama_kv_cache_num_layers(cache) -> int:
    n = ctypes.c_int32()
    _check(lib().llama_kv_cache_num_layers(cache, ctypes.byref(n)), "llama_kv_cache_num_layers")
    return n.value


def llama_stack_create(layers, final_norm):
    h = ctypes.c_void_p()
    arr = (ctypes.c_void_p * len(layers))(*[l.value if isinstance(l, ctypes.c_void_p) else l for l in layers])
    _check(lib().llama_stack_create(arr, len(layers), _ptr(final_norm), ctypes.byref(h)), "llama_stack_create")
    return h


def llama_stack_workspace_bytes(stack, max_tokens: int, max_batch: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().llama_stack_workspace_bytes(stack, max_tokens, max_batch, ctypes.byref(n)),
           "llama_stack_workspace_bytes")
    return n.value


def llama_stack_destroy(stack):
    _check(lib().llama_stack_destroy(stack), "llama_stack_destroy")


def _nbytes(t, nbytes):
    """Size of a workspace argument: the tensor's bytes unless given explicitly."""
    if nbytes is not None:
        return int(nbytes)
    if isinstance(t, torch.Tensor):
        return t.numel() * t.element_size()
    raise ValueError("workspace given as an address needs workspace_bytes")


def llama_stack_prefill(stack, cache, batch: int, seq_len: int, seq_ids, x, out, out_dtype: int,
                        workspace, stream=None, workspace_bytes=None):
    _check(lib().llama_stack_prefill(stack, cache, batch, seq_len, _i32_array(seq_ids), _ptr(x), _ptr(out),
                                     out_dtype, _ptr(workspace), _nbytes(workspace, workspace_bytes),
                                     _stream(stream)), "llama_stack_prefill")


def llama_stack_decode(stack, cache, batch: int, seq_ids, x, out, out_dtype: int, workspace, stream=None,
                       workspace_bytes=None):
    _check(lib().llama_stack_decode(stack, cache, batch, _i32_array(seq_ids), _ptr(x), _ptr(out), out_dtype,
                                    _ptr(workspace), _nbytes(workspace, workspace_bytes), _stream(stream)),
           "llama_stack_decode")


def llama_kv_cache_destroy(cache):
    _check(lib().llama_kv_cache_destroy(cache), "llama_kv_cache_destroy")


def llama_kv_cache_add_seq(cache) -> int:
    sid = ctypes.c_int32()
    _check(lib().llama_kv_cache_add_seq(cache, ctypes.byref(sid)), "llama_kv_cache_add_seq")
    return sid.value


def llama_kv_cache_free_seq(cache, seq_id: int):
    _check(lib().llama_kv_cache_free_seq(cache, seq_id), "llama_kv_cache_free_seq")


def llama_kv_cache_seq_len(cache, seq_id: int) -> int:
    n = ctypes.c_int32()
    _check(lib().llama_kv_cache_seq_len(cache, seq_id, ctypes.byref(n)), "llama_kv_cache_seq_len")
    return n.value


def llama_kv_cache_free_blocks(cache) -> int:
    n = ctypes.c_int32()
    _check(lib().llama_kv_cache_free_blocks(cache, ctypes.byref(n)), "llama_kv_cache_free_blocks")
    return n.value


def llama_kv_cache_write(cache, seq_id: int, n_tokens: int, k_dev, v_dev, stream=None):
    _check(lib().llama_kv_cache_write(cache, seq_id, n_tokens, _ptr(k_dev), _ptr(v_dev), _stream(stream)),
           "llama_kv_cache_write")


def llama_kv_cache_read(cache, seq_id: int, start: int, n: int, k_dev, v_dev, stream=None):
    _check(lib().llama_kv_cache_read(cache, seq_id, start, n, _ptr(k_dev), _ptr(v_dev), _stream(stream)),
           "llama_kv_cache_read")


def llama_layer_prefill(layer, cache, batch: int, seq_len: int, seq_ids, x, out, out_dtype: int,
                        workspace, stream=None, workspace_bytes=None):
    _check(lib().llama_layer_prefill(layer, cache, batch, seq_len, _i32_array(seq_ids), _ptr(x), _ptr(out),
                                     out_dtype, _ptr(workspace), _nbytes(workspace, workspace_bytes),
                                     _stream(stream)), "llama_layer_prefill")


def llama_layer_decode(layer, cache, batch: int, seq_ids, x, out, out_dtype: int, workspace, stream=None,
                       workspace_bytes=None):
    _check(lib().llama_layer_decode(layer, cache, batch, _i32_array(seq_ids), _ptr(x), _ptr(out), out_dtype,
                                    _ptr(workspace), _nbytes(workspace, workspace_bytes), _stream(stream)),
           "llama_layer_decode")


def llama_layer_decode_noalloc(layer, cache, batch: int, seq_ids, x, out, out_dtype: int, stream=None):
    """llama_layer_decode with the library's static scratch buffer as workspace (allocates nothing)."""
    _check(lib().llama_layer_decode_noalloc(layer, cache, batch, _i32_array(seq_ids), _ptr(x), _ptr(out), out_dtype,
                                            _stream(stream)), "llama_layer_decode_noalloc")


def llama_layer_profile_enable(layer, enable: bool):
    _check(lib().llama_layer_profile_enable(layer, 1 if enable else 0), "llama_layer_profile_enable")


def llama_layer_profile_read(layer, reset: bool = True) -> dict:
    """{kernel family: (launches, total_ms)} since the last reset (waits for the device)."""
    buf = (LlamaKernelTime * 32)()
    n = ctypes.c_int32()
    _check(lib().llama_layer_profile_read(layer, buf, 32, ctypes.byref(n), 1 if reset else 0),
           "llama_layer_profile_read")
    return {buf[i].name.decode(): (buf[i].launches, buf[i].total_ms) for i in range(n.value)}


# ---------------------------------------------------------------------------
# owners of the caller-side device buffers
# ---------------------------------------------------------------------------

_TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _check_tensor(t: torch.Tensor, what: str, dtype, device, shape=None):
    """The C ABI takes raw pointers: reject tensors it would misread."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what}: expected a torch.Tensor")
    if t.device.type != device.type or (device.index is not None and t.device.index != device.index):
        raise ValueError(f"{what}: on {t.device}, the layer is on {device}")
    if t.dtype != dtype:
        raise ValueError(f"{what}: dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{what}: must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what}: shape {tuple(t.shape)}, expected {tuple(shape)}")


def _dev_bytes(n: int, device) -> torch.Tensor:
    # 256-byte aligned by the caching allocator (it aligns blocks to 512 bytes)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


class DecoderLayer:
    """A packed layer on one device.  ``weights`` maps the nine HF names to tensors."""

    def __init__(self, config: dict, weights: dict, dtype: str, max_position: int, device="cuda", stream=None):
        self.dtype = dtype
        self.tdtype = _TORCH_DT[dtype]
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        self.cfg = make_config(config["hidden_size"], config["intermediate_size"],
                               config["num_attention_heads"], config["num_key_value_heads"],
                               config["rms_norm_eps"], config["rope_theta"], max_position, dtype,
                               config.get("rope_style", "interleaved"))
        self.packed = _dev_bytes(llama_layer_packed_bytes(self.cfg), self.device)
        src = {k: v.to(self.device, self.tdtype).contiguous() for k, v in weights.items()}
        w = LlamaLayerWeights(*[src[n].data_ptr() for n in
                                ("q_proj", "k_proj", "v_proj", "o_proj", "gate_proj", "up_proj", "down_proj",
                                 "input_layernorm", "post_attention_layernorm")])
        self.handle = llama_layer_create(self.cfg, w, self.packed, stream)
        del src
        self._ws = None

    def workspace(self, tokens: int, batch: int) -> torch.Tensor:
        need = llama_layer_workspace_bytes(self.handle, tokens, batch)
        if self._ws is None or self._ws.numel() < need:
            self._ws = _dev_bytes(need, self.device)
        return self._ws

    def prefill(self, cache: "PagedKVCache", seq_ids, x: torch.Tensor, out_dtype="f32", out=None, stream=None):
        B, S, d = x.shape
        odt = _TORCH_DT[out_dtype]
        _check_tensor(x, "x", self.tdtype, self.device, (B, S, self.cfg.hidden_size))
        if out is None:
            out = torch.empty((B, S, d), dtype=odt, device=self.device)
        _check_tensor(out, "out", odt, self.device, (B, S, d))
        ws = self.workspace(B * S, B)
        llama_layer_prefill(self.handle, cache.handle, B, S, list(seq_ids), x, out,
                            LLAMA_DTYPE_F32 if out_dtype == "f32" else LLAMA_DTYPE_BF16, ws, stream)
        return out

    def decode(self, cache: "PagedKVCache", seq_ids, x: torch.Tensor, out_dtype="f32", out=None, stream=None):
        B, d = x.shape
        odt = _TORCH_DT[out_dtype]
        _check_tensor(x, "x", self.tdtype, self.device, (B, self.cfg.hidden_size))
        if out is None:
            out = torch.empty((B, d), dtype=odt, device=self.device)
        _check_tensor(out, "out", odt, self.device, (B, d))
        ws = self.workspace(B, B)
        llama_layer_decode(self.handle, cache.handle, B, list(seq_ids), x, out,
                           LLAMA_DTYPE_F32 if out_dtype == "f32" else LLAMA_DTYPE_BF16, ws, stream)
        return out

    def close(self):
        if getattr(self, "handle", None):
            llama_layer_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class PagedKVCache:
    """A paged K/V pool of ``num_blocks`` 16-token blocks, for one layer or
    (``n_layers`` > 1) for every layer of a stack, sharing one block table."""

    def __init__(self, layer: DecoderLayer, num_blocks: int, max_seqs: int, block_order=None, n_layers: int = 1):
        self.layer = layer
        self.n_layers = n_layers
        self.pool = _dev_bytes(llama_kv_cache_bytes_layers(layer.cfg, n_layers, num_blocks, 16, max_seqs),
                               layer.device)
        self.handle = llama_kv_cache_create_layers(layer.cfg, n_layers, num_blocks, 16, max_seqs, self.pool,
                                                   block_order)

    def add_seq(self) -> int:
        return llama_kv_cache_add_seq(self.handle)

    def free_seq(self, sid: int):
        llama_kv_cache_free_seq(self.handle, sid)

    def seq_len(self, sid: int) -> int:
        return llama_kv_cache_seq_len(self.handle, sid)

    def free_blocks(self) -> int:
        return llama_kv_cache_free_blocks(self.handle)

    def write(self, sid: int, k: torch.Tensor, v: torch.Tensor, stream=None):
        """k, v: [n, G, D] (one layer) or [n_layers, n, G, D]."""
        n = k.shape[0] if self.n_layers == 1 and k.dim() == 3 else k.shape[1]
        G, D = self.layer.cfg.num_key_value_heads, self.layer.cfg.hidden_size // self.layer.cfg.num_attention_heads
        shape = (n, G, D) if self.n_layers == 1 and k.dim() == 3 else (self.n_layers, n, G, D)
        k, v = k.contiguous(), v.contiguous()
        _check_tensor(k, "k", self.layer.tdtype, self.layer.device, shape)
        _check_tensor(v, "v", self.layer.tdtype, self.layer.device, shape)
        llama_kv_cache_write(self.handle, sid, n, k, v, stream)

    def read(self, sid: int, start: int, n: int):
        """[n, G, D] K and V (one layer) or [n_layers, n, G, D]."""
        G, D = self.layer.cfg.num_key_value_heads, self.layer.cfg.hidden_size // self.layer.cfg.num_attention_heads
        shape = (n, G, D) if self.n_layers == 1 else (self.n_layers, n, G, D)
        k = torch.empty(shape, dtype=self.layer.tdtype, device=self.layer.device)
        v = torch.empty_like(k)
        llama_kv_cache_read(self.handle, sid, start, n, k, v)
        return k, v

    def close(self):
        if getattr(self, "handle", None):
            llama_kv_cache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class DecoderStack:
    """``layers`` (DecoderLayer, one config) run in order, then the final RMSNorm
    with gamma ``final_norm`` [d]; calls take a PagedKVCache with as many layers."""

    def __init__(self, layers, final_norm: torch.Tensor):
        self.layers = list(layers)
        l0 = self.layers[0]
        self.device = l0.device
        self.final_norm = final_norm.to(l0.device, l0.tdtype).contiguous()
        self.handle = llama_stack_create([l.handle for l in self.layers], self.final_norm)
        self._ws = None

    def cache(self, num_blocks: int, max_seqs: int, block_order=None) -> PagedKVCache:
        return PagedKVCache(self.layers[0], num_blocks, max_seqs, block_order, n_layers=len(self.layers))

    def workspace(self, tokens: int, batch: int) -> torch.Tensor:
        need = llama_stack_workspace_bytes(self.handle, tokens, batch)
        if self._ws is None or self._ws.numel() < need:
            self._ws = _dev_bytes(need, self.device)
        return self._ws

    def prefill(self, cache: PagedKVCache, seq_ids, x: torch.Tensor, out_dtype="f32", out=None, stream=None):
        B, S, d = x.shape
        l0 = self.layers[0]
        _check_tensor(x, "x", l0.tdtype, self.device, (B, S, l0.cfg.hidden_size))
        if out is None:
            out = torch.empty((B, S, d), dtype=_TORCH_DT[out_dtype], device=self.device)
        _check_tensor(out, "out", _TORCH_DT[out_dtype], self.device, (B, S, d))
        ws = self.workspace(B * S, B)
        llama_stack_prefill(self.handle, cache.handle, B, S, list(seq_ids), x, out,
                            LLAMA_DTYPE_F32 if out_dtype == "f32" else LLAMA_DTYPE_BF16, ws, stream)
        return out

    def decode(self, cache: PagedKVCache, seq_ids, x: torch.Tensor, out_dtype="f32", out=None, stream=None):
        B, d = x.shape
        l0 = self.layers[0]
        _check_tensor(x, "x", l0.tdtype, self.device, (B, l0.cfg.hidden_size))
        if out is None:
            out = torch.empty((B, d), dtype=_TORCH_DT[out_dtype], device=self.device)
        _check_tensor(out, "out", _TORCH_DT[out_dtype], self.device, (B, d))
        ws = self.workspace(B, B)
        llama_stack_decode(self.handle, cache.handle, B, list(seq_ids), x, out,
                           LLAMA_DTYPE_F32 if out_dtype == "f32" else LLAMA_DTYPE_BF16, ws, stream)
        return out

    def close(self):
        if getattr(self, "handle", None):
            llama_stack_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
