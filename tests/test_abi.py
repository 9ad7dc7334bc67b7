"""CPU checks of the C-ABI library: it loads, exports every declared symbol, and
its host-side validation and block bookkeeping behave as documented.  No call
here reaches the GPU (calls that would are expected to fail validation first,
or take a fake pool address that is never dereferenced)."""
import ctypes
import os
import re
import subprocess

import pytest

from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "llama_layer.h")


@pytest.fixture(scope="session")
def L():
    from decoder_block_amd import build, llama_layer
    if not os.path.exists(llama_layer.LIB_PATH):
        build.build()
    return llama_layer


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(llama_\w+)\s*\(", text)))


def test_library_exports_every_declared_function(L):
    lib = L.lib()
    names = declared_functions()
    assert len(names) >= 16
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(L.EXPORTED) == names


def test_status_strings(L):
    assert L.llama_status_string(0) == "ok"
    assert L.llama_status_string(-4) == "KV cache full"


def _cfg(L, **kw):
    base = dict(hidden_size=4096, intermediate_size=14336, num_attention_heads=32, num_key_value_heads=8,
                rms_norm_eps=1e-5, rope_theta=500000.0, max_position=8321, dtype="bf16")
    base.update(kw)
    return L.make_config(**base)


def test_packed_bytes_cover_the_weights(L):
    n = L.llama_layer_packed_bytes(_cfg(L))
    weights = 2 * (4096 * 6144 + 4096 * 4096 + 2 * 14336 * 4096 + 4096 * 14336)
    rope = 2 * 8321 * 64 * 4
    gamma2 = 4096 * 4
    assert weights + rope + gamma2 <= n <= weights + rope + gamma2 + 8 * 256


@pytest.mark.parametrize("kw,status", [
    (dict(num_key_value_heads=3), "LLAMA_ERR_SHAPE"),          # H % G != 0
    (dict(hidden_size=4100), "LLAMA_ERR_SHAPE"),               # d % H != 0
    (dict(hidden_size=96 * 32), "LLAMA_ERR_UNSUPPORTED"),      # head_dim 96
    (dict(num_attention_heads=128, num_key_value_heads=2, hidden_size=8192), "LLAMA_ERR_UNSUPPORTED"),  # R = 64
    (dict(rms_norm_eps=0.0), "LLAMA_ERR_INVALID_ARG"),
    (dict(rope_theta=float("nan")), "LLAMA_ERR_INVALID_ARG"),
    (dict(max_position=0), "LLAMA_ERR_INVALID_ARG"),
    (dict(dtype=5), "LLAMA_ERR_DTYPE"),
    (dict(rope_style=2), "LLAMA_ERR_INVALID_ARG"),
])
def test_config_validation(L, kw, status):
    with pytest.raises(L.LlamaError) as e:
        L.llama_layer_packed_bytes(_cfg(L, **kw))
    assert L.STATUS[e.value.status] == status


def test_kv_cache_bytes_and_block_size(L):
    cfg = _cfg(L)
    n = L.llama_kv_cache_bytes(cfg, 1000, 16, 64)
    pool = 2 * 1000 * 8 * 16 * 128 * 2
    table = 64 * ((8321 + 15) // 16) * 4
    assert pool + table <= n <= pool + table + 3 * 256
    with pytest.raises(L.LlamaError):
        L.llama_kv_cache_bytes(cfg, 1000, 32, 64)


def test_cache_bookkeeping_without_device(L):
    cfg = _cfg(L, max_position=64)
    fake_pool = 1 << 40  # never dereferenced by these calls
    with pytest.raises(L.LlamaError):
        L.llama_kv_cache_create(cfg, 4, 16, 2, fake_pool, block_order=[0, 0, 1, 2])
    c = L.llama_kv_cache_create(cfg, 4, 16, 2, fake_pool, block_order=[3, 1, 0, 2])
    a = L.llama_kv_cache_add_seq(c)
    b = L.llama_kv_cache_add_seq(c)
    assert (a, b) == (0, 1)
    with pytest.raises(L.LlamaError) as e:
        L.llama_kv_cache_add_seq(c)
    assert L.STATUS[e.value.status] == "LLAMA_ERR_CACHE_FULL"
    assert L.llama_kv_cache_seq_len(c, a) == 0
    assert L.llama_kv_cache_free_blocks(c) == 4
    # writes beyond max_position or the pool are rejected before any device work
    with pytest.raises(L.LlamaError) as e:
        L.llama_kv_cache_write(c, a, 65, 1 << 41, 1 << 41, stream=0)
    assert L.STATUS[e.value.status] == "LLAMA_ERR_POSITION"
    with pytest.raises(L.LlamaError) as e:
        L.llama_kv_cache_read(c, a, 0, 1, 1 << 41, 1 << 41, stream=0)
    assert L.STATUS[e.value.status] == "LLAMA_ERR_POSITION"
    L.llama_kv_cache_free_seq(c, b)
    with pytest.raises(L.LlamaError) as e:
        L.llama_kv_cache_seq_len(c, b)
    assert L.STATUS[e.value.status] == "LLAMA_ERR_BAD_SEQ"
    L.llama_kv_cache_destroy(c)


def test_forward_rejects_null_handles(L):
    lib = L.lib()
    ids = (ctypes.c_int32 * 1)(0)
    assert lib.llama_layer_prefill(None, None, 1, 1, ids, None, None, 0, None, 0, None) == -1
    assert lib.llama_layer_decode(None, None, 1, ids, None, None, 0, None, 0, None) == -1
    assert lib.llama_stack_prefill(None, None, 1, 1, ids, None, None, 0, None, 0, None) == -1
    assert lib.llama_stack_decode(None, None, 1, ids, None, None, 0, None, 0, None) == -1


def test_binding_rejects_tensors_the_abi_would_misread(L):
    # The binding passes raw pointers; it must refuse what the pointer alone
    # cannot describe (CPU tensors stand in for device tensors here).
    import torch
    dev = torch.device("cpu")
    x = torch.zeros(2, 3, 8, dtype=torch.bfloat16)
    L._check_tensor(x, "x", torch.bfloat16, dev, (2, 3, 8))
    # a device without an index accepts any index of its type
    assert torch.device("cuda").index is None
    L._check_tensor(torch.zeros(2, device="meta"), "x", torch.float32, torch.device("meta"), (2,))
    with pytest.raises(ValueError, match="contiguous"):
        L._check_tensor(x.transpose(0, 1), "x", torch.bfloat16, dev, None)
    with pytest.raises(ValueError, match="dtype"):
        L._check_tensor(x.float(), "x", torch.bfloat16, dev, (2, 3, 8))
    with pytest.raises(ValueError, match="shape"):
        L._check_tensor(x, "x", torch.bfloat16, dev, (2, 3, 16))
    with pytest.raises(ValueError, match="on cpu"):
        L._check_tensor(x, "x", torch.bfloat16, torch.device("meta"), (2, 3, 8))
    with pytest.raises(TypeError):
        L._check_tensor([0], "x", torch.bfloat16, dev)


def test_host_runtime_under_asan_ubsan():
    """Builds the host runtime with stub kernels under ASan/UBSan and runs its checks."""
    from decoder_block_amd import build
    exe = build.build_host_asan()
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120,
                       env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1"))
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout
