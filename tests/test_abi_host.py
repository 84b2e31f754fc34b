"""Host-side checks of the C ABI: the library loads, exports every declared
symbol, sizes workspaces, and rejects bad arguments before touching a GPU.

No call here reaches a kernel launch: every call either is a pure host query
or fails argument validation, which runs before anything is enqueued.
"""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "strata_moe.h")


def _lib():
    from quantized_expert_ffn_histogram_amd import _abi

    if not os.path.exists(_abi.LIB_PATH):
        pytest.skip("library not built")
    return _abi, _abi.load()


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(strata_\w+)\s*\(", text)))


def test_header_declares_the_four_calls():
    syms = declared_symbols()
    for name in ("strata_moe_route", "strata_moe_permute", "strata_moe_ffn", "strata_moe_combine"):
        assert name in syms


def test_every_declared_symbol_is_exported():
    abi, lib = _lib()
    syms = declared_symbols()
    out = subprocess.run(["nm", "-D", "--defined-only", abi.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (strata_\w+)", out))
    for name in syms:
        assert name in exported, name
        assert hasattr(lib, name)
        assert name in abi.SIGNATURES


def test_workspace_size_valid_and_invalid():
    _, lib = _lib()
    # prefill chunk: h (T*k*I fp16) dominates
    n = lib.strata_moe_workspace_size(6144, 512, 10, 2048, 512, 64)
    assert n >= 6144 * 10 * 512 * 2
    assert n % 256 == 0
    assert lib.strata_moe_workspace_size(4, 512, 10, 2048, 512, 64) > 0
    assert lib.strata_moe_workspace_size(4, 512, 600, 2048, 512, 64) == 0  # k > E
    assert lib.strata_moe_workspace_size(4, 512, 10, 2048, 512, 48) == 0  # bad group
    assert lib.strata_moe_workspace_size(-1, 512, 10, 2048, 512, 64) == 0


def _err(lib):
    return lib.strata_moe_last_error().decode()


@pytest.mark.parametrize(
    "T,E,k,code,needle",
    [
        (-1, 16, 2, 1, "T=-1"),
        (4, 0, 1, 1, "E=0"),
        (4, 2000, 2, 2, "E=2000"),
        (4, 16, 0, 1, "k=0"),
        (4, 16, 17, 1, "k=17 exceeds E=16"),
        (4, 512, 40, 2, "k=40"),
    ],
)
def test_route_rejects_bad_sizes(T, E, k, code, needle):
    _, lib = _lib()
    assert lib.strata_moe_route(None, T, E, k, None, None, None) == code
    assert needle in _err(lib)
    assert _err(lib).startswith("strata_moe_route")


def test_route_rejects_null_and_misaligned_pointers():
    _, lib = _lib()
    assert lib.strata_moe_route(None, 4, 16, 2, None, None, None) == 1
    assert "logits is NULL" in _err(lib)
    assert lib.strata_moe_route(ctypes.c_void_p(0x1004), 4, 16, 2, ctypes.c_void_p(0x2000),
                                ctypes.c_void_p(0x3000), None) == 1
    assert "not 16-byte aligned" in _err(lib)


@pytest.mark.parametrize(
    "T,H,E,k,code,needle",
    [
        (4, 100, 16, 2, 2, "H=100"),
        (4, 0, 16, 2, 2, "H=0"),
        (4, 32768, 16, 2, 2, "H=32768"),
        (4, 256, 16, 17, 1, "k=17 exceeds E=16"),
        (-1, 256, 16, 2, 1, "T=-1"),
        (1 << 20, 2048, 16, 2, 2, "2^30"),
    ],
)
def test_router_rejects_bad_sizes(T, H, E, k, code, needle):
    _, lib = _lib()
    assert lib.strata_moe_router(None, T, H, None, E, k, None, None, None, None) == code
    assert needle in _err(lib)
    assert _err(lib).startswith("strata_moe_router")


def test_router_rejects_null_and_misaligned_pointers():
    _, lib = _lib()
    assert lib.strata_moe_router(None, 4, 256, None, 16, 2, None, None, None, None) == 1
    assert "x_bf16 is NULL" in _err(lib)
    assert lib.strata_moe_router(ctypes.c_void_p(0x1000), 4, 256, ctypes.c_void_p(0x2008), 16, 2,
                                 ctypes.c_void_p(0x3000), ctypes.c_void_p(0x4000), ctypes.c_void_p(0x5000),
                                 None) == 1
    assert "not 16-byte aligned" in _err(lib)
    assert lib.strata_moe_router(None, 0, 256, None, 16, 2, None, None, None, None) == 0  # T = 0: nothing


def test_zero_tokens_is_ok_and_launches_nothing():
    _, lib = _lib()
    assert lib.strata_moe_route(None, 0, 16, 2, None, None, None) == 0
    assert _err(lib) == ""
    assert lib.strata_moe_combine(None, None, None, 0, 2, 256, None, None) == 0


def test_permute_requires_workspace_for_large_inputs():
    _, lib = _lib()
    fake = ctypes.c_void_p(0x10000)
    args = [fake, 6144, 512, 10, fake, fake, fake, fake]
    assert lib.strata_moe_permute(*args, None, 0, None) == 3
    assert "workspace is NULL" in _err(lib)
    assert lib.strata_moe_permute(*args, fake, 16, None) == 3
    assert "workspace_bytes=16" in _err(lib)
    assert lib.strata_moe_permute(*args, ctypes.c_void_p(0x10010), 1 << 30, None) == 1
    assert "256-byte aligned" in _err(lib)


def _weights(abi, E=16, H=256, I=128, g=32, ptr=0x10000):
    p = ctypes.c_void_p(ptr).value
    return abi.StrataMoeWeights(p, p, p, p, p, p, E, H, I, g)


@pytest.mark.parametrize(
    "kw,code,needle",
    [
        (dict(g=48), 2, "group=48"),
        (dict(H=300), 2, "hidden=300"),
        (dict(I=100), 2, "inter=100"),
        (dict(E=2000), 2, "E=2000"),
    ],
)
def test_ffn_rejects_unsupported_shapes(kw, code, needle):
    abi, lib = _lib()
    w = _weights(abi, **kw)
    fake = ctypes.c_void_p(0x10000)
    rc = lib.strata_moe_ffn(fake, 8, 2, ctypes.byref(w), fake, fake, None, fake, fake, 1 << 30, None)
    assert rc == code
    assert needle in _err(lib)


def test_ffn_rejects_null_weights_and_small_workspace():
    abi, lib = _lib()
    fake = ctypes.c_void_p(0x10000)
    assert lib.strata_moe_ffn(fake, 8, 2, None, fake, fake, None, fake, fake, 1 << 30, None) == 1
    assert "w is NULL" in _err(lib)
    w = _weights(abi)
    w.down = None
    assert lib.strata_moe_ffn(fake, 8, 2, ctypes.byref(w), fake, fake, None, fake, fake, 1 << 30, None) == 1
    assert "w->down is NULL" in _err(lib)
    w = _weights(abi)
    assert lib.strata_moe_ffn(fake, 8, 2, ctypes.byref(w), fake, fake, None, fake, fake, 64, None) == 3
    assert "workspace_bytes=64" in _err(lib)


@pytest.mark.parametrize(
    "fmt,side,kw,code,needle",
    [
        (0, ("gate_zero",), {}, 1, "takes no zero points"),
        (0, ("down_hi",), {}, 1, "takes no zero points or fifth-bit words"),
        (1, ("gate_zero", "up_zero"), {}, 1, "needs gate_zero, up_zero and down_zero"),
        (1, ("gate_zero", "up_zero", "down_zero", "up_hi"), {}, 1, "takes no fifth-bit words"),
        (1, ("gate_zero", "up_zero", "down_zero"), dict(I=384, g=128), 2, "even number of groups"),
        (2, ("gate_hi", "up_hi"), {}, 1, "needs gate_hi, up_hi and down_hi"),
        (2, ("gate_hi", "up_hi", "down_hi", "down_zero"), {}, 1, "takes no zero points"),
        (3, (), {}, 1, "format=3"),
        (-1, (), {}, 1, "format=-1"),
    ],
)
def test_weight_format_descriptor_is_checked(fmt, side, kw, code, needle):
    """Each weight format takes exactly its own side arrays; the asymmetric
    format's two-per-byte zero points need an even number of groups per row."""
    abi, lib = _lib()
    w = _weights(abi, **kw)
    w.format = fmt
    for name in side:
        setattr(w, name, 0x20000)
    fake = ctypes.c_void_p(0x10000)
    rc = lib.strata_moe_ffn(fake, 8, 2, ctypes.byref(w), fake, fake, None, fake, fake, 1 << 30, None)
    assert rc == code, _err(lib)
    assert needle in _err(lib)


@pytest.mark.parametrize("layout", [2, -1])
def test_weight_layout_is_checked(layout):
    abi, lib = _lib()
    w = _weights(abi)
    w.layout = layout
    fake = ctypes.c_void_p(0x10000)
    assert lib.strata_moe_ffn(fake, 8, 2, ctypes.byref(w), fake, fake, None, fake, fake, 1 << 30, None) == 1
    assert f"layout={layout}" in _err(lib)


def test_tiled_layout_passes_the_layout_check():
    # layout 1 is accepted: the call goes on to the next check (an invalid format here)
    abi, lib = _lib()
    w = _weights(abi)
    w.layout, w.format = 1, 3
    fake = ctypes.c_void_p(0x10000)
    assert lib.strata_moe_ffn(fake, 8, 2, ctypes.byref(w), fake, fake, None, fake, fake, 1 << 30, None) == 1
    assert "format=3" in _err(lib) and "layout" not in _err(lib)


@pytest.mark.parametrize(
    "src,dst,rows,K,needle",
    [
        (0x10000, 0x80000, 33, 128, "rows=33"),
        (0x10000, 0x80000, -32, 128, "rows=-32"),
        (0x10000, 0x80000, 32, 64, "K=64"),
        (0x10000, 0x80000, 32, 192, "K=192"),
        (None, 0x80000, 32, 128, "src is NULL"),
        (0x10000, None, 32, 128, "dst is NULL"),
        (0x10000, 0x80008, 32, 128, "16-byte aligned"),
        (0x10000, 0x10000 + 2032, 32, 128, "overlap"),   # 32 rows x 64 bytes = 2048 bytes
        (0x10000 + 2032, 0x10000, 32, 128, "overlap"),
    ],
)
def test_tile_weights_rejects_bad_arguments(src, dst, rows, K, needle):
    abi, lib = _lib()
    rc = lib.strata_moe_tile_weights(ctypes.c_void_p(src), ctypes.c_void_p(dst), rows, K, None)
    assert rc == 1, _err(lib)
    assert needle in _err(lib)


def test_tile_weights_of_zero_rows_enqueues_nothing():
    abi, lib = _lib()
    assert lib.strata_moe_tile_weights(None, None, 0, 128, None) == 0


def test_fifth_bit_words_must_be_word_aligned():
    abi, lib = _lib()
    w = _weights(abi)
    w.format = 2
    w.gate_hi, w.up_hi, w.down_hi = 0x20000, 0x20002, 0x20000
    fake = ctypes.c_void_p(0x10000)
    assert lib.strata_moe_ffn(fake, 8, 2, ctypes.byref(w), fake, fake, None, fake, fake, 1 << 30, None) == 1
    assert "not 4-byte aligned" in _err(lib)


def test_ffn_path_override_is_checked(monkeypatch):
    abi, lib = _lib()
    fake = ctypes.c_void_p(0x10000)
    w = _weights(abi)
    monkeypatch.setenv("STRATA_MOE_FFN_PATH", "fastest")
    assert lib.strata_moe_ffn(fake, 8, 2, ctypes.byref(w), fake, fake, None, fake, fake, 1 << 30, None) == 1
    assert "STRATA_MOE_FFN_PATH=fastest" in _err(lib)
    monkeypatch.setenv("STRATA_MOE_FFN_PATH", "gemv")  # T=64 is outside the GEMV envelope
    assert lib.strata_moe_ffn(fake, 64, 2, ctypes.byref(w), fake, fake, None, fake, fake, 1 << 30, None) == 2
    assert "gemv" in _err(lib)


def test_layer_rejects_bad_arguments_before_launch(monkeypatch):
    abi, lib = _lib()
    fake = ctypes.c_void_p(0x10000)
    w = _weights(abi)

    def call(T=4, k=2, wp=ctypes.byref(w), counts=fake, logits=fake, ws_bytes=1 << 30):
        return lib.strata_moe_layer(logits, fake, T, k, wp, fake, fake, counts, fake, fake, fake, fake, fake,
                                    ws_bytes, None)

    assert call(wp=None) == 1 and "w is NULL" in _err(lib)
    assert call(k=17) == 1 and "k=17 exceeds E=16" in _err(lib)
    assert call(T=-1) == 1 and "T=-1" in _err(lib)
    assert call(counts=None) == 1 and "counts is NULL" in _err(lib)
    assert call(logits=None) == 1 and "logits is NULL" in _err(lib)
    assert call(logits=ctypes.c_void_p(0x10004)) == 1 and "not 16-byte aligned" in _err(lib)
    assert call(ws_bytes=64) == 3 and "workspace_bytes=64" in _err(lib)
    bad = _weights(abi, g=48)
    assert call(wp=ctypes.byref(bad)) == 2 and "group=48" in _err(lib)
    assert _err(lib).startswith("strata_moe_layer")
    monkeypatch.setenv("STRATA_MOE_FFN_PATH", "fastest")
    assert call() == 1 and "STRATA_MOE_FFN_PATH=fastest" in _err(lib)
    monkeypatch.setenv("STRATA_MOE_FFN_PATH", "gemv")
    assert call(T=64) == 2 and "gemv" in _err(lib)


def test_combine_rejects_bad_h():
    _, lib = _lib()
    fake = ctypes.c_void_p(0x10000)
    assert lib.strata_moe_combine(fake, fake, fake, 4, 2, 6, fake, None) == 2
    assert "H=6" in _err(lib)


def test_binding_raises_without_library(tmp_path):
    from quantized_expert_ffn_histogram_amd import _abi

    with pytest.raises(RuntimeError, match="no CPU or PyTorch fallback"):
        _abi.load(str(tmp_path / "missing.so"))


def test_permute_workspace_query():
    _, lib = _lib()
    assert lib.strata_moe_permute_workspace_size(4, 512, 10) == 0  # 40 pairs: one workgroup, no workspace
    n = lib.strata_moe_permute_workspace_size(6144, 512, 10)
    assert n >= 60 * 512 * 4 and n % 256 == 0  # 60 segments of 1024 pairs, one histogram row each
    assert n <= lib.strata_moe_workspace_size(6144, 512, 10, 2048, 512, 64)
    assert lib.strata_moe_permute_workspace_size(4, 16, 17) == ctypes.c_size_t(-1).value
    assert "k=17 exceeds E=16" in _err(lib)


def test_noalloc_layer_checks_sizes_before_launch():
    """strata_moe_layer_noalloc refuses shapes whose workspace exceeds its
    static scratch, and bad arguments, before touching a device."""
    abi, lib = _lib()
    fake = ctypes.c_void_p(0x10000)

    def call(T, wp, k=10):
        return lib.strata_moe_layer_noalloc(fake, fake, T, k, wp, fake, fake, fake, fake, fake, fake, fake, None)

    big = _weights(abi, E=512, H=2048, I=512, g=64)
    assert call(6144, ctypes.byref(big)) == 2
    msg = _err(lib)
    need = lib.strata_moe_workspace_size(6144, 512, 10, 2048, 512, 64)
    assert msg.startswith("strata_moe_layer_noalloc") and str(need) in msg and str(64 << 20) in msg
    assert call(4, None) == 1 and "w is NULL" in _err(lib)
    assert call(4, ctypes.byref(_weights(abi, g=48)), k=2) == 2 and "group=48" in _err(lib)
    assert call(4, ctypes.byref(_weights(abi)), k=17) == 1 and "k=17 exceeds E=16" in _err(lib)


@pytest.mark.parametrize(
    "T,Hkv,D,L,code,needle",
    [
        (-1, 8, 128, 16, 1, "T=-1"),
        (4, 8, 128, 0, 1, "L=0"),
        (4, 3, 128, 16, 2, "Hkv=3"),
        (4, 8, 64, 16, 2, "D=64"),
        (1 << 27, 8, 128, 16, 2, "too large"),
    ],
)
def test_kv_quantize_pair_rejects_bad_sizes(T, Hkv, D, L, code, needle):
    _, lib = _lib()
    assert lib.strata_kv_quantize_pair(None, None, T, Hkv, D, None, None, None, None, None, L, None) == code
    assert needle in _err(lib)
    assert _err(lib).startswith("strata_kv_quantize_pair")


def test_kv_quantize_pair_rejects_null_pointers_and_accepts_zero_tokens():
    _, lib = _lib()
    p = ctypes.c_void_p(0x10000)
    assert lib.strata_kv_quantize_pair(None, p, 4, 8, 128, p, p, p, p, p, 16, None) == 1
    assert "k_bf16 is NULL" in _err(lib)
    assert lib.strata_kv_quantize_pair(p, None, 4, 8, 128, p, p, p, p, p, 16, None) == 1
    assert "v_bf16 is NULL" in _err(lib)
    assert lib.strata_kv_quantize_pair(p, p, 4, 8, 128, p, p, p, None, p, 16, None) == 1
    assert "v_codes is NULL" in _err(lib)
    assert lib.strata_kv_quantize_pair(None, None, 0, 8, 128, None, None, None, None, None, 16, None) == 0
    assert _err(lib) == ""
