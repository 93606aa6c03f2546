"""Host-side checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects bad arguments before touching a device."""
import ctypes
import os
import re

import pytest

import transformer_block_fwd_amd as tb
from transformer_block_fwd_amd import _abi
from workload import CONFIGS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pblock.h")


@pytest.fixture(scope="module", autouse=True)
def built_library():
    if not os.path.exists(_abi.LIB_PATH):
        from transformer_block_fwd_amd.build import build

        build(verbose=False)
    return _abi.lib()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pblock_\w+)\s*\(", text)))


def test_header_symbols_exported():
    names = header_functions()
    assert len(names) >= 12, names
    lib = ctypes.CDLL(_abi.LIB_PATH)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    # the binding declares every one of them too
    assert set(names) <= set(_abi._SIGNATURES), set(names) - set(_abi._SIGNATURES)


def test_binding_names_match_abi():
    for n in header_functions():
        assert hasattr(tb, n), n
    # and lists them among its public names
    assert set(header_functions()) <= set(tb.__all__), set(header_functions()) - set(tb.__all__)


def test_validate_accepts_all_workloads():
    for name, cfg in CONFIGS.items():
        assert tb.pblock_validate_cfg(cfg) == 0, name


@pytest.mark.parametrize("field,value,code", [
    ("B", 0, _abi.PBLOCK_ERR_SHAPE), ("S", 0, _abi.PBLOCK_ERR_SHAPE), ("W", 0, _abi.PBLOCK_ERR_SHAPE),
    ("hd", 96, _abi.PBLOCK_ERR_SHAPE), ("hd", 32, _abi.PBLOCK_ERR_SHAPE), ("H", 0, _abi.PBLOCK_ERR_SHAPE),
    ("d", 100, _abi.PBLOCK_ERR_SHAPE), ("d", 65536, _abi.PBLOCK_ERR_SHAPE), ("ffn", 96, _abi.PBLOCK_ERR_SHAPE),
    ("ffn", 0, _abi.PBLOCK_ERR_SHAPE), ("dtype", 7, _abi.PBLOCK_ERR_DTYPE),
    ("add_residual", 2, _abi.PBLOCK_ERR_ARG), ("ln_eps", 0.0, _abi.PBLOCK_ERR_ARG),
    ("ln_eps", float("nan"), _abi.PBLOCK_ERR_ARG), ("ln_eps", -1e-5, _abi.PBLOCK_ERR_ARG),
])
def test_validate_rejects(field, value, code):
    c = tb.as_cfg(CONFIGS["small"])
    setattr(c, field, value)
    assert tb.pblock_validate_cfg(c) == code
    assert _abi.last_error() != ""


def test_validate_rejects_too_many_tokens():
    c = tb.as_cfg(CONFIGS["small"])
    c.B, c.S = 1 << 13, 1 << 12  # 2^25 tokens
    assert tb.pblock_validate_cfg(c) == _abi.PBLOCK_ERR_SHAPE


def test_workspace_and_flops():
    for cfg in CONFIGS.values():
        es = 2 if cfg.dtype == "bf16" else 4
        ws = tb.pblock_workspace_bytes(cfg)
        mt = -(-cfg.M // 256) * 256 + 256  # GEMM row operands u, AG: whole 256-row tiles plus one
        need = es * (mt * cfg.d + cfg.M * 3 * cfg.A + mt * cfg.k_out)
        need += cfg.M * cfg.hd * 4  # rotary table: fp32 (cos, sin) for hd/2 pairs at M positions
        slack = 6 * 256
        if cfg.dtype == "bf16":
            # GEMM scratch (host estimate at 256 CUs): one fp32 256x256 partial tile per CU
            need += 256 * 256 * 256 * 4
        assert need <= ws <= need + slack
        assert tb.pblock_flops(cfg) == pytest.approx(cfg.flops(), rel=1e-12)
    bad = tb.as_cfg(CONFIGS["small"])
    bad.hd = 3
    assert tb.pblock_flops(bad) < 0
    with pytest.raises(tb.PblockError):
        tb.pblock_workspace_bytes(bad)


def test_strerror_covers_codes():
    for code in list(_abi.STATUS_NAMES) + [-99]:
        assert isinstance(tb.pblock_strerror(code), str) and tb.pblock_strerror(code)


def test_null_arguments():
    lib = _abi.lib()
    assert lib.pblock_create(None, None) == _abi.PBLOCK_ERR_NULL
    h = ctypes.c_void_p()
    assert lib.pblock_create(None, ctypes.byref(h)) == _abi.PBLOCK_ERR_NULL
    c = tb.as_cfg(CONFIGS["tiny"])
    w = tb.PblockWeights(16, 16, 16, 16)
    assert lib.pblock_forward(None, 16, ctypes.byref(w), ctypes.byref(c), 32, None) == _abi.PBLOCK_ERR_NULL
    assert lib.pblock_destroy(None) == _abi.PBLOCK_OK
    assert lib.pblock_set_timing(None, 1) == _abi.PBLOCK_ERR_NULL
    assert lib.pblock_copy_intermediates(None, None, None, None, None) == _abi.PBLOCK_ERR_NULL
    var = tb.make_variant(rope=True)
    assert lib.pblock_forward_variant(None, 16, ctypes.byref(w), None, ctypes.byref(c), ctypes.byref(var), 32,
                                      None) == _abi.PBLOCK_ERR_NULL


def test_attention_entry_rejects_before_device():
    lib = _abi.lib()
    f = lib.pblock_swa_attention
    A = 2 * 64
    ok = dict(qkv=4096, ld=3 * A, o=1 << 30, ldo=A, B=1, S=10, H=2, hd=64, W=4, dt=_abi.PBLOCK_BF16)

    def call(**kw):
        a = {**ok, **kw}
        return f(a["qkv"], a["ld"], a["o"], a["ldo"], a["B"], a["S"], a["H"], a["hd"], a["W"], a["dt"], None)

    assert call(qkv=0) == _abi.PBLOCK_ERR_NULL
    assert call(dt=5) == _abi.PBLOCK_ERR_DTYPE
    assert call(hd=80) == _abi.PBLOCK_ERR_SHAPE
    assert call(W=0) == _abi.PBLOCK_ERR_SHAPE
    assert call(ld=3 * A - 8) == _abi.PBLOCK_ERR_SHAPE
    assert call(ldo=A + 4) == _abi.PBLOCK_ERR_SHAPE
    assert call(qkv=4096 + 8) == _abi.PBLOCK_ERR_ALIGN
    assert call(o=4096 + 64) == _abi.PBLOCK_ERR_ALIAS


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="checks the no-device path")
def test_create_without_device():
    with pytest.raises(tb.PblockError) as ei:
        tb.pblock_create(CONFIGS["tiny"])
    assert ei.value.code == _abi.PBLOCK_ERR_DEVICE


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(_abi, "_lib", None)
    monkeypatch.setattr(_abi, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(RuntimeError, match="not found"):
        tb.pblock_validate_cfg(CONFIGS["tiny"])


def test_train_workspace_bytes():
    """The training workspace is sized on the host: bf16 only, d <= 16384, and at least the saved
    activations (u, q|k|v, [attention | GeLU], FC1 pre-activation) plus dy, dO, dz (bf16) and du
    (fp32); the weights are read in place, so it does not grow with them."""
    for name, cfg in CONFIGS.items():
        if cfg.dtype != "bf16":
            with pytest.raises(tb.PblockError) as ei:
                tb.pblock_train_workspace_bytes(cfg)
            assert ei.value.code == _abi.PBLOCK_ERR_DTYPE
            continue
        n = tb.pblock_train_workspace_bytes(cfg)
        saved = 2 * cfg.M * (cfg.d + 3 * cfg.A + cfg.k_out + cfg.ffn)
        scratch = 2 * cfg.M * (cfg.d + cfg.A + cfg.n_in) + 4 * cfg.M * cfg.d
        assert saved + scratch <= n < saved + scratch + 2 * cfg.d * cfg.n_in, name
    big = tb.as_cfg(CONFIGS["small"])
    big.d = 16384 + 64
    assert _abi.lib().pblock_train_workspace_bytes(ctypes.byref(big)) == _abi.PBLOCK_ERR_SHAPE
