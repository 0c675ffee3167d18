"""The C-ABI library loads and exports every function include/tfb.h declares
(CPU only: no compute call is made)."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tfb.h")
LIB = os.path.join(ROOT, "transformer_fwd_bwd_amd", "libtfb.so")


def declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(tfb_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_hot_path():
    names = declared()
    for must in ("tfb_init", "tfb_tensor_create", "tfb_matmul", "tfb_linear", "tfb_layernorm", "tfb_gelu",
                 "tfb_embedding", "tfb_causal_attention", "tfb_softmax_cross_entropy", "tfb_backward",
                 "tfb_adamw_step", "tfb_tape_reset"):
        assert must in names


@pytest.mark.skipif(not os.path.exists(LIB), reason="libtfb.so not built")
def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(tfb_\w+)$", out, flags=re.M))
    missing = [n for n in declared() if n not in exported]
    assert not missing, missing


@pytest.mark.skipif(not os.path.exists(LIB), reason="libtfb.so not built")
def test_binding_loads_and_declares_signatures():
    import transformer_fwd_bwd_amd as T
    lib = T.load_library()
    for name in declared():
        assert hasattr(lib, name), name
    assert set(T.SIGNATURES) | {"tfb_last_error"} >= set(declared()) - set(T._EXTRA_SIGNATURES)


def test_ops_fail_loudly_without_the_library(tmp_path):
    import transformer_fwd_bwd_amd as T
    with pytest.raises(RuntimeError):
        T.load_library.__wrapped__(str(tmp_path / "missing.so")) if hasattr(T.load_library, "__wrapped__") \
            else _load_fresh(str(tmp_path / "missing.so"))


def _load_fresh(path):
    import transformer_fwd_bwd_amd as T
    saved = T._lib
    T._lib = None
    try:
        return T.load_library(path)
    finally:
        T._lib = saved
