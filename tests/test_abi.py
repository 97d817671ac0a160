"""The C-ABI boundary on the CPU: the libraries load, export what the headers
declare, and reject bad arguments before any HIP call (no kernel is launched)."""
import ctypes
import os
import re
import subprocess

import pytest

import flashattention_tiling_online_amd as fa
from flashattention_tiling_online_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared(header):
    text = open(os.path.join(ROOT, "include", header)).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_\w+)\s*\(", text)))


def test_fa_h_symbols_exported():
    lib = binding.lib()
    names = _declared("fa.h")
    assert names == sorted(binding.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_oracle_h_symbols_exported(oracle_lib):
    for n in _declared("fa_oracle.h"):
        assert hasattr(oracle_lib, n), n


def test_product_library_does_not_contain_oracle():
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\b(fa_\w+)\b", out))
    assert exported == set(binding.EXPORTS)
    ldd = subprocess.run(["ldd", binding.LIB_PATH], capture_output=True, text=True).stdout
    assert "oracle" not in ldd


def test_product_sources_do_not_reference_oracle():
    pkg = os.path.dirname(fa.__file__)
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle", text, re.M), f
                assert "fa_oracle" not in text, f


# fake, aligned, non-null "device" pointers: every call below must fail validation
# (or be a no-op) before the library touches HIP
P = 0x10000


def _call(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=1, Nq=8, Nk=8, d=64, causal=0, scale=0.125,
             dtype=fa.FA_DTYPE_BF16, stream=0)
    a.update(kw)
    return fa.fa_fwd_raw(**a)


@pytest.mark.parametrize("kw,want", [
    (dict(q=0), fa.FA_ERR_INVALID_ARG),
    (dict(k=0), fa.FA_ERR_INVALID_ARG),
    (dict(v=0), fa.FA_ERR_INVALID_ARG),
    (dict(o=0), fa.FA_ERR_INVALID_ARG),
    (dict(lse=0), fa.FA_ERR_INVALID_ARG),
    (dict(B=-1), fa.FA_ERR_INVALID_ARG),
    (dict(H=-2), fa.FA_ERR_INVALID_ARG),
    (dict(Nq=-1), fa.FA_ERR_INVALID_ARG),
    (dict(Nk=-1), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(d=0), fa.FA_ERR_UNSUPPORTED),
    (dict(d=256), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=7), fa.FA_ERR_INVALID_ARG),
    (dict(causal=2), fa.FA_ERR_INVALID_ARG),
    (dict(scale=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(scale=-0.5), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), fa.FA_ERR_INVALID_ARG),
    (dict(q=P + 8), fa.FA_ERR_INVALID_ARG),
    (dict(o=P + 2), fa.FA_ERR_INVALID_ARG),
    (dict(lse=P + 2), fa.FA_ERR_INVALID_ARG),
    (dict(Nk=0), fa.FA_ERR_INVALID_ARG),
    (dict(Nq=1 << 31, d=64), fa.FA_ERR_INVALID_ARG),
    (dict(Nk=(1 << 24) + 1, d=128), fa.FA_ERR_INVALID_ARG),
    (dict(B=1 << 16, H=1 << 15), fa.FA_ERR_INVALID_ARG),
    # empty problems: nothing to compute, no GPU work
    (dict(B=0), fa.FA_OK),
    (dict(H=0), fa.FA_OK),
    (dict(Nq=0), fa.FA_OK),
    (dict(Nq=0, Nk=0), fa.FA_OK),
    (dict(B=0, q=0, k=0, v=0, o=0, lse=0), fa.FA_OK),   # empty tensors may have null data
    (dict(Nq=0, q=P + 2), fa.FA_OK),
    (dict(B=0, d=80), fa.FA_ERR_UNSUPPORTED),          # still validated when empty
    (dict(Nq=0, scale=0.0), fa.FA_ERR_INVALID_ARG),
])
def test_validation_before_any_hip_call(kw, want):
    assert _call(**kw) == want


def test_status_strings_and_tiles():
    assert fa.fa_status_str(fa.FA_OK) == "FA_OK"
    assert fa.fa_status_str(fa.FA_ERR_LAUNCH) == "FA_ERR_LAUNCH"
    assert fa.fa_status_str(99) == "FA_ERR_UNKNOWN"
    for dt in (fa.FA_DTYPE_F32, fa.FA_DTYPE_F16, fa.FA_DTYPE_BF16):
        for d in (64, 128):
            assert fa.fa_tile_rows(dt, d, True) > 0
    assert fa.fa_tile_rows(fa.FA_DTYPE_BF16, 80, False) == 0
    assert fa.fa_tile_rows(5, 64, False) == 0


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(binding, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(binding, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        binding.lib()
