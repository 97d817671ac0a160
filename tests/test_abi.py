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


def _split(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=1, Nq=8, Nk=1024, d=64, causal=0, scale=0.125,
             dtype=fa.FA_DTYPE_BF16, n_splits=4, workspace=P, workspace_bytes=1 << 30, stream=0)
    a.update(kw)
    return fa.fa_fwd_split_raw(**a)


@pytest.mark.parametrize("kw,want", [
    (dict(n_splits=0), fa.FA_ERR_INVALID_ARG),
    (dict(n_splits=257), fa.FA_ERR_INVALID_ARG),
    (dict(n_splits=-3), fa.FA_ERR_INVALID_ARG),
    (dict(workspace=0), fa.FA_ERR_INVALID_ARG),
    (dict(workspace=P + 8), fa.FA_ERR_INVALID_ARG),
    (dict(workspace_bytes=100), fa.FA_ERR_INVALID_ARG),
    (dict(q=0), fa.FA_ERR_INVALID_ARG),
    (dict(lse=P + 2), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=9), fa.FA_ERR_INVALID_ARG),
    (dict(causal=3), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(Nk=0), fa.FA_ERR_INVALID_ARG),
    (dict(Nq=0), fa.FA_OK),
    (dict(B=0, q=0, k=0, v=0, o=0, lse=0, workspace=0), fa.FA_OK),
])
def test_split_validation_before_any_hip_call(kw, want):
    assert _split(**kw) == want


def _merge(**kw):
    a = dict(o_parts=P, lse_parts=P, n_parts=3, B=1, H=2, Nq=8, d=128, o=P, lse=P,
             dtype=fa.FA_DTYPE_BF16, stream=0)
    a.update(kw)
    return fa.fa_merge_raw(**a)


@pytest.mark.parametrize("kw,want", [
    (dict(n_parts=0), fa.FA_ERR_INVALID_ARG),
    (dict(B=-1), fa.FA_ERR_INVALID_ARG),
    (dict(d=80), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=4), fa.FA_ERR_INVALID_ARG),
    (dict(o_parts=0), fa.FA_ERR_INVALID_ARG),
    (dict(lse_parts=0), fa.FA_ERR_INVALID_ARG),
    (dict(o=0), fa.FA_ERR_INVALID_ARG),
    (dict(lse=0), fa.FA_ERR_INVALID_ARG),
    (dict(o_parts=P + 4), fa.FA_ERR_INVALID_ARG),
    (dict(o=P + 2), fa.FA_ERR_INVALID_ARG),
    (dict(lse_parts=P + 1), fa.FA_ERR_INVALID_ARG),
    (dict(Nq=0, o_parts=0, lse_parts=0, o=0, lse=0), fa.FA_OK),
])
def test_merge_validation_before_any_hip_call(kw, want):
    assert _merge(**kw) == want


def _bwd(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, dout=P, dq=P, dk=P, dv=P, B=1, H=2, Nq=64, Nk=64, d=128,
             causal=0, scale=0.1, dtype=fa.FA_DTYPE_BF16, workspace=P, workspace_bytes=1 << 20,
             stream=0)
    a.update(kw)
    return fa.fa_bwd_raw(**a)


@pytest.mark.parametrize("kw,want", [
    (dict(dtype=fa.FA_DTYPE_F32), fa.FA_ERR_UNSUPPORTED),
    (dict(d=80), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=5), fa.FA_ERR_INVALID_ARG),
    (dict(causal=-1), fa.FA_ERR_INVALID_ARG),
    (dict(scale=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(B=-1), fa.FA_ERR_INVALID_ARG),
    (dict(Nk=0), fa.FA_ERR_INVALID_ARG),
    (dict(q=0), fa.FA_ERR_INVALID_ARG),
    (dict(o=0), fa.FA_ERR_INVALID_ARG),
    (dict(lse=0), fa.FA_ERR_INVALID_ARG),
    (dict(dout=0), fa.FA_ERR_INVALID_ARG),
    (dict(dq=0), fa.FA_ERR_INVALID_ARG),
    (dict(dk=0), fa.FA_ERR_INVALID_ARG),
    (dict(dv=0), fa.FA_ERR_INVALID_ARG),
    (dict(dv=P + 8), fa.FA_ERR_INVALID_ARG),
    (dict(lse=P + 1), fa.FA_ERR_INVALID_ARG),
    (dict(workspace=0), fa.FA_ERR_INVALID_ARG),
    (dict(workspace=P + 4), fa.FA_ERR_INVALID_ARG),
    (dict(workspace_bytes=256), fa.FA_ERR_INVALID_ARG),
    (dict(Nq=1 << 31), fa.FA_ERR_INVALID_ARG),
    (dict(B=0), fa.FA_OK),
    (dict(Nq=0, Nk=0, k=0, v=0, dk=0, dv=0), fa.FA_OK),
])
def test_bwd_validation_before_any_hip_call(kw, want):
    assert _bwd(**kw) == want


def _fwd_drop(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=1, Nq=8, Nk=8, d=64, causal=0, scale=0.125,
             p_drop=0.1, seed=1, dtype=fa.FA_DTYPE_BF16, stream=0)
    a.update(kw)
    return fa.fa_fwd_dropout_raw(**a)


def _bwd_drop(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, dout=P, dq=P, dk=P, dv=P, B=1, H=2, Nq=64, Nk=64, d=128,
             causal=0, scale=0.1, p_drop=0.1, seed=1, dtype=fa.FA_DTYPE_BF16, workspace=P,
             workspace_bytes=1 << 20, stream=0)
    a.update(kw)
    return fa.fa_bwd_dropout_raw(**a)


@pytest.mark.parametrize("kw,want", [
    (dict(p_drop=1.0), fa.FA_ERR_INVALID_ARG),
    (dict(p_drop=-0.01), fa.FA_ERR_INVALID_ARG),
    (dict(p_drop=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(p_drop=0.999), fa.FA_ERR_INVALID_ARG),          # rounds to t = 256
    (dict(dtype=fa.FA_DTYPE_F32), fa.FA_ERR_UNSUPPORTED),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(q=0), fa.FA_ERR_INVALID_ARG),
    (dict(scale=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(Nk=0), fa.FA_ERR_INVALID_ARG),
    (dict(B=0), fa.FA_OK),
    (dict(Nq=0, p_drop=0.5, seed=(1 << 64) - 1), fa.FA_OK),
])
def test_dropout_validation_before_any_hip_call(kw, want):
    assert _fwd_drop(**kw) == want
    bkw = {k: v for k, v in kw.items() if k != "Nq"}
    if "Nq" in kw:  # no queries: the backward writes zero key gradients (a GPU call)
        bkw["B"] = 0
    assert _bwd_drop(**bkw) == want


def test_bwd_workspace_size():
    assert fa.fa_bwd_workspace(2, 8, 1024, 64) == 2 * 8 * 1024 * 4
    assert fa.fa_bwd_workspace(1, 1, 3, 128) == 256
    assert fa.fa_bwd_workspace(1, 1, 0, 64) == 0
    assert fa.fa_bwd_workspace(1, 1, 8, 96) == -1
    assert fa.fa_bwd_workspace(-1, 1, 8, 64) == -1


def test_split_workspace_size():
    # n_splits * rows * d fp32 partial outputs, padded to 256 B, then n_splits * rows fp32 L
    rows = 2 * 8 * 1024
    assert fa.fa_fwd_split_workspace(2, 8, 1024, 64, 4) == 4 * rows * 64 * 4 + 4 * rows * 4
    assert fa.fa_fwd_split_workspace(1, 1, 3, 128, 2) == 3072 + 24
    assert fa.fa_fwd_split_workspace(1, 1, 0, 128, 2) == 0
    for bad in [(-1, 1, 1, 64, 2), (1, 1, 1, 80, 2), (1, 1, 1, 64, 0), (1, 1, 1, 64, 257)]:
        assert fa.fa_fwd_split_workspace(*bad) == -1


def test_split_hint():
    bf16, f32 = fa.FA_DTYPE_BF16, fa.FA_DTYPE_F32
    # 2x8 heads x 8 query tiles of 128 rows = 128 workgroups, 2 per CU: 4 would fill the
    # GPU, but 16 key tiles keep at most 2 ranges of 8 tiles
    assert fa.fa_split_hint(2, 8, 1024, 1024, 64, 0, bf16) == 2
    # 512 workgroups of 256 rows already fill the GPU
    assert fa.fa_split_hint(1, 16, 8192, 8192, 128, 1, bf16) == 1
    # fp32: 2 workgroups, 4 key tiles, two tiles per range
    assert fa.fa_split_hint(1, 1, 256, 256, 64, 0, f32) == 2
    # short queries, long keys: 32 workgroups -> 8 ranges of 32 tiles
    assert fa.fa_split_hint(4, 8, 256, 16384, 128, 0, bf16) == 8
    assert fa.fa_split_hint(1, 1, 1, 1 << 20, 128, 0, bf16) == 16
    assert fa.fa_split_hint(1, 1, 8, 64, 64, 0, bf16) == 1
    assert fa.fa_split_hint(0, 1, 8, 64, 64, 0, bf16) == 0
    assert fa.fa_split_hint(1, 1, 8, 64, 96, 0, bf16) == 0


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


def _split_static(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=2, Nq=64, Nk=640, d=128, causal=0, scale=0.125,
             dtype=fa.FA_DTYPE_BF16, n_splits=4, stream=0)
    a.update(kw)
    return fa.fa_fwd_split_static_raw(**a)


@pytest.mark.parametrize("kw,want", [
    (dict(n_splits=0), fa.FA_ERR_INVALID_ARG),
    (dict(n_splits=257), fa.FA_ERR_INVALID_ARG),
    (dict(q=0), fa.FA_ERR_INVALID_ARG),
    (dict(o=P + 8), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(Nk=0), fa.FA_ERR_INVALID_ARG),
    (dict(Nq=0), fa.FA_OK),
    # partials of 64 x 16 x 4096 rows x 128 x 4 B x 2 ranges = 1 GiB: beyond the array
    (dict(B=64, H=16, Nq=4096, Nk=128, n_splits=2), fa.FA_ERR_SCRATCH),
])
def test_split_static_validation_before_any_hip_call(kw, want):
    assert _split_static(**kw) == want


def test_split_static_limit_matches_header():
    text = open(os.path.join(ROOT, "include", "fa.h")).read()
    m = re.search(r"#define FA_STATIC_SCRATCH_BYTES \((\d+)LL << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == fa.FA_STATIC_SCRATCH_BYTES
    assert fa.fa_status_str(fa.FA_ERR_SCRATCH) == "FA_ERR_SCRATCH"


def _masked(**kw):
    a = dict(q=P, k=P, v=P, mask=P, mask_b=1, mask_h=1, o=P, lse=P, B=2, H=3, Nq=64, Nk=100,
             d=128, causal=0, scale=0.125, dtype=fa.FA_DTYPE_BF16, stream=0)
    a.update(kw)
    return fa.fa_fwd_masked_raw(**a)


@pytest.mark.parametrize("kw,want", [
    (dict(mask=0), fa.FA_ERR_INVALID_ARG),
    (dict(mask=P + 2), fa.FA_ERR_INVALID_ARG),
    (dict(mask_b=0), fa.FA_ERR_INVALID_ARG),
    (dict(mask_b=3), fa.FA_ERR_INVALID_ARG),
    (dict(mask_h=2), fa.FA_ERR_INVALID_ARG),
    (dict(mask_h=4), fa.FA_ERR_INVALID_ARG),
    (dict(q=0), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(causal=2), fa.FA_ERR_INVALID_ARG),
    (dict(Nk=0), fa.FA_ERR_INVALID_ARG),
    (dict(Nq=0), fa.FA_OK),
    (dict(B=0, q=0, k=0, v=0, o=0, lse=0, mask=0), fa.FA_OK),
])
def test_masked_validation_before_any_hip_call(kw, want):
    assert _masked(**kw) == want
