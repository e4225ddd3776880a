"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments on the host before any HIP call."""

import ctypes
import os
import re
import shutil
import subprocess

import pytest
import torch

from mla_decode_paged_split_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_decode.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", text)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["mla_decode_workspace_size", "mla_decode_plan", "mla_decode_run", "mla_decode_run_paged",
              "mla_decode_attend", "mla_decode_merge", "mla_decode_quantize_q", "mla_decode_quantize_q_dynamic", "mla_decode_reduce", "mla_status_string",
              "mla_decode_abi_version"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(B.library_path())
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_binding_constants_match_header():
    """Every MLA_* constant the binding restates has the header's value (macros and enumerators)."""
    text = open(HEADER).read()
    values = {}
    # macros: a number, or (N << M), with an optional u suffix
    for name, num, shift in re.findall(r"#define\s+(MLA_[A-Z0-9_]+)\s+\(?([0-9]+)u?(?:\s*<<\s*([0-9]+))?\)?", text):
        values[name] = int(num) << int(shift or 0)
    for name, value in re.findall(r"\b(MLA_[A-Z0-9_]+)\s*=\s*([0-9]+)", text):  # enumerators
        values[name] = int(value)
    checked = [name for name in B.__all__ if name in values]
    for name in checked:
        assert getattr(B, name) == values[name], name
    assert len(checked) >= 13, sorted(values)


def test_struct_layout_matches_header():
    # 13 int32 fields and one float; the plan carries params + pointer + size + 2 int32 + 3 offsets
    assert ctypes.sizeof(B.MlaDecodeParams) == 56
    assert ctypes.sizeof(B.MlaDecodePlan) == 56 + 8 + 8 + 8 + 24


def test_abi_version_and_status_strings():
    assert B.mla_decode_abi_version() == 4
    for code in range(5):
        s = B.mla_status_string(code)
        assert s.startswith("MLA_")
    assert "unknown" in B.mla_status_string(99)


def _params(**kw):
    base = dict(batch=4, q_dtype="bf16", kv_dtype="fp8", num_units=256)
    base.update(kw)
    return B.make_params(**base)


def test_workspace_size_is_host_arithmetic():
    p = _params(batch=64, num_units=256)
    n = B.mla_decode_workspace_size(p)
    # counters (64 int32 + 8 int32 of split record, padded to 256 B), then the partial slots: two per
    # share (2*256) and, with 256 shares for 64 sequences, 256/64 = 4 per sequence (64*4); partial O
    # 16*512 fp32 and partial lse 16 fp32 per slot
    slots = 2 * 256 + 64 * 4
    assert n == 512 + slots * 16 * 512 * 4 + slots * 16 * 4
    # fewer than two shares per sequence: no per-sequence slots
    assert B.mla_decode_workspace_size(_params(batch=1000, num_units=4)) == 4096 + 2 * 4 * 16 * 512 * 4 + 512
    # 8 per sequence with 8 shares per sequence; 16 at most (64 shares per sequence)
    assert B.mla_decode_workspace_size(_params(batch=32, num_units=256)) == \
        256 + (512 + 32 * 8) * 16 * 512 * 4 + (512 + 32 * 8) * 16 * 4
    assert B.mla_decode_workspace_size(_params(batch=4, num_units=256)) == \
        256 + (512 + 4 * 16) * 16 * 512 * 4 + (512 + 4 * 16) * 16 * 4
    # with several query tokens every partial slot has a row per token
    assert B.mla_decode_workspace_size(_params(batch=64, total_q=128, num_units=256, max_q_len=2)) == \
        512 + 2 * slots * 16 * 512 * 4 + 2 * slots * 16 * 4


@pytest.mark.parametrize(
    "kw,code",
    [
        (dict(batch=0), B.MLA_ERR_INVALID_ARG),
        (dict(total_q=0), B.MLA_ERR_INVALID_ARG),
        (dict(num_units=-1), B.MLA_ERR_INVALID_ARG),
        (dict(min_chunk=33), B.MLA_ERR_INVALID_ARG),
        (dict(min_chunk=-32), B.MLA_ERR_INVALID_ARG),
        (dict(flags=8), B.MLA_ERR_INVALID_ARG),
        (dict(q_dtype="fp8", flags=B.MLA_FLAG_FUSED_Q_CAST | 8), B.MLA_ERR_INVALID_ARG),
        (dict(q_dtype=7), B.MLA_ERR_INVALID_ARG),
        (dict(num_heads=8), B.MLA_ERR_UNSUPPORTED),
        (dict(num_kv_heads=2), B.MLA_ERR_UNSUPPORTED),
        (dict(qk_dim=512, v_dim=512), B.MLA_ERR_UNSUPPORTED),
        (dict(v_dim=128), B.MLA_ERR_UNSUPPORTED),
        (dict(page_size=0), B.MLA_ERR_INVALID_ARG),
        (dict(page_size=12), B.MLA_ERR_UNSUPPORTED),
        (dict(page_size=2048), B.MLA_ERR_UNSUPPORTED),
        (dict(total_q=8), B.MLA_ERR_INVALID_ARG),  # more query rows than batch * max_q_len
        (dict(total_q=3), B.MLA_ERR_INVALID_ARG),  # fewer than one per sequence
        (dict(total_q=65, max_q_len=16), B.MLA_ERR_INVALID_ARG),
        (dict(max_q_len=-1), B.MLA_ERR_INVALID_ARG),
        (dict(max_q_len=17, total_q=8), B.MLA_ERR_UNSUPPORTED),
        (dict(logit_cap=-1.0), B.MLA_ERR_INVALID_ARG),
        (dict(logit_cap=float("nan")), B.MLA_ERR_INVALID_ARG),
        (dict(logit_cap=float("inf")), B.MLA_ERR_INVALID_ARG),
        (dict(q_dtype="fp8", kv_dtype="bf16"), B.MLA_ERR_UNSUPPORTED),
        (dict(flags=B.MLA_FLAG_FUSED_Q_CAST), B.MLA_ERR_INVALID_ARG),  # needs fp8 q_dtype
        (dict(flags=16), B.MLA_ERR_INVALID_ARG),
    ],
)
def test_plan_rejects_bad_params_before_any_hip_call(kw, code):
    """Every rejection happens on the host: no device is needed to see it."""
    p = _params(**kw)
    plan = B.MlaDecodePlan()
    got = B.lib().mla_decode_plan(ctypes.byref(p), 4096, 1 << 30, None, ctypes.byref(plan))
    assert got == code
    assert B.mla_decode_workspace_size(p) == 0


def test_plan_workspace_checks():
    p = _params()
    plan = B.MlaDecodePlan()
    L = B.lib()
    assert L.mla_decode_plan(ctypes.byref(p), None, 1 << 30, None, ctypes.byref(plan)) == B.MLA_ERR_WORKSPACE
    assert L.mla_decode_plan(ctypes.byref(p), 4096 + 8, 1 << 30, None, ctypes.byref(plan)) == B.MLA_ERR_WORKSPACE
    assert L.mla_decode_plan(ctypes.byref(p), 4096, 100, None, ctypes.byref(plan)) == B.MLA_ERR_WORKSPACE
    assert L.mla_decode_plan(ctypes.byref(p), 4096, 1 << 30, None, None) == B.MLA_ERR_INVALID_ARG


def _fake_plan(**kw):
    p = _params(**kw)
    plan = B.MlaDecodePlan()
    plan.params = p
    plan.params.min_chunk = 256
    plan.workspace = 4096
    plan.workspace_bytes = B.mla_decode_workspace_size(_params())
    return plan


def test_run_rejects_bad_arguments_before_any_hip_call():
    L = B.lib()
    plan = _fake_plan()
    ptrs = [4096] * 5
    ok_scale = 8192

    def run(pl, q=4096, kv=4096, qo=4096, kvp=4096, idx=4096, qs=None, ks=ok_scale, sm=1 / 24, out=4096):
        return L.mla_decode_run(ctypes.byref(pl) if pl is not None else None, q, kv, qo, kvp, idx, qs, ks, sm, out,
                                None)

    assert run(None) == B.MLA_ERR_INVALID_ARG
    assert run(plan, q=None) == B.MLA_ERR_INVALID_ARG
    assert run(plan, kv=None) == B.MLA_ERR_INVALID_ARG
    assert run(plan, idx=None) == B.MLA_ERR_INVALID_ARG
    assert run(plan, out=None) == B.MLA_ERR_INVALID_ARG
    assert run(plan, ks=None) == B.MLA_ERR_INVALID_ARG  # fp8 KV needs its scale
    assert run(plan, sm=float("nan")) == B.MLA_ERR_INVALID_ARG
    assert run(plan, sm=float("inf")) == B.MLA_ERR_INVALID_ARG
    a8 = _fake_plan(q_dtype="fp8")
    assert run(a8) == B.MLA_ERR_INVALID_ARG  # fp8 Q needs its scale
    small = _fake_plan()
    small.workspace_bytes = 100
    assert run(small) == B.MLA_ERR_WORKSPACE
    nows = _fake_plan()
    nows.workspace = None
    assert run(nows) == B.MLA_ERR_WORKSPACE
    bad = _fake_plan(num_heads=32)
    assert run(bad) == B.MLA_ERR_UNSUPPORTED
    unresolved = _fake_plan()
    unresolved.params.min_chunk = 0
    assert run(unresolved) == B.MLA_ERR_INVALID_ARG
    # the two halves check the same things before any HIP call
    assert L.mla_decode_attend(ctypes.byref(plan), None, 4096, 4096, 4096, 4096, None, None, ok_scale, 1 / 24,
                               4096, None, None) == B.MLA_ERR_INVALID_ARG
    assert L.mla_decode_merge(ctypes.byref(plan), 4096, None, 4096, None, None) == B.MLA_ERR_INVALID_ARG
    assert L.mla_decode_merge(None, 4096, 4096, 4096, None, None) == B.MLA_ERR_INVALID_ARG
    assert L.mla_decode_merge(ctypes.byref(small), 4096, 4096, 4096, None, None) == B.MLA_ERR_WORKSPACE
    del ptrs


def test_misaligned_pointers_are_rejected_before_any_launch():
    # q, kv and out move in 16-byte pieces; indices, scales and lse_out are 4-byte words
    L = B.lib()
    plan = _fake_plan()
    sc = 8192

    def attend(q=4096, kv=4096, qo=4096, kvp=4096, idx=4096, last=None, qs=None, ks=sc, out=4096, lse=None):
        return L.mla_decode_attend(ctypes.byref(plan), q, kv, qo, kvp, idx, last, qs, ks, 1 / 24, out, lse, None)

    assert attend(q=4096 + 8) == B.MLA_ERR_INVALID_ARG
    assert attend(kv=4096 + 4) == B.MLA_ERR_INVALID_ARG
    assert attend(out=4096 + 2) == B.MLA_ERR_INVALID_ARG
    assert attend(idx=4096 + 2) == B.MLA_ERR_INVALID_ARG
    assert attend(qo=4096 + 1) == B.MLA_ERR_INVALID_ARG
    assert attend(kvp=4096 + 3) == B.MLA_ERR_INVALID_ARG
    assert attend(last=4096 + 2) == B.MLA_ERR_INVALID_ARG
    assert attend(ks=sc + 1) == B.MLA_ERR_INVALID_ARG
    assert attend(lse=8192 + 2) == B.MLA_ERR_INVALID_ARG
    assert L.mla_decode_merge(ctypes.byref(plan), 4096, 4096, 4096 + 8, None, None) == B.MLA_ERR_INVALID_ARG
    assert L.mla_decode_merge(ctypes.byref(plan), 4096, 4096, 4096, 8192 + 1, None) == B.MLA_ERR_INVALID_ARG
    R = L.mla_decode_reduce
    assert R(4096 + 4, 4096, 4096, 2, 4096, None, None) == B.MLA_ERR_INVALID_ARG  # part_o
    assert R(4096, 4096 + 2, 4096, 2, 4096, None, None) == B.MLA_ERR_INVALID_ARG  # part_lse
    assert R(4096, 4096, 4096 + 2, 2, 4096, None, None) == B.MLA_ERR_INVALID_ARG  # part_indptr
    assert R(4096, 4096, 4096, 2, 4096 + 8, None, None) == B.MLA_ERR_INVALID_ARG  # out
    assert R(4096, 4096, 4096, 2, 4096, 8192 + 2, None) == B.MLA_ERR_INVALID_ARG  # lse_out


def test_quantize_and_reduce_argument_checks():
    L = B.lib()
    assert L.mla_decode_quantize_q(4096, 1 << 20, -1, None) == B.MLA_ERR_INVALID_ARG
    assert L.mla_decode_quantize_q(None, None, 0, None) == B.MLA_OK  # nothing to do, nothing enqueued
    assert L.mla_decode_quantize_q(None, 4096, 10, None) == B.MLA_ERR_INVALID_ARG
    # overlapping source and destination
    assert L.mla_decode_quantize_q(4096, 4100, 10, None) == B.MLA_ERR_INVALID_ARG
    D = L.mla_decode_quantize_q_dynamic
    assert D(4096, 1 << 20, 8192, 1 << 24, 1024, -1, None) == B.MLA_ERR_INVALID_ARG  # negative size
    assert D(4096, 1 << 20, None, 1 << 24, 1024, 10, None) == B.MLA_ERR_INVALID_ARG  # no q_scale
    assert D(4096, 1 << 20, 8192, None, 1024, 10, None) == B.MLA_ERR_WORKSPACE  # no scratch
    assert D(4096, 1 << 20, 8192, 1 << 24, 1023, 10, None) == B.MLA_ERR_WORKSPACE  # scratch too small
    assert D(4096, 1 << 20, 8192, (1 << 24) + 2, 1024, 10, None) == B.MLA_ERR_WORKSPACE  # misaligned
    assert D(None, 1 << 20, 8192, 1 << 24, 1024, 10, None) == B.MLA_ERR_INVALID_ARG
    assert D(4096, 4100, 8192, 1 << 24, 1024, 10, None) == B.MLA_ERR_INVALID_ARG  # q overlaps its output
    assert D(4096, 1 << 20, 8192, (1 << 20) + 4, 1024, 10, None) == B.MLA_ERR_INVALID_ARG  # scratch overlaps
    assert L.mla_decode_reduce(4096, 4096, 4096, 0, 4096, None, None) == B.MLA_ERR_INVALID_ARG
    assert L.mla_decode_reduce(None, 4096, 4096, 2, 4096, None, None) == B.MLA_ERR_INVALID_ARG
    assert L.mla_decode_reduce(4096, 4096, None, 2, 4096, None, None) == B.MLA_ERR_INVALID_ARG


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device path")
def test_auto_units_without_a_device_reports_hip_error():
    p = _params(num_units=0)
    assert B.mla_decode_workspace_size(p) == 0
    plan = B.MlaDecodePlan()
    assert B.lib().mla_decode_plan(ctypes.byref(p), 4096, 1 << 30, None, ctypes.byref(plan)) == B.MLA_ERR_HIP


def test_binding_has_no_cpu_fallback():
    # the product path refuses host tensors instead of computing on the CPU
    with pytest.raises(ValueError):
        B._ptr(torch.zeros(4))


@pytest.mark.parametrize("kw", [dict(page_size=16), dict(page_size=1024), dict(max_q_len=4, total_q=13),
                                dict(flags=B.MLA_FLAG_CAUSAL, max_q_len=2, total_q=8), dict(logit_cap=30.0)])
def test_widened_params_pass_host_validation(kw):
    # accepted shapes get a workspace size with explicit units (no device query needed)
    assert B.mla_decode_workspace_size(_params(**kw)) > 0


def test_abi_from_plain_c(tmp_path):
    """The header and library serve a plain C99 program (gcc, no HIP compiler, no Python): version, status
    strings, workspace sizing and host-side rejections, all without a device."""
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    libdir = os.path.dirname(B.library_path())
    exe = str(tmp_path / "abi_from_c")
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(root, "include"),
           "-I", "/opt/rocm/include", os.path.join(root, "tests", "c", "abi_from_c.c"), "-L", libdir, "-lmla_decode",
           f"-Wl,-rpath,{libdir}", "-L", "/opt/rocm/lib", "-lamdhip64", "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    res = subprocess.run([exe], capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.count("ok  ") == 10, res.stdout
