"""C-ABI library: loads, exports every declared entry point, and rejects bad arguments
before touching the GPU (CPU only: no compute call is made here)."""

import ctypes
import os
import subprocess

import pytest

from compressive_memory_transformer_segment_amd import binding

EXPECTED = {
    "infini_attn_create", "infini_attn_forward_segment", "infini_attn_forward_stream",
    "infini_attn_forward_stream_ex", "infini_attn_forward_stream_local", "infini_attn_reset_state",
    "infini_attn_get_state",
    "infini_attn_set_state", "infini_attn_set_beta", "infini_attn_device_bytes",
    "infini_attn_window_tokens", "infini_attn_destroy", "infini_attn_status_string",
    "infini_attn_profile_enable", "infini_attn_profile_read",
    "infini_attn_project_qkv", "infini_attn_project_out", "infini_attn_forward_layer",
    "infini_attn_decode_step", "infini_attn_decode_flush", "infini_attn_decode_position",
    "infini_attn_backward", "infini_attn_forward_stream_noalloc",
}


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from compressive_memory_transformer_segment_amd import build
        build.build(verbose=False)
    return binding.load()


def test_header_declares_the_expected_entry_points():
    assert set(binding.exported_names()) == EXPECTED


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(binding.LIB_PATH)
    for name in binding.exported_names():
        assert hasattr(raw, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True, text=True)
    exported = {line.split()[-1] for line in out.stdout.splitlines() if " T " in line}
    assert EXPECTED <= exported
    # only the C-ABI is exported from the library's own code
    assert not [s for s in exported if s.startswith("_ZN6infini")]


def test_status_strings(lib):
    assert binding.status_string(0) == "ok"
    assert binding.status_string(-1) == "invalid argument"
    assert binding.status_string(-2) == "unsupported configuration"
    assert binding.status_string(-3) == "HIP runtime error"
    assert binding.status_string(-4) == "out of device memory"
    assert "static scratch" in binding.status_string(-5)
    assert binding.status_string(12345) == "unknown status"


def _cfg(**kw):
    base = dict(batch=1, heads=2, head_dim=128, segment_len=256, update=0, io_dtype=0, eps=1e-6,
                softmax_scale=0.0, max_window_segments=0)
    base.update(kw)
    return binding.Config(*[base[f] for f, _ in binding.Config._fields_])


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), -1), (dict(heads=0), -1), (dict(segment_len=0), -1), (dict(update=2), -1),
    (dict(io_dtype=5), -1), (dict(eps=-1.0), -1), (dict(eps=float("nan")), -1),
    (dict(softmax_scale=float("inf")), -1), (dict(head_dim=96), -2), (dict(head_dim=256), -2),
    # one segment's fp32 rows must stay inside a 32-bit buffer range
    (dict(segment_len=(1 << 22) + 1), -2), (dict(batch=1 << 11, heads=1 << 10), -2),
])
def test_create_rejects_bad_configs_without_a_gpu(lib, kw, status):
    h = ctypes.c_void_p()
    beta = (ctypes.c_float * 2)(0.0, 0.0)
    assert lib.infini_attn_create(ctypes.byref(_cfg(**kw)), beta, None, ctypes.byref(h)) == status
    assert not h.value


def test_calls_on_a_missing_handle_fail_cleanly(lib):
    null = ctypes.c_void_p()
    bogus = ctypes.c_void_p(0x1000)
    p = ctypes.c_void_p(0x10000)
    assert lib.infini_attn_destroy(null) == 0
    assert lib.infini_attn_destroy(bogus) == -1
    for h in (null, bogus):
        assert lib.infini_attn_forward_stream(h, p, p, p, p, 16, None) == -1
        assert lib.infini_attn_forward_segment(h, p, p, p, p, 16, None) == -1
        assert lib.infini_attn_forward_stream_ex(h, p, p, p, p, None, None, 16, None) == -1
        assert lib.infini_attn_forward_stream_local(h, p, p, p, None, None, p, 16, None) == -1
        assert lib.infini_attn_reset_state(h, None) == -1
        assert lib.infini_attn_get_state(h, p, p, None) == -1
        assert lib.infini_attn_set_state(h, p, p, None) == -1
        assert lib.infini_attn_set_beta(h, (ctypes.c_float * 1)(0.0)) == -1
        assert lib.infini_attn_device_bytes(h) == -1
        assert lib.infini_attn_window_tokens(h) == -1
        assert lib.infini_attn_profile_enable(h, 1) == -1
        assert lib.infini_attn_profile_read(h, ctypes.byref(binding.Profile())) == -1
        assert lib.infini_attn_project_qkv(h, p, p, p, p, p, 16, 64, None) == -1
        assert lib.infini_attn_project_out(h, p, p, p, 16, 64, None) == -1
        assert lib.infini_attn_forward_layer(h, p, p, p, p, 16, 64, None) == -1
        assert lib.infini_attn_decode_step(h, p, p, p, p, None) == -1
        assert lib.infini_attn_decode_flush(h, None) == -1
        assert lib.infini_attn_decode_position(h) == -1
        assert lib.infini_attn_backward(h, p, p, p, p, None, None, None, None, p, p, p, p, None, None, 16,
                                        None) == -1
