"""CPU checks of the C ABI: the library loads, exports every declared entry point,
and its host-only functions (validation, split plan, status text) behave as the
header states. Nothing here launches a kernel."""

import ctypes
import os
import re

import pytest

from exact_attention_47_amd import attn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "defined")))


def test_header_declares_the_expected_api():
    names = declared_functions()
    for n in ("attn_fwd", "attn_fwd_ex", "attn_fwd_workspace_size", "hadamard_quant",
              "quant_per_tensor", "attn_fwd_fp8", "attn_status_string", "attn_abi_version"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(attn.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert missing == []


def test_binding_signatures_cover_every_declared_symbol():
    assert sorted(attn._SIGS) == declared_functions()


def test_version_and_status_strings():
    assert attn.abi_version() == 4
    lib = attn.load()
    for code in (0, -1, -2, -3, -4, -5):
        assert lib.attn_status_string(code).decode() not in ("", "unknown status")
    assert lib.attn_status_string(-99).decode() == "unknown status"


P = 0x10000  # fake, 16-byte aligned "device" addresses: validation never dereferences them


def chk(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=2, S_q=128, S_k=128, D=128, causal=0, scale=0.125, dtype=2)
    a.update(kw)
    return attn.check_args(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["S_q"], a["S_k"],
                           a["D"], a["causal"], a["scale"], a["dtype"])


def test_validation_accepts_good_arguments():
    assert chk() == attn.OK
    for d in (64, 128, 256):
        assert chk(D=d) == attn.OK
    assert chk(dtype=0, D=64) == attn.OK
    assert chk(causal=1, S_q=100, S_k=300) == attn.OK


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), attn.ERR_INVALID_ARG),
    (dict(lse=None), attn.ERR_INVALID_ARG),
    (dict(B=0), attn.ERR_INVALID_ARG),
    (dict(S_k=-1), attn.ERR_INVALID_ARG),
    (dict(dtype=7), attn.ERR_INVALID_ARG),
    (dict(causal=2), attn.ERR_INVALID_ARG),
    (dict(scale=0.0), attn.ERR_INVALID_ARG),
    (dict(scale=float("nan")), attn.ERR_INVALID_ARG),
    (dict(scale=float("inf")), attn.ERR_INVALID_ARG),
    (dict(D=96), attn.ERR_UNSUPPORTED),
    (dict(D=32), attn.ERR_UNSUPPORTED),
    (dict(dtype=0, D=256), attn.ERR_UNSUPPORTED),
    (dict(causal=1, S_q=300, S_k=100), attn.ERR_UNSUPPORTED),
    (dict(q=P + 8), attn.ERR_MISALIGNED),
    (dict(o=P + 2), attn.ERR_MISALIGNED),
    (dict(lse=P + 2), attn.ERR_MISALIGNED),
])
def test_validation_rejects(kw, code):
    assert chk(**kw) == code


def test_split_plan():
    # the decode shape splits its 32K keys; ordinary prefill does not
    assert attn.num_splits(64, 32, 1, 32768, 128) > 1
    assert attn.num_splits(2, 16, 8192, 8192, 128) == 1
    # fewer 256-row query tiles than half the chip's CUs against 8K+ keys: a split whose partial results
    # fit attn_fwd_noalloc's scratch, none where they would not, nor for short key ranges or full grids
    for shape in ((1, 8, 1024, 65536, 128), (1, 2, 600, 9000, 128), (1, 1, 200, 8192, 256), (1, 32, 256, 32768, 64)):
        assert attn.num_splits(*shape) > 1, shape
        assert 0 < attn.workspace_size(*shape) <= attn.NOALLOC_SCRATCH_BYTES, shape
    assert attn.num_splits(1, 8, 2048, 65536, 128) == 1
    assert attn.num_splits(1, 2, 600, 8000, 128) == 1
    assert attn.num_splits(1, 16, 16384, 16384, 128) == 1
    assert attn.num_splits(2, 8, 8192, 8192, 256) == 1
    assert attn.num_splits(1, 1, 128, 128, 128, 1) == 1
    # requests are clamped to the number of key tiles (tiles hold at least 32 keys)
    # and never leave a split empty
    assert 1 <= attn.num_splits(1, 1, 4, 100, 128, 16) <= 4
    assert attn.num_splits(1, 1, 4, 4096, 128, 4) == 4
    for n_req in (2, 3, 5, 7):
        assert attn.num_splits(1, 1, 4, 1000, 128, n_req) <= n_req
    assert attn.workspace_size(1, 1, 4, 640, 128, 1) == 0
    # the float32 kernel's 32-key tile clamps a request differently from the 128-key bf16 tile
    assert attn.num_splits(1, 1, 4, 300, 128, 5, dtype=attn.F32) == 5
    assert attn.num_splits(1, 1, 4, 300, 128, 5, dtype=attn.BF16) == 3
    assert attn.num_splits(1, 1, 4, 300, 128, 5, dtype=9) == 1
    n = attn.num_splits(64, 32, 1, 32768, 128)
    assert attn.workspace_size(64, 32, 1, 32768, 128) >= n * 64 * 32 * (128 + 1) * 4


def varlen(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, cu_q=P, cu_k=P, B=2, H=2, total_q=300, total_k=400, max_q=200,
             max_k=250, D=128, causal=0, scale=0.125, dtype=2)
    a.update(kw)
    return attn.load().attn_fwd_varlen(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cu_q"], a["cu_k"], a["B"],
                                       a["H"], a["total_q"], a["total_k"], a["max_q"], a["max_k"], a["D"],
                                       a["causal"], ctypes.c_float(a["scale"]), a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(cu_q=None), attn.ERR_INVALID_ARG),
    (dict(k=None), attn.ERR_INVALID_ARG),
    (dict(B=0), attn.ERR_INVALID_ARG),
    (dict(total_q=-1), attn.ERR_INVALID_ARG),
    (dict(max_q=301), attn.ERR_INVALID_ARG),
    (dict(max_k=-2), attn.ERR_INVALID_ARG),
    (dict(dtype=9), attn.ERR_INVALID_ARG),
    (dict(causal=3), attn.ERR_INVALID_ARG),
    (dict(scale=-1.0), attn.ERR_INVALID_ARG),
    (dict(dtype=0), attn.ERR_UNSUPPORTED),
    (dict(D=192), attn.ERR_UNSUPPORTED),
    (dict(D=96), attn.ERR_UNSUPPORTED),
    # D = 256: K rows of the longest sequence span (2.1M + 32) * H * 512 bytes >= 2^31, past the
    # kernel's 32-bit buffer offsets (refused on the host before any launch)
    (dict(D=256, total_k=3_000_000, max_k=2_100_000), attn.ERR_UNSUPPORTED),
    (dict(q=P + 8), attn.ERR_MISALIGNED),
    (dict(cu_k=P + 2), attn.ERR_MISALIGNED),
])
def test_varlen_validation_rejects(kw, code):
    """Host-side checks of attn_fwd_varlen: each bad argument is refused before anything is enqueued."""
    assert varlen(**kw) == code


def test_varlen_empty_query_batch_is_a_no_op():
    # zero query rows: nothing to compute, NULL q/o/lse allowed, nothing enqueued
    assert varlen(q=None, o=None, lse=None, total_q=0, max_q=0) == attn.OK


def rope(**kw):
    a = dict(x=P, x8=P, sc=P, sg=P, c=P, s=P, B=1, H=2, S=128, D=128, br=64, mode=0, dt=2)
    a.update(kw)
    return attn.load().rope_hadamard_quant(a["x"], a["x8"], a["sc"], a["sg"], a["c"], a["s"], a["B"], a["H"],
                                           a["S"], a["D"], a["br"], a["mode"], a["dt"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(c=None), attn.ERR_INVALID_ARG),
    (dict(S=0), attn.ERR_INVALID_ARG),
    (dict(mode=2), attn.ERR_INVALID_ARG),
    (dict(dt=0), attn.ERR_INVALID_ARG),
    (dict(br=32), attn.ERR_UNSUPPORTED),
    (dict(D=96), attn.ERR_UNSUPPORTED),
    (dict(s=P + 4), attn.ERR_MISALIGNED),
])
def test_rope_hadamard_quant_validation_rejects(kw, code):
    """Host-side checks of rope_hadamard_quant: each bad argument is refused before anything is enqueued."""
    assert rope(**kw) == code


def persistent(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=2, S_q=128, S_k=128, D=128, causal=0, scale=0.125, dtype=2, n_wg=0)
    a.update(kw)
    return attn.load().attn_fwd_persistent(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["S_q"],
                                           a["S_k"], a["D"], a["causal"], ctypes.c_float(a["scale"]), a["dtype"],
                                           a["n_wg"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(n_wg=-1), attn.ERR_INVALID_ARG),
    (dict(lse=None), attn.ERR_INVALID_ARG),
    (dict(S_k=0), attn.ERR_INVALID_ARG),
    (dict(causal=2), attn.ERR_INVALID_ARG),
    (dict(dtype=0), attn.ERR_UNSUPPORTED),
    (dict(D=256), attn.ERR_UNSUPPORTED),
    (dict(causal=1, S_q=200, S_k=100), attn.ERR_UNSUPPORTED),
    (dict(v=P + 8), attn.ERR_MISALIGNED),
])
def test_persistent_validation_rejects(kw, code):
    """Host-side checks of attn_fwd_persistent: each bad argument is refused before the device is queried."""
    assert persistent(**kw) == code


def test_noalloc_refuses_splits_beyond_its_scratch():
    """attn_fwd_noalloc decides on the host, before touching the device, that a split needing more
    than ATTN_NOALLOC_SCRATCH_BYTES cannot run; the decode workload's split fits."""
    lib = attn.load()
    B, H, S_q, S_k, D = 8, 32, 64, 8192, 128
    assert attn.workspace_size(B, H, S_q, S_k, D) > attn.NOALLOC_SCRATCH_BYTES
    rc = lib.attn_fwd_noalloc(P, P, P, P, P, B, H, S_q, S_k, D, 0, ctypes.c_float(0.125), attn.BF16, None)
    assert rc == attn.ERR_WORKSPACE
    # argument errors come first, as in attn_fwd
    assert lib.attn_fwd_noalloc(None, P, P, P, P, B, H, S_q, S_k, D, 0, ctypes.c_float(0.125), attn.BF16,
                                None) == attn.ERR_INVALID_ARG
    assert 0 < attn.workspace_size(64, 32, 1, 32768, 128) <= attn.NOALLOC_SCRATCH_BYTES
    hdr = open(HEADER).read()
    assert f"#define ATTN_NOALLOC_SCRATCH_BYTES (16u << 20)" in hdr and attn.NOALLOC_SCRATCH_BYTES == 16 << 20


def fp8(**kw):
    a = dict(q8=P, k8=P, v8=P, qs=P, ks=P, vs=P, o=P, lse=P, B=1, H=2, S_q=128, S_k=128, D=128, causal=0,
             scale=0.125, br=64, vt=0)
    a.update(kw)
    return attn.load().attn_fwd_fp8(a["q8"], a["k8"], a["v8"], a["qs"], a["ks"], a["vs"], a["o"], a["lse"], a["B"],
                                    a["H"], a["S_q"], a["S_k"], a["D"], a["causal"], ctypes.c_float(a["scale"]),
                                    a["br"], a["vt"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(vs=None), attn.ERR_INVALID_ARG),
    (dict(vt=2), attn.ERR_INVALID_ARG),
    (dict(S_k=0), attn.ERR_INVALID_ARG),
    (dict(D=64), attn.ERR_UNSUPPORTED),
    (dict(br=32), attn.ERR_UNSUPPORTED),
    (dict(causal=1, S_q=200, S_k=128), attn.ERR_UNSUPPORTED),
    (dict(vt=1, S_k=100), attn.ERR_UNSUPPORTED),       # transposed V rows must be 16-byte aligned
    (dict(k8=P + 8), attn.ERR_MISALIGNED),
])
def test_fp8_validation_rejects(kw, code):
    """Host-side checks of attn_fwd_fp8 (including the transposed-V layout): refused before any launch."""
    assert fp8(**kw) == code


def test_mfma_stream_rejects_bad_arguments_on_the_host():
    """attn_mfma_stream checks its arguments before it asks for the device (nothing is dereferenced)."""
    lib = attn.load()
    P = ctypes.c_void_p(4096)
    f = ctypes.c_double(0.0)
    assert lib.attn_mfma_stream(3, 10, P, 1 << 20, ctypes.byref(f), None) == attn.ERR_INVALID_ARG
    assert lib.attn_mfma_stream(-1, 10, P, 1 << 20, ctypes.byref(f), None) == attn.ERR_INVALID_ARG
    assert lib.attn_mfma_stream(0, 0, P, 1 << 20, ctypes.byref(f), None) == attn.ERR_INVALID_ARG
    assert lib.attn_mfma_stream(0, 10, None, 1 << 20, ctypes.byref(f), None) == attn.ERR_INVALID_ARG
    assert lib.attn_mfma_stream(0, 10, P, 1 << 20, None, None) == attn.ERR_INVALID_ARG
    assert lib.attn_mfma_stream(1, 10, ctypes.c_void_p(4100), 1 << 20, ctypes.byref(f), None) == attn.ERR_MISALIGNED
