"""The C-ABI library on the CPU: it loads, exports every declared symbol, and
rejects bad arguments before touching the GPU.

Pointers passed here are fake integer addresses: every call in this file is
rejected by host-side validation, so nothing is dereferenced and no HIP call
is made. The one test that lets a call through to HIP runs only on a host
without a GPU.
"""

import ctypes
import os
import re
import subprocess

import pytest

import weight_activation_quantized_amd as mq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mq.h")

OK, NULL, SHAPE, ALIGN, UNSUP, WS, ALIAS, HIP = range(8)


@pytest.fixture(scope="module")
def lib():
    return mq.library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mq_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["mq_quant_per_token_int8", "mq_w8a8_scaled_mm", "mq_w8a8_mm_i32", "mq_w4a16_gemm",
              "mq_w4a16_gemv", "mq_w4a16_gemv_workspace_bytes", "mq_w4a16_block_weights",
              "mq_w4a16_gemv_blocked", "mq_w4a16_gemv_blocked_workspace_bytes", "mq_w8a8_linear",
              "mq_w8a8_linear_workspace_bytes", "mq_w4a16_gemm_workspace_bytes", "mq_kv_quant", "mq_abi_version",
              "mq_status_string", "mq_last_error", "mq_int4_reorder", "mq_int4_transpose", "mq_u16_transpose",
              "mq_quant_per_token_int8_bf16", "mq_w8a8_scaled_mm_bf16", "mq_w8a8_linear_bf16",
              "mq_kv_quant_bf16", "mq_w8a8_linear_noalloc", "mq_w4a16_gemm_bf16", "mq_w4a16_gemv_bf16",
              "mq_w4a16_gemv_blocked_bf16"]:
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", mq.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_abi_version_and_status_strings(lib):
    assert lib.mq_abi_version() == 2
    names = [lib.mq_status_string(i).decode() for i in range(8)]
    assert names == ["MQ_OK", "MQ_ERR_NULL", "MQ_ERR_SHAPE", "MQ_ERR_ALIGN", "MQ_ERR_UNSUPPORTED",
                     "MQ_ERR_WORKSPACE", "MQ_ERR_ALIAS", "MQ_ERR_HIP"]
    assert lib.mq_status_string(99).decode() == "MQ_ERR_UNKNOWN"


# fake, well-aligned, far-apart device addresses
A, B, C, D, E, F = (0x10_0000_0000 * (i + 1) for i in range(6))


def _err(lib):
    return lib.mq_last_error().decode()


def test_quant_validation(lib):
    q = lib.mq_quant_per_token_int8
    assert q(None, B, C, 4, 64, None) == NULL
    assert q(A, B, C, -1, 64, None) == SHAPE
    assert q(A, B, C, 4, 8, None) == SHAPE          # K < 16
    assert q(A, B, C, 4, 72, None) == SHAPE         # K % 16
    assert q(A, B, C, 4, (1 << 20) + 16, None) == SHAPE
    assert "K=" in _err(lib)
    assert q(A + 8, B, C, 4, 64, None) == ALIGN
    assert q(A, B + 4, C, 4, 64, None) == ALIGN
    assert q(A, B, C + 2, 4, 64, None) == ALIGN
    assert q(A, A + 64, C, 4, 64, None) == ALIAS    # xq inside x
    assert q(A, B, B + 64, 4, 64, None) == ALIAS    # s_tok inside xq
    assert q(A, B, C, 0, 64, None) == OK            # empty problem: nothing enqueued
    assert _err(lib) == ""
    assert q(None, None, None, 0, 64, None) == OK   # empty tensors may have NULL data
    assert q(A, None, C, 2, 64, None) == NULL
    assert "xq" in _err(lib)


def test_empty_problems_accept_null(lib):
    assert lib.mq_w8a8_scaled_mm(None, None, C, D, None, 0, 8, 64, None) == OK
    assert lib.mq_w8a8_scaled_mm(A, B, None, None, None, 4, 0, 64, None) == OK
    assert lib.mq_w8a8_mm_i32(None, B, None, 0, 8, 64, None) == OK
    assert lib.mq_w4a16_gemm(None, B, C, D, None, 0, 64, 256, 128, None, 0, None) == OK
    assert lib.mq_w4a16_gemv(None, B, C, D, None, 0, 64, 256, 128, None, 0, None) == OK
    # weights are never empty (N >= 8, K >= 128)
    assert lib.mq_w4a16_gemm(None, None, C, D, None, 0, 64, 256, 128, None, 0, None) == NULL


def test_w8a8_validation(lib):
    s = lib.mq_w8a8_scaled_mm
    assert s(A, None, C, D, E, 4, 8, 64, None) == NULL
    assert s(A, B, C, D, E, 4, 8, 60, None) == SHAPE
    assert s(A, B, C, D, E, 4, 8, 133136 + 16, None) == SHAPE
    assert s(A, B, C, D, E + 2, 4, 8, 133136, None) == ALIGN      # the largest K passes the shape check
    assert s(A, B, C, D, E, 4, -8, 64, None) == SHAPE
    assert s(A + 1, B, C, D, E, 4, 8, 64, None) == ALIGN
    assert s(A, B + 1, C, D, E, 4, 8, 64, None) == ALIGN
    assert s(A, B, C, D, E + 2, 4, 8, 64, None) == ALIGN
    assert s(A, B, C, D, C + 16, 4, 8, 64, None) == ALIAS
    assert s(A, B, C, D, E, 0, 8, 64, None) == OK
    assert s(A, B, C, D, E, 4, 0, 64, None) == OK
    i = lib.mq_w8a8_mm_i32
    assert i(A, None, C, 4, 8, 64, None) == NULL
    assert i(A, B, A + 16, 4, 8, 64, None) == ALIAS
    assert i(A, B, C + 8, 4, 8, 64, None) == ALIGN
    assert i(A, B, C, 4, 8, 40, None) == SHAPE


def test_w4a16_gemm_validation(lib):
    g = lib.mq_w4a16_gemm
    assert g(A, B, C, D, None, 4, 64, 256, 128, None, 0, None) == NULL
    # groups of 32, 64 and 128 rows and -1 (one scale / zero point per column
    # over all of K) are provided; others are not
    for group in (96, 256, 16, 0, -2):
        assert g(A, B, C, D, E, 4, 64, 256, group, None, 0, None) == UNSUP, group
    assert g(A, B, C, D, E, 4, 64, 192, 64, None, 0, None) == SHAPE      # K % 128, also for smaller groups
    assert g(A, B, C, D, E, 4, 64, 192, -1, None, 0, None) == SHAPE      # per-channel runs as groups of 128
    for group in (32, 64, 128, -1):
        assert g(A, B, C, D, E, 0, 64, 256, group, None, 0, None) == OK
    # the workspace is optional; given for a small grid it must be large enough
    wsb = lib.mq_w4a16_gemm_workspace_bytes
    assert wsb(4096, 4096, 4096, 128) == 0               # 256 tiles: never split
    need = wsb(2048, 4096, 4096, 128)                     # 128 tiles: split
    assert need > 0 and need % (4 * 2048 * 4096) == 0
    assert g(A, B, C, D, E, 2048, 4096, 4096, 128, F, need - 4, None) == WS
    assert g(A, B, C, D, E, 2048, 4096, 4096, 128, F + 4, need, None) == ALIGN
    assert g(A, B, C, D, E, 2048, 4096, 4096, 128, E, need, None) == ALIAS
    assert g(A, B, C, D, E, 4, 60, 256, 128, None, 0, None) == SHAPE     # N % 8
    assert g(A, B, C, D, E, 4, (1 << 27) + 8, 256, 128, None, 0, None) == SHAPE
    assert g(A, B, C, D, E, 4, 64, 200, 128, None, 0, None) == SHAPE     # K % 128
    assert g(A, B, C, D, E, 4, 64, 0, 128, None, 0, None) == SHAPE
    assert g(A + 8, B, C, D, E, 4, 64, 256, 128, None, 0, None) == ALIGN
    assert g(A, B + 2, C, D, E, 4, 64, 256, 128, None, 0, None) == ALIGN
    assert g(A, B, C, D, B + 16, 4, 64, 256, 128, None, 0, None) == ALIAS
    assert g(A, B, C, D, E, 0, 64, 256, 128, None, 0, None) == OK


def test_w4a16_gemv_validation(lib):
    v = lib.mq_w4a16_gemv
    ws = lib.mq_w4a16_gemv_workspace_bytes
    assert v(A, B, C, D, E, 65, 64, 256, 128, F, 1 << 20, None) == UNSUP
    assert "M <= 64" in _err(lib)
    # a problem that needs a workspace: small N -> K split across workgroups
    need = ws(1, 128, 4096, 128)
    assert need > 0
    assert v(A, B, C, D, E, 1, 128, 4096, 128, None, 0, None) == WS
    assert v(A, B, C, D, E, 1, 128, 4096, 128, F, need - 4, None) == WS
    assert v(A, B, C, D, E, 1, 128, 4096, 128, F + 4, need, None) == ALIGN
    assert v(A, B, C, D, E, 1, 128, 4096, 128, A, need, None) == ALIAS   # workspace over x
    assert v(A, B, C, D, E, 1, 128, 4096, 128, E, need, None) == ALIAS   # workspace over y
    assert v(A, B, C, D, E, 0, 128, 4096, 128, None, 0, None) == OK


def test_gemv_workspace_plan(lib):
    ws = lib.mq_w4a16_gemv_workspace_bytes
    # rejected problems need nothing
    assert ws(0, 512, 512, 128) == 0
    assert ws(65, 512, 512, 128) == 0
    assert ws(4, 512, 512, 96) == 0
    assert ws(4, 512, 512, -2) == 0
    # the workspace holds splits * M * N fp32 partial sums, with splits a
    # divisor of the group count K/G; the LDS-staged kernel (N % 32 == 0)
    # keeps at most 1024 rows per split
    for group in (32, 64, 128):
        for M, N, K in [(1, 24576, 4096), (4, 24576, 4096), (16, 24576, 4096), (1, 6144, 4096),
                        (8, 4096, 4096), (1, 4096, 12288), (4, 512, 512), (3, 424, 384),
                        (64, 24576, 4096), (64, 4096, 12288), (33, 6144, 4096), (40, 424, 384),
                        (1, 3072, 1024), (16, 3072, 1024)]:
            b = ws(M, N, K, group)
            assert b % (4 * M * N) == 0
            splits = b // (4 * M * N) or 1
            assert (K // group) % splits == 0
            if N % 32 == 0:
                assert K // splits <= 1024


def test_kv_quant_validation(lib):
    k = lib.mq_kv_quant
    assert k(A, B, C, 16, 128, 2, None) == UNSUP
    assert k(A, B, C, 16, 96, 8, None) == SHAPE       # not a power of two
    assert k(A, B, C, 16, 1024, 8, None) == SHAPE
    assert k(A, B, C, 1 << 26, 512, 8, None) == SHAPE   # 2^35 values: more than 2^32 lanes
    assert k(None, B, C, 16, 128, 8, None) == NULL
    assert k(A + 8, B, C, 16, 128, 8, None) == ALIGN
    assert k(A, B + 4, C, 16, 128, 8, None) == ALIGN   # 8-bit codes: 8-byte stores
    assert k(A, B + 2, C, 16, 128, 4, None) == ALIGN   # 4-bit codes: 4-byte stores
    assert k(A, B, C + 4, 16, 128, 8, None) == ALIGN
    assert k(A, A + 64, C, 16, 128, 8, None) == ALIAS
    assert k(A, B, C, 0, 128, 8, None) == OK


def test_w8a8_linear_validation(lib):
    f = lib.mq_w8a8_linear
    ws = lib.mq_w8a8_linear_workspace_bytes
    # sized for the two kernels at every M (the fused one-token path, K <=
    # 12288, leaves it unused)
    assert ws(1, 4096) >= 4096 + 4 and ws(2, 4096) >= 2 * 4096 + 2 * 4
    assert ws(3, 4096) >= 3 * 4096 + 3 * 4                # codes + scales
    assert ws(17, 4096) >= 17 * 4096 + 17 * 4
    assert ws(17, 40) == 0                               # rejected shape (K % 16)
    assert f(A, B, C, E, 4, 64, 40, None, 0, None) == SHAPE     # K % 16
    assert f(A, B, C, E, 4, 64, 133152, None, 0, None) == SHAPE  # int32 accumulator bound
    assert f(None, B, C, E, 4, 64, 64, None, 0, None) == NULL
    assert f(A + 8, B, C, E, 4, 64, 64, None, 0, None) == ALIGN
    assert f(A, B, C + 2, E, 4, 64, 64, None, 0, None) == ALIGN
    assert f(A, B, C, A + 16, 1, 64, 64, F, ws(1, 64), None) == ALIAS
    assert f(A, B, C, A + 16, 1, 16384, 64, None, 0, None) == ALIAS   # fused one-token form: no workspace
    assert f(A, B, C, E, 1, 64, 12304, None, 0, None) == WS           # one token, K > 12288: two kernels
    need = ws(32, 64)
    assert f(A, B, C, E, 32, 64, 64, None, 0, None) == WS
    assert f(A, B, C, E, 32, 64, 64, F, need - 4, None) == WS
    assert f(A, B, C, E, 32, 64, 64, F + 4, need, None) == ALIGN
    assert f(A, B, C, E, 32, 64, 64, E, need, None) == ALIAS   # workspace over y
    assert f(A, B, C, E, 0, 64, 64, None, 0, None) == OK


def test_w4a16_blocked_validation(lib):
    b = lib.mq_w4a16_block_weights
    assert b(B, C, 48, 256, None) == SHAPE       # N % 32
    assert b(B, C, 256, 200, None) == SHAPE      # K % 128
    assert b(None, C, 256, 256, None) == NULL
    assert b(B + 4, C + 8, 256, 256, None) == ALIGN   # blocked output needs 16 bytes
    assert b(B, B + 16, 256, 256, None) == ALIAS
    assert b(B, C, 0, 256, None) == OK
    v = lib.mq_w4a16_gemv_blocked
    ws = lib.mq_w4a16_gemv_blocked_workspace_bytes
    assert v(A, B, C, D, E, 1, 264, 256, 128, F, 1 << 20, None) == SHAPE   # N % 32
    assert v(A, B + 4, C, D, E, 1, 256, 256, 128, F, 1 << 20, None) == ALIGN
    assert v(A, B, C, D, E, 1, 256, 256, 96, F, 1 << 20, None) == UNSUP
    assert v(A, B, C, D, E, 65, 256, 256, 128, F, 1 << 20, None) == UNSUP
    assert v(A, B, C, D, E, 0, 256, 256, 128, None, 0, None) == OK
    # scale tables of 2^31 bytes or more (32-bit offsets in the kernels)
    assert v(A, B, C, D, E, 1, 32768, 1 << 20, 32, F, 1 << 40, None) == SHAPE and "scales" in _err(lib)
    assert ws(1, 32768, 1 << 20, 32) == 0
    # wide layers need no workspace; narrow ones with up to 8 tokens and
    # short K neither (one workgroup per strip takes all of K); narrow ones
    # with long K or more tokens split K and need one
    assert ws(1, 24576, 4096, 128) == 0
    assert ws(1, 4096, 4096, 128) == 0 and ws(4, 6144, 4096, 128) == 0
    assert ws(16, 4096, 4096, 128) > 0
    need = ws(1, 4096, 12288, 128)
    assert need > 0 and need % (4 * 4096) == 0
    assert v(A, B, C, D, E, 1, 4096, 12288, 128, None, 0, None) == WS
    assert v(A, B, C, D, E, 1, 4096, 12288, 128, F, need - 4, None) == WS
    assert ws(1, 264, 4096, 128) == 0 and ws(65, 4096, 4096, 128) == 0
    # a split divides the chunk count (K/128) and the workspace holds its partials
    for M, N, K in [(1, 6144, 4096), (16, 4096, 12288), (32, 3072, 1024), (64, 96, 640)]:
        b = ws(M, N, K, 128)
        splits = b // (4 * min(M, 64) * N) or 1
        assert b % (4 * min(M, 64) * N) == 0 and (K // 128) % splits == 0


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="lets a launch through; only meaningful without a GPU")
def test_valid_call_without_gpu_reports_hip_error(lib):
    st = lib.mq_quant_per_token_int8(A, B, C, 4, 64, None)
    assert st == HIP
    assert "hip" in _err(lib).lower()


def test_python_wrapper_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(4, 64, dtype=torch.float16)
    with pytest.raises(ValueError, match="GPU"):
        mq.quant_per_token_int8(x)


def test_mqerror_carries_status():
    e = mq.MqError(SHAPE, "K=3 bad")
    assert e.status == SHAPE and e.status_name == "MQ_ERR_SHAPE" and "K=3" in str(e)


def test_checkpoint_layout_validation(lib):
    import ctypes
    awq = (ctypes.c_uint8 * 8)(0, 2, 4, 6, 1, 3, 5, 7)
    dup = (ctypes.c_uint8 * 8)(0, 0, 4, 6, 1, 3, 5, 7)
    big = (ctypes.c_uint8 * 8)(0, 2, 4, 6, 1, 3, 5, 8)
    r = lib.mq_int4_reorder
    assert r(A, B, 16, dup, None) == UNSUP and b"permutation" in lib.mq_last_error()
    assert r(A, B, 16, big, None) == UNSUP
    assert r(A, B, -1, awq, None) == SHAPE
    assert r(A, B, 1 << 34, awq, None) == SHAPE
    assert r(None, B, 16, awq, None) == NULL
    assert r(A + 4, B, 16, awq, None) == ALIGN
    assert r(A, A + 32, 16, awq, None) == ALIAS
    assert r(A, B, 0, awq, None) == OK and r(A, B, 0, None, None) == OK
    t = lib.mq_int4_transpose
    assert t(A, B, 12, 64, awq, None) == SHAPE          # A % 8
    assert t(A, B, 64, 12, awq, None) == SHAPE          # B % 8
    assert t(A, B, 65536 * 128, 8, awq, None) == SHAPE  # grid rows
    assert t(A, B, 64, 64, dup, None) == UNSUP
    assert t(None, B, 64, 64, None, None) == NULL
    assert t(A + 2, B, 64, 64, None, None) == ALIGN
    assert t(A, A + 1024, 64, 64, None, None) == ALIAS  # 2 KB of words overlap
    assert t(A, B, 0, 64, None, None) == OK
    u = lib.mq_u16_transpose
    assert u(A, B, 65536 * 64, 8, None) == SHAPE
    assert u(A, B, 8, (1 << 30) + 1, None) == SHAPE
    assert u(None, B, 8, 8, None) == NULL
    assert u(A + 1, B, 8, 8, None) == ALIGN
    assert u(A, A + 64, 8, 8, None) == ALIAS
    assert u(A, B, 0, 8, None) == OK


def test_bf16_entries_validate_like_fp16(lib):
    q, q16 = lib.mq_quant_per_token_int8_bf16, lib.mq_quant_per_token_int8
    for args in ((A, B, C, 4, 40, None), (None, B, C, 4, 64, None), (A + 8, B, C, 4, 64, None),
                 (A, A + 16, C, 4, 64, None), (A, B, C, 0, 64, None)):
        assert q(*args) == q16(*args)
    assert q(A, B, C, 4, 40, None) == SHAPE and q(A, B, C, 0, 64, None) == OK
    f, f16 = lib.mq_w8a8_scaled_mm_bf16, lib.mq_w8a8_scaled_mm
    for args in ((A, B, C, D, E, 4, 64, 40, None), (A, B, C, D, A + 16, 4, 64, 64, None),
                 (A, B, C, D, E + 8, 4, 64, 64, None), (A, B, C, D, E, 0, 64, 64, None)):
        assert f(*args) == f16(*args)
    assert f(A, B, C, D, E, 4, 64, 133152, None) == SHAPE
    g, g16 = lib.mq_w8a8_linear_bf16, lib.mq_w8a8_linear
    for args in ((A, B, C, E, 4, 64, 40, None, 0, None), (A, B, C, A + 16, 1, 64, 64, None, 0, None),
                 (A, B, C, E, 32, 64, 64, None, 0, None), (A, B, C, E, 0, 64, 64, None, 0, None)):
        assert g(*args) == g16(*args)
    assert g(A, B, C, E, 32, 64, 64, None, 0, None) == WS


def test_kv_quant_bf16_validates_like_fp16(lib):
    k, k16 = lib.mq_kv_quant_bf16, lib.mq_kv_quant
    for args in ((A, B, C, 16, 128, 2, None), (A, B, C, 16, 96, 8, None), (None, B, C, 16, 128, 8, None),
                 (A + 8, B, C, 16, 128, 8, None), (A, A + 64, C, 16, 128, 8, None), (A, B, C, 0, 128, 8, None),
                 (A, B, C, 1 << 26, 512, 8, None)):
        assert k(*args) == k16(*args)


def test_w8a8_linear_noalloc_validation(lib):
    f = lib.mq_w8a8_linear_noalloc
    assert f(A, None, C, D, 4, 8, 64, None) == NULL
    assert f(A, B, C, D, 4, 8, 60, None) == SHAPE
    assert f(A + 8, B, C, D, 4, 8, 64, None) == ALIGN
    assert f(A, B, C, A + 16, 4, 8, 64, None) == ALIAS
    # the scratch holds mq_w8a8_linear_workspace_bytes(M, K) <= MQ_NOALLOC_SCRATCH_BYTES
    assert mq.NOALLOC_SCRATCH_BYTES == 33816576
    assert lib.mq_w8a8_linear_workspace_bytes(2048, 12288) <= mq.NOALLOC_SCRATCH_BYTES
    assert lib.mq_w8a8_linear_workspace_bytes(4096, 12288) > mq.NOALLOC_SCRATCH_BYTES
    assert f(A, B, C, D, 4096, 8, 12288, None) == WS       # rejected before any HIP call
    assert "scratch" in _err(lib)
    assert f(A, B, C, D, 0, 8, 64, None) == OK             # empty problem: nothing enqueued, no lookup


def test_per_channel_group(lib):
    # group -1: every entry accepts it, and plans it as groups of 128 rows
    # (the workspace sizes are those of group 128)
    for fn in (lib.mq_w4a16_gemm, lib.mq_w4a16_gemv, lib.mq_w4a16_gemv_blocked,
               lib.mq_w4a16_gemm_bf16, lib.mq_w4a16_gemv_bf16, lib.mq_w4a16_gemv_blocked_bf16):
        assert fn(A, B, C, D, E, 0, 256, 512, -1, None, 0, None) == OK
        assert fn(A, B, C, D, E, 0, 256, 512, -3, None, 0, None) == UNSUP
    for M, N, K in [(2048, 4096, 4096), (300, 1032, 1024), (4096, 4096, 4096)]:
        assert lib.mq_w4a16_gemm_workspace_bytes(M, N, K, -1) == lib.mq_w4a16_gemm_workspace_bytes(M, N, K, 128)
    for M, N, K in [(1, 128, 4096), (16, 4096, 12288), (40, 4096, 4096)]:
        assert lib.mq_w4a16_gemv_workspace_bytes(M, N, K, -1) == lib.mq_w4a16_gemv_workspace_bytes(M, N, K, 128)
    for M, N, K in [(1, 4096, 12288), (16, 4096, 4096), (64, 6144, 4096), (1, 24576, 4096)]:
        assert (lib.mq_w4a16_gemv_blocked_workspace_bytes(M, N, K, -1) ==
                lib.mq_w4a16_gemv_blocked_workspace_bytes(M, N, K, 128))
    assert lib.mq_w4a16_gemv_blocked_workspace_bytes(1, 4096, 12288, -2) == 0
