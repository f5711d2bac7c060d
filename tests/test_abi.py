"""The C-ABI library builds, loads and exports every entry point include/mxgemm.h
declares; argument errors are reported on the host before anything reaches a
device.  Runs without a GPU (no kernel is ever launched here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxgemm.h")


@pytest.fixture(scope="module")
def mx():
    from block_scaled_precision_act_amd import build, mxgemm
    if not os.path.exists(mxgemm.LIB_PATH):
        build.build(verbose=False)
    return mxgemm


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_four_path_entry_points():
    names = declared_functions()
    for n in ("mx_quant_act_bf16", "mx_gemm_a4w4_bf16", "ptpc_quant_act_fp8", "gemm_a8w8_ptpc_bf16"):
        assert n in names


def test_every_declared_symbol_is_exported(mx):
    lib = ctypes.CDLL(mx.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert hasattr(mx, name) or name == "mx_status_string", name


def test_version_and_status_strings(mx):
    assert mx.mx_abi_version() == 1
    for code in range(7):
        assert mx.status_string(code).startswith("MX_")
    assert mx.status_string(99) == "MX_ERROR_UNKNOWN"


FAKE = 0x10000  # a non-null, 64K-aligned address that is never dereferenced


def test_quantizer_argument_errors(mx):
    assert mx.mx_quant_act_bf16(FAKE, -1, 64, FAKE, FAKE) == mx.MX_ERROR_INVALID_VALUE
    assert mx.mx_quant_act_bf16(FAKE, 4, 48, FAKE, FAKE) == mx.MX_ERROR_UNSUPPORTED_SHAPE
    assert mx.mx_quant_act_bf16(FAKE, 4, 0, FAKE, FAKE) == mx.MX_ERROR_UNSUPPORTED_SHAPE
    assert mx.mx_quant_act_bf16(None, 4, 64, FAKE, FAKE) == mx.MX_ERROR_INVALID_VALUE
    assert mx.mx_quant_act_bf16(FAKE + 2, 4, 64, FAKE, FAKE) == mx.MX_ERROR_MISALIGNED
    assert mx.mx_quant_act_bf16(FAKE, 4, 64, FAKE + 8, FAKE) == mx.MX_ERROR_MISALIGNED
    assert mx.mx_quant_act_bf16(None, 0, 64, None, None) == mx.MX_SUCCESS  # empty: no-op
    assert mx.mx_quant_weight_f32(FAKE, 4, 40, FAKE, FAKE) == mx.MX_ERROR_UNSUPPORTED_SHAPE
    assert mx.ptpc_quant_act_fp8(FAKE, 4, 12, FAKE, FAKE) == mx.MX_ERROR_UNSUPPORTED_SHAPE
    assert mx.ptpc_quant_act_fp8(FAKE, 4, 64, FAKE, FAKE + 2) == mx.MX_ERROR_MISALIGNED
    assert mx.ptpc_quant_act_fp8(FAKE, 4, 64, None, FAKE) == mx.MX_ERROR_INVALID_VALUE
    assert mx.ptpc_quant_weight_f32(FAKE, -3, 64, FAKE, FAKE) == mx.MX_ERROR_INVALID_VALUE
    assert mx.ptpc_quant_act_fp8(None, 0, 64, None, None) == mx.MX_SUCCESS


def test_gemm_argument_errors(mx):
    g4 = mx.mx_gemm_a4w4_bf16
    assert g4(FAKE, FAKE, FAKE, FAKE, FAKE, -1, 8, 128) == mx.MX_ERROR_INVALID_VALUE
    assert g4(FAKE, FAKE, FAKE, FAKE, FAKE, 8, -1, 128) == mx.MX_ERROR_INVALID_VALUE
    assert g4(FAKE, FAKE, FAKE, FAKE, FAKE, 8, 8, 96) == mx.MX_ERROR_UNSUPPORTED_SHAPE
    assert g4(FAKE, FAKE, FAKE, FAKE, FAKE, 8, 8, 0) == mx.MX_ERROR_UNSUPPORTED_SHAPE
    assert g4(FAKE, None, FAKE, FAKE, FAKE, 8, 8, 128) == mx.MX_ERROR_INVALID_VALUE
    assert g4(FAKE + 4, FAKE, FAKE, FAKE, FAKE, 8, 8, 128) == mx.MX_ERROR_MISALIGNED
    assert g4(FAKE, FAKE + 2, FAKE, FAKE, FAKE, 8, 8, 128) == mx.MX_ERROR_MISALIGNED
    assert g4(FAKE, FAKE, FAKE, FAKE, FAKE + 1, 8, 8, 128) == mx.MX_ERROR_MISALIGNED
    assert g4(None, None, None, None, None, 0, 8, 128) == mx.MX_SUCCESS
    assert g4(None, None, None, None, None, 8, 0, 128) == mx.MX_SUCCESS
    # the split-K decode GEMM (M <= 64, K parts of 2048, at least 4 of them, 128 .. 256 workgroups): tiles x
    # K parts x 4 waves x fragments x 4 KB of partial slots
    assert mx.mx_gemm_a4w4_workspace_bytes(64, 4096, 8192) == 32 * 4 * 4 * 2 * 4096
    assert mx.mx_gemm_a4w4_workspace_bytes(32, 2048, 16384) == 16 * 8 * 4 * 1 * 4096
    assert mx.mx_gemm_a4w4_workspace_bytes(64, 7168, 8192) == 56 * 4 * 4 * 2 * 4096
    assert mx.mx_gemm_a4w4_workspace_bytes(1, 7168, 8192) == 56 * 4 * 4 * 1 * 4096
    assert mx.mx_gemm_a4w4_workspace_bytes(64, 4096, 16384) == 8 << 20     # 256 workgroups: the largest
    assert mx.mx_gemm_a4w4_workspace_bytes(64, 7168, 16384) == 0    # 448 workgroups: not resident at once
    assert mx.mx_gemm_a4w4_workspace_bytes(64, 7168, 4096) == 0     # 2 parts: the decode rings
    # the layer: room for the one-launch path's partial slots and for the two-launch path's codes and
    # scales, which sit past the largest partial area (8 MiB)
    assert mx.mx_linear_a4w4_workspace_bytes(64, 7168, 8192) == (8 << 20) + 64 * 4096 + 64 * 256
    assert mx.mx_linear_a4w4_workspace_bytes(1, 7168, 8192) == (8 << 20) + 4096 + 256
    assert mx.mx_linear_a4w4_workspace_bytes(100, 7168, 8192) == (8 << 20) + 100 * 4096 + 25600
    assert mx.mx_gemm_a4w4_workspace_bytes(64, 128 * 256 + 1, 8192) == 0  # more than 256 tiles
    # 64 < M <= 128: the split over two row halves, 2 x tiles x parts x 4 waves x 2 fragments x 4 KB
    assert mx.mx_gemm_a4w4_workspace_bytes(65, 7168, 8192) == 2 * 56 * 2 * 4 * 2 * 4096
    assert mx.mx_gemm_a4w4_workspace_bytes(128, 7168, 16384) == 2 * 56 * 2 * 4 * 2 * 4096   # parts of 8192
    assert mx.mx_gemm_a4w4_workspace_bytes(100, 2900, 16384) == 2 * 23 * 4 * 4 * 2 * 4096
    assert mx.mx_gemm_a4w4_workspace_bytes(128, 7168, 4096) == 0    # the two-row-halves ring
    # M > 128, at most 128 tiles of 128 x 128, K % 2048 == 0: two K parts, tiles x 4 waves x 4 fragments x 4 KB
    # (compact slots: only the one written per slice and wave)
    assert mx.mx_gemm_a4w4_workspace_bytes(129, 7168, 8192) == 112 * 4 * 4 * 4096
    assert mx.mx_gemm_a4w4_workspace_bytes(256, 7168, 8192) == 112 * 4 * 4 * 4096
    assert mx.mx_gemm_a4w4_workspace_bytes(200, 1000, 4096) == 16 * 4 * 4 * 4096
    assert mx.mx_gemm_a4w4_workspace_bytes(2048, 1024, 2048) == 128 * 4 * 4 * 4096 == 8 << 20  # the largest
    assert mx.mx_gemm_a4w4_workspace_bytes(257, 7168, 8192) == 0    # 168 tiles: one per workgroup
    assert mx.mx_gemm_a4w4_workspace_bytes(256, 7168, 8192 + 1024) == 0   # K % 2048 != 0
    assert mx.mx_gemm_a4w4_workspace_bytes(64, 512, 8192) == 0      # too few tiles to split
    assert mx.mx_gemm_a4w4_workspace_bytes(64, 7168, 8192 + 128) == 0
    assert g4(FAKE, FAKE, FAKE, FAKE, FAKE, 64, 4096, 8192, None, 0) == mx.MX_ERROR_WORKSPACE
    assert g4(FAKE, FAKE, FAKE, FAKE, FAKE, 64, 4096, 8192, FAKE, 1024) == mx.MX_ERROR_WORKSPACE
    na = mx.mx_gemm_a4w4_bf16_noalloc
    # (no call with valid arguments here: it would reach the device with fake pointers)
    assert na(FAKE, FAKE, FAKE, FAKE, FAKE, 8, 8, 96) == mx.MX_ERROR_UNSUPPORTED_SHAPE
    assert na(FAKE, None, FAKE, FAKE, FAKE, 64, 4096, 8192) == mx.MX_ERROR_INVALID_VALUE
    assert na(FAKE, FAKE, FAKE, FAKE, FAKE + 1, 64, 4096, 8192) == mx.MX_ERROR_MISALIGNED
    assert na(None, None, None, None, None, 0, 4096, 8192) == mx.MX_SUCCESS
    lin = mx.mx_linear_a4w4_bf16
    wsl = mx.mx_linear_a4w4_workspace_bytes(64, 7168, 8192)
    assert lin(FAKE, FAKE, FAKE, FAKE, 64, 7168, 8192, None, 0) == mx.MX_ERROR_WORKSPACE
    assert lin(FAKE, FAKE, FAKE, FAKE, 64, 7168, 8192, FAKE, wsl - 1) == mx.MX_ERROR_WORKSPACE
    assert lin(FAKE, FAKE, FAKE, FAKE, 64, 7168, 8096, FAKE, wsl) == mx.MX_ERROR_UNSUPPORTED_SHAPE  # K % 128
    assert lin(FAKE + 8, FAKE, FAKE, FAKE, 64, 7168, 8192, FAKE, wsl) == mx.MX_ERROR_MISALIGNED
    assert lin(FAKE, FAKE, FAKE, FAKE, 64, 7168, 8192, FAKE + 16, wsl) == mx.MX_ERROR_MISALIGNED    # 256-byte ws
    assert lin(None, FAKE, FAKE, FAKE, 64, 7168, 8192, FAKE, wsl) == mx.MX_ERROR_INVALID_VALUE
    assert lin(None, None, None, None, 0, 7168, 8192, None, 0) == mx.MX_SUCCESS
    g8 = mx.gemm_a8w8_ptpc_bf16
    assert g8(FAKE, FAKE, FAKE, FAKE, FAKE, 8, 8, 64) == mx.MX_ERROR_UNSUPPORTED_SHAPE
    assert g8(FAKE, FAKE + 2, FAKE, FAKE, FAKE, 8, 8, 128) == mx.MX_ERROR_MISALIGNED
    assert g8(None, None, None, None, None, 0, 0, 128) == mx.MX_SUCCESS
    # the FP8 split-K decode GEMM: 33 <= M <= 64, K parts of 2048 (4 or 8), 128 .. 256 workgroups
    w8 = mx.gemm_a8w8_ptpc_workspace_bytes
    assert w8(64, 7168, 8192) == 56 * 4 * 4 * 2 * 4096
    assert w8(33, 4096, 16384) == 32 * 8 * 4 * 2 * 4096
    assert w8(32, 7168, 8192) == 0      # the decode ring (measured as fast at M <= 32)
    assert w8(64, 7168, 4096) == 0      # 2 parts
    assert w8(64, 7168, 16384) == 0     # 448 workgroups
    assert w8(65, 7168, 8192) == 0
    # M > 128, at most 128 tiles of 128 x 128 (and K / 2 >= 1024): two K parts, tiles x 64 KB; at most 256 tiles:
    # full K, no workspace
    assert w8(256, 7168, 8192) == 112 * 64 * 1024 == 7340032
    assert w8(129, 1001, 4096) == 16 * 64 * 1024
    assert w8(300, 1000, 2048) == 24 * 64 * 1024
    assert w8(300, 1000, 1024) == 0                                        # parts would be under 1024
    assert w8(512, 7168, 8192) == 0                                        # 224 tiles: full K
    # past 256 tiles of 128, at most 128 tiles of 256 x 224: K in parts of them, tiles x 4 waves x (parts - 1) x 56 KB
    assert w8(1024, 7168, 8192) == 128 * 4 * 1 * 56 * 1024                # 2 parts
    assert w8(1100, 4096, 4096) == 95 * 4 * 1 * 56 * 1024
    assert w8(1025, 7168, 8192) == 0                                       # 160 tiles: one workgroup each
    assert g8(FAKE, FAKE, FAKE, FAKE, FAKE, 64, 7168, 8192, None, 0) == mx.MX_ERROR_WORKSPACE
    assert g8(FAKE, FAKE, FAKE, FAKE, FAKE, 64, 7168, 8192, FAKE, 1024) == mx.MX_ERROR_WORKSPACE
    assert g8(FAKE, FAKE, FAKE, FAKE, FAKE, 64, 7168, 8192, FAKE + 8, w8(64, 7168, 8192)) == mx.MX_ERROR_MISALIGNED


def test_grouped_gemm_argument_errors(mx):
    gg = mx.mx_gemm_a4w4_grouped_bf16
    ok_args = (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    assert gg(*ok_args, -1, 16, 512, 2048) == mx.MX_ERROR_INVALID_VALUE       # G
    assert gg(*ok_args, 4, -1, 512, 2048) == mx.MX_ERROR_INVALID_VALUE        # max_rows
    assert gg(*ok_args, 4, 16, -1, 2048) == mx.MX_ERROR_INVALID_VALUE         # N
    assert gg(*ok_args, 4, 16, 512, 1000) == mx.MX_ERROR_UNSUPPORTED_SHAPE    # K % 512
    assert gg(*ok_args, 4, 16, 512, 18432) == mx.MX_ERROR_UNSUPPORTED_SHAPE   # K > 16384
    assert gg(*ok_args, 65536, 16, 512, 2048) == mx.MX_ERROR_UNSUPPORTED_SHAPE
    assert gg(FAKE, FAKE, FAKE, FAKE, FAKE, None, 4, 16, 512, 2048) == mx.MX_ERROR_INVALID_VALUE
    assert gg(FAKE, FAKE + 4, FAKE, FAKE, FAKE, FAKE, 4, 16, 512, 2048) == mx.MX_ERROR_MISALIGNED
    assert gg(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 2, 4, 16, 512, 2048) == mx.MX_ERROR_MISALIGNED
    assert gg(None, None, None, None, None, None, 0, 16, 512, 2048) == mx.MX_SUCCESS   # no groups
    assert gg(None, None, None, None, None, None, 4, 0, 512, 2048) == mx.MX_SUCCESS   # empty groups


def test_valid_arguments_without_a_gpu_report_no_device(mx):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present: valid arguments would launch a kernel")
    assert mx.mx_quant_act_bf16(FAKE, 4, 64, FAKE, FAKE) == mx.MX_ERROR_DEVICE


def test_tensor_helpers_reject_bad_inputs_before_the_library(mx):
    import torch
    with pytest.raises(TypeError):
        mx.quant_act_mx(torch.zeros(2, 64, dtype=torch.float32))
    with pytest.raises(ValueError):
        mx.quant_act_mx(torch.zeros(2, 64, dtype=torch.bfloat16))  # not a device tensor


def test_tensor_helpers_reject_bad_outputs(mx):
    """A caller-supplied output of the wrong dtype, shape, device or layout is refused before its
    pointer reaches a kernel (the kernels write shape-many elements through it)."""
    import torch
    like = torch.zeros(2, 64, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        mx._out(torch.zeros(2, 32, dtype=torch.float32), torch.uint8, (2, 32), like, "q")
    with pytest.raises(ValueError, match="shape"):
        mx._out(torch.zeros(2, 31, dtype=torch.uint8), torch.uint8, (2, 32), like, "q")
    with pytest.raises(ValueError, match="shape"):
        mx._out(torch.zeros(64, 2, dtype=torch.bfloat16), torch.bfloat16, (2, 64), like, "y")
    with pytest.raises(ValueError, match="device"):
        mx._out(torch.zeros(2, 32, dtype=torch.uint8), torch.uint8, (2, 32), like, "q")   # host memory
    assert mx._out(None, torch.uint8, (2, 32), like, "q").shape == (2, 32)
