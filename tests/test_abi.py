"""The C-ABI library loads on a host without a GPU, exports every function the
header declares, and rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_int4.h")
# MOE_LIB selects another build of the library (the host-sanitizer build)
LIB = os.environ.get("MOE_LIB") or os.path.join(ROOT, "int4_routed_expert_moe_amd", "libmoe_int4.so")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from int4_routed_expert_moe_amd import build
        build.build(verbose=False)
    return ctypes.CDLL(LIB)


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)
    return sorted(set(names))


def test_header_declares_the_layer_calls():
    names = _declared()
    for n in ("moe_route", "moe_permute", "moe_int4_grouped_swiglu", "moe_int4_grouped_down", "moe_combine",
              "moe_linear_bf16", "moe_rmsnorm_bf16", "moe_quant_act_int8"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_names_match_header():
    from int4_routed_expert_moe_amd import moe
    assert sorted(moe.EXPORTS) == _declared()
    for n in _declared():
        if n not in ("moe_status_string", "moe_last_error_detail") and not n.endswith("_workspace_bytes"):
            assert hasattr(moe, n), n


def _status(lib, fn, *args):
    f = getattr(lib, fn)
    f.restype = ctypes.c_int
    return f(*args)


def test_host_validation_rejects_bad_arguments(lib):
    P = ctypes.c_void_p
    fake = P(0x1000)          # never dereferenced: validation fails first
    odd = P(0x1002)           # misaligned
    null = None
    lib.moe_last_error_detail.restype = ctypes.c_char_p
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_route_workspace_bytes.restype = ctypes.c_size_t
    # route: k > E, E too large, H not a multiple of 128, null pointers, small workspace
    assert _status(lib, "moe_route", fake, fake, fake, 4, 256, 8, 9, 1, fake, fake, fake, ctypes.c_size_t(1 << 20), null) == -2
    assert _status(lib, "moe_route", fake, fake, fake, 4, 256, 2000, 8, 1, fake, fake, fake, ctypes.c_size_t(1 << 30), null) == -2
    assert _status(lib, "moe_route", fake, fake, fake, 4, 200, 16, 2, 1, fake, fake, fake, ctypes.c_size_t(1 << 20), null) == -2
    # a router matrix of 4 GiB (1024 experts x 2^21 hidden, bf16) is past the kernel's 32-bit offsets
    assert _status(lib, "moe_route", fake, fake, fake, 4, 1 << 21, 1024, 2, 1, fake, fake, fake, ctypes.c_size_t(1 << 30), null) == -2
    assert _status(lib, "moe_route", null, fake, fake, 4, 256, 16, 2, 1, fake, fake, fake, ctypes.c_size_t(1 << 20), null) == -1
    assert _status(lib, "moe_route", odd, fake, fake, 4, 256, 16, 2, 1, fake, fake, fake, ctypes.c_size_t(1 << 20), null) == -1
    assert _status(lib, "moe_route", fake, fake, fake, 4, 256, 16, 2, 1, fake, fake, fake, ctypes.c_size_t(8), null) == -3
    assert b"workspace" in lib.moe_last_error_detail()
    assert lib.moe_route_workspace_bytes(64, 7168, 384) == 64 * 384 * 4 + 64 * (7168 // 64) * 384 * 4  # logits + block sums
    assert lib.moe_route_workspace_bytes(4096, 7168, 384) == 4096 * 384 * 4  # logits
    # zero tokens is a no-op
    assert _status(lib, "moe_route", null, null, null, 0, 256, 16, 2, 1, null, null, null, ctypes.c_size_t(0), null) == 0
    # permute: E too large, k > 16, null counts; from 16384 slots a workspace of per-block counts
    z = ctypes.c_size_t(0)
    assert _status(lib, "moe_permute", fake, 4, 2, 4096, fake, fake, fake, fake, null, z, null) == -2
    assert _status(lib, "moe_permute", fake, 4, 17, 64, fake, fake, fake, fake, null, z, null) == -2
    assert _status(lib, "moe_permute", fake, 4, 2, 64, null, fake, fake, fake, null, z, null) == -1
    lib.moe_permute_workspace_bytes.restype = ctypes.c_size_t
    assert lib.moe_permute_workspace_bytes(64, 8, 384) == 0              # one workgroup
    assert lib.moe_permute_workspace_bytes(2047, 8, 384) == 0            # 16376 slots
    assert lib.moe_permute_workspace_bytes(2048, 8, 384) == 16 * 384 * 4  # 16 blocks of 1024 slots
    assert lib.moe_permute_workspace_bytes(8192, 8, 384) == 64 * 384 * 4
    assert lib.moe_permute_workspace_bytes(3001, 7, 5) == 21 * 5 * 4      # ragged last block
    # the workspace-free permutation: its fixed buffer holds 256 blocks x 1024 experts of counts
    assert _status(lib, "moe_permute_noalloc", fake, 32769, 8, 1024, fake, fake, fake, fake, null) == -2
    assert b"262144" in lib.moe_last_error_detail()
    assert _status(lib, "moe_permute_noalloc", fake, 4, 2, 64, null, fake, fake, fake, null) == -1
    need = ctypes.c_size_t(16 * 384 * 4)
    assert _status(lib, "moe_permute", fake, 2048, 8, 384, fake, fake, fake, fake, null, z, null) == -3
    assert _status(lib, "moe_permute", fake, 2048, 8, 384, fake, fake, fake, fake, fake, ctypes.c_size_t(100), null) == -3
    assert _status(lib, "moe_permute", fake, 2048, 8, 384, fake, fake, fake, fake, odd, need, null) == -1
    # grouped gemms: bad mode, unsupported widths, scales in the wrong mode, null pointers
    g = "moe_int4_grouped_swiglu"
    assert _status(lib, g, 7, fake, null, fake, fake, fake, fake, fake, fake, 4, 2, 16, 256, 128, fake, null, null) == -1
    assert _status(lib, g, 0, fake, null, fake, fake, fake, fake, fake, fake, 4, 2, 16, 200, 128, fake, null, null) == -2
    assert _status(lib, g, 0, fake, null, fake, fake, fake, fake, fake, fake, 4, 2, 16, 256, 96, fake, null, null) == -2
    assert _status(lib, g, 0, fake, fake, fake, fake, fake, fake, fake, fake, 4, 2, 16, 256, 128, fake, null, null) == -1
    assert _status(lib, g, 1, fake, null, fake, fake, fake, fake, fake, fake, 4, 2, 16, 256, 128, fake, null, null) == -1
    assert _status(lib, g, 0, fake, null, null, fake, fake, fake, fake, fake, 4, 2, 16, 256, 128, fake, null, null) == -1
    # one expert's packed matrix must stay below 2 GiB (32-bit addressing inside the kernels)
    assert _status(lib, g, 0, fake, null, fake, fake, fake, fake, fake, fake, 4, 2, 16, 65536, 65536, fake, null, null) == -2
    assert b"2 GiB" in lib.moe_last_error_detail()
    d = "moe_int4_grouped_down"
    assert _status(lib, d, 0, fake, null, fake, fake, fake, 4, 2, 16, 65536, 65536, fake, null) == -2
    assert b"2 GiB" in lib.moe_last_error_detail()
    assert _status(lib, d, 0, fake, null, fake, fake, fake, 4, 2, 16, 128, 384, fake, null) == -2
    # scale check: null or misaligned pointers, and nothing to check
    cs = "moe_int4_check_scales"
    lib.moe_int4_check_scales.argtypes = [P, ctypes.c_size_t, P, P]
    assert _status(lib, cs, null, 16, fake, null) == -1
    assert _status(lib, cs, P(0x1001), 16, fake, null) == -1
    assert _status(lib, cs, fake, 16, P(0x1002), null) == -1
    assert _status(lib, cs, null, 0, null, null) == 0
    assert _status(lib, d, 1, fake, null, fake, fake, fake, 4, 2, 16, 128, 256, fake, null) == -1
    # combine: exact mode with a shared input, misaligned output
    assert _status(lib, "moe_combine", 1, fake, fake, fake, fake, 4, 2, 256, fake, null) == -1
    assert _status(lib, "moe_combine", 0, fake, fake, fake, null, 4, 2, 256, odd, null) == -1
    # dense: N not a multiple of 64, K not a multiple of 128
    assert _status(lib, "moe_linear_bf16", fake, fake, null, fake, 4, 100, 256, null, ctypes.c_size_t(0), null) == -2
    assert _status(lib, "moe_linear_bf16", fake, fake, null, fake, 4, 128, 200, null, ctypes.c_size_t(0), null) == -2
    lib.moe_dense_workspace_bytes.restype = ctypes.c_size_t
    need = lib.moe_dense_workspace_bytes(64, 4096, 7168)
    assert need > 0  # decode shapes split K
    assert _status(lib, "moe_dense_swiglu_bf16", fake, fake, fake, fake, 64, 7168, 2048, null, ctypes.c_size_t(0), null) == -3
    assert lib.moe_dense_workspace_bytes(8192, 4096, 7168) == 0
    assert _status(lib, "moe_rmsnorm_bf16", fake, fake, ctypes.c_float(-1.0), fake, 4, 64, null) == -1
    assert _status(lib, "moe_int4_group_sums_i32", fake, fake, 20, 16, 64, fake, null) == -2
    # prepack: N not a multiple of 16, K not a multiple of 128, overlapping output, misaligned scale
    pp = "moe_int4_prepack"
    assert _status(lib, pp, fake, fake, 2, 24, 256, P(0x100000), P(0x200000), null) == -2
    assert _status(lib, pp, fake, fake, 2, 32, 200, P(0x100000), P(0x200000), null) == -2
    assert _status(lib, pp, fake, fake, 2, 32, 256, fake, P(0x200000), null) == -1
    assert _status(lib, pp, fake, P(0x3004), 2, 32, 256, P(0x100000), P(0x200000), null) == -1
    assert _status(lib, pp, null, null, 0, 32, 256, null, null, null) == 0
    # grouped routing: topk_group > n_group, groups not dividing E, k beyond the kept groups, NaN scale
    rg = "moe_route_grouped"
    lib.moe_route_grouped.argtypes = [P, P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_float, P, P, P, ctypes.c_size_t, P]
    big = ctypes.c_size_t(1 << 30)
    assert _status(lib, rg, fake, fake, fake, 4, 256, 64, 4, 1, 4, 5, 1.0, fake, fake, fake, big, null) == -1
    assert _status(lib, rg, fake, fake, fake, 4, 256, 64, 4, 1, 5, 2, 1.0, fake, fake, fake, big, null) == -2
    assert _status(lib, rg, fake, fake, fake, 4, 256, 64, 9, 1, 8, 1, 1.0, fake, fake, fake, big, null) == -2
    assert _status(lib, rg, fake, fake, fake, 4, 256, 64, 4, 1, 8, 2, float("nan"), fake, fake, fake, big, null) == -1
    assert _status(lib, rg, null, null, null, 0, 256, 64, 4, 1, 8, 2, 1.0, null, null, null, ctypes.c_size_t(0), null) == 0
    # ExactLinear 8-bit weights: K not a multiple of 128, null pointer, zero rows
    assert _status(lib, "moe_exact_linear_i8w", fake, fake, fake, fake, 4, 64, 96, fake, null) == -2
    assert _status(lib, "moe_exact_linear_i8w", null, fake, fake, fake, 4, 64, 128, fake, null) == -1
    assert _status(lib, "moe_exact_linear_i8w", null, null, null, null, 0, 64, 128, null, null) == 0
    # staging conversion: K not a multiple of 8, null pointer, overlap, zero rows
    assert _status(lib, "moe_act_f16p", fake, 4, 12, P(0x200000), null) == -2
    assert _status(lib, "moe_act_f16p", null, 4, 16, P(0x200000), null) == -1
    assert _status(lib, "moe_act_f16p", P(0x100000), 4, 16, P(0x100010), null) == -1
    assert _status(lib, "moe_act_f16p", null, 0, 16, null, null) == 0
    # grouped calls accept the staging-format mode and reject others
    assert _status(lib, g, 3, fake, null, fake, fake, fake, fake, fake, fake, 4, 2, 16, 256, 128, fake, null, null) == -1
    assert _status(lib, g, 2, fake, fake, fake, fake, fake, fake, fake, fake, 4, 2, 16, 256, 128, fake, null, null) == -1
    assert lib.moe_status_string(-3) == b"workspace missing or too small"
