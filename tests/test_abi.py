"""CPU checks of the C ABI: the library loads, exports every entry point that
include/fa.h declares, and rejects bad arguments on the host before any HIP
call (no GPU is needed; every case below fails validation, so nothing is
launched).  Requires the library to be built (``__graft_entry__.build()``)."""

import os
import re

import pytest

from attention_fa2_tiles_amd import lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

if not os.path.exists(lib.LIB_PATH):
    pytest.skip("libfa2tiles.so not built; run python -m attention_fa2_tiles_amd.build", allow_module_level=True)

# tests/test_abi_sanitized.py reruns this module against a copy of the library
# whose host layer is built with AddressSanitizer and UBSan
_SANITIZED = os.environ.get("FA2TILES_ABI_TEST_LIB")
if _SANITIZED:
    lib._lib = lib.load(_SANITIZED)


def test_library_under_test():
    # the sanitized rerun must exercise the sanitized copy, not the plain one
    assert lib.load()._name == (_SANITIZED or lib.LIB_PATH)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_\w+|pw_\w+|resmerge_\w+|lse_merge_\w+)\s*\(", text)))


def test_exports_every_declared_symbol():
    L = lib.load()
    names = declared_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(L, n), f"{n} declared in fa.h but not exported"
    # the binding covers exactly the declared surface
    assert sorted(lib.EXPORTS) == names


def test_version_and_strerror():
    assert lib.fa_version() >= 100
    for code, name in lib.STATUS.items():
        assert lib.fa_strerror(code).startswith(name)
    assert "unknown" in lib.fa_strerror(12345)


def test_workspace_sizes():
    assert lib.fa_bwd_workspace_size(2, 3, 128, 256, 64, 2) == 2 * 3 * 128 * 4
    assert lib.pw_bwd_workspace_size(1, 1, 64, 64, 64, 1) == 64 * 4
    assert lib.fa_bwd_workspace_size(0, 3, 128, 256, 64, 2) == 0
    n = lib.resmerge_bwd_workspace_size(32768, 4096)
    assert n > 0 and n % (4096 * 4) == 0
    assert lib.resmerge_bwd_workspace_size(-1, 8) == 0


# Fake, 16-byte-aligned device addresses: never dereferenced, because each
# case below is rejected by host-side validation first.
A = 0x100000
P = [A + 0x1000 * i for i in range(20)]


def status(fn, *args):
    with pytest.raises(lib.FAError) as e:
        fn(*args)
    return e.value.status


def fwd_args(**kw):
    a = dict(dtype=2, q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], B=1, H=2, M=128, N=128, D=64,
             causal=1, sm_scale=0.0, stream=None)
    a.update(kw)
    return list(a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1),
    (dict(lse=None), -1),
    (dict(dtype=7), -3),
    (dict(v=P[2] + 8), -4),
    (dict(lse=P[4] + 2), -4),
    (dict(B=0), -2),
    (dict(M=-64), -2),
    (dict(D=96), -6),
    (dict(D=48), -6),
    (dict(D=8), -6),
    (dict(causal=2), -6),
    (dict(sm_scale=-1.0), -6),
    (dict(sm_scale=float("nan")), -6),
    (dict(sm_scale=float("inf")), -6),
    (dict(B=1 << 20, H=1 << 20), -2),
])
def test_fa_fwd_rejects(kw, code):
    assert status(lib.fa_fwd, *fwd_args(**kw)) == code


def test_bwd_rejects_small_workspace():
    args = [2, P[0], P[1], P[2], P[3], P[5], P[4], P[6], P[7], P[8], P[9], 2 * 128 * 4 - 4,
            1, 2, 128, 128, 64, 1, 0.0, None]
    assert status(lib.fa_bwd, *args) == -5
    args[10] = None
    args[11] = 1 << 20
    assert status(lib.fa_bwd, *args) == -5
    args = [2, P[0], P[1], P[2], P[3], P[5], P[4], None, P[7], P[8], P[9], 1 << 20,
            1, 2, 128, 128, 64, 1, 0.0, None]
    assert status(lib.fa_bwd, *args) == -1
    # the variant with an LSE gradient: that gradient is optional but must be 4-byte aligned
    args = [2, P[0], P[1], P[2], P[3], P[5], P[4], P[4] + 2, P[6], P[7], P[8], P[9], 1 << 20,
            1, 2, 128, 128, 64, 1, 0.0, None]
    assert status(lib.fa_bwd_dlse, *args) == -4
    args[7] = None
    args[12] = 4
    assert status(lib.fa_bwd_dlse, *args) == -5


def test_noalloc_backward_rejects():
    f = lib.fa_bwd_noalloc
    ok = [2, P[0], P[1], P[2], P[3], P[4], P[5], P[6], P[7], P[8], 1, 2, 128, 128, 64, 1, 0.0]
    assert status(f, *ok[:7], None, *ok[8:]) == -1                    # dq missing
    assert status(f, *ok[:10], 1, 1024, 4096, 64, 64, 1, 0.0) == -6   # 2^22 rows: beyond the device array
    assert status(f, *ok[:14], 24, *ok[15:]) == -6                    # head dim outside the set
    assert status(f, 9, *ok[1:]) == -3


@pytest.mark.parametrize("D", [8, 48, 96, 512])
def test_head_dims_outside_the_set_rejected(D):
    # every entry point takes D in {16, 32, 64, 128, 256}, the tutorial's set
    assert status(lib.fa_fwd_jvp, 1, P[0], P[1], P[2], P[3], P[4], P[5], P[6], P[7], P[8],
                  1, 1, 64, 64, D, 0, 0.0) == -6
    assert status(lib.fa_bwd_dq, 2, P[0], P[1], P[2], P[3], P[4], P[5], P[6],
                  1, 1, 64, 64, D, 0, 0.0) == -6
    assert status(lib.pw_fwd, 2, P[0], P[1], P[2], P[3], P[4], P[5], P[6],
                  1, 1, 64, 64, D, 1, 0.0, 10) == -6
    args = [2, P[0], P[1], P[2], P[3], P[5], P[4], P[6], P[7], P[8], P[9], 1 << 20,
            1, 2, 128, 128, D, 1, 0.0, None]
    assert status(lib.fa_bwd, *args) == -6
    assert status(lib.fa_bwd_delta, 1, P[0], P[1], None, P[2], 1, 1, 64, D) == -6


def test_fp8_forward_rejects():
    f = lib.fa_fwd_fp8
    ok = [2, P[0], P[1], P[2], P[3], P[4], 1, 2, 64, 128, 128, 1, 0.0]
    assert status(f, *ok[:9], 100, *ok[10:]) == -6      # N not a multiple of 16
    assert status(f, *ok[:10], 32, *ok[11:]) == -6      # head dim 32 has no fp8 kernel
    assert status(f, 0, *ok[1:]) == -3                  # fp32 output is not offered
    assert status(f, *ok[:3], None, *ok[4:]) == -1
    assert status(f, 2, P[0] + 8, *ok[2:]) == -4


def test_step_entry_points_reject():
    assert status(lib.fa_bwd_delta, 1, P[0], P[1], None, None, 1, 1, 64, 64) == -1
    assert status(lib.fa_bwd_delta, 1, P[0], P[1], None, P[2], 1, 1, 64, 48) == -6
    assert status(lib.fa_bwd_delta, 1, P[0], P[1], P[3] + 1, P[2], 1, 1, 64, 64) == -4
    assert status(lib.fa_bwd_dkdv, 2, P[0], P[1], P[2], P[3], P[4], P[5], P[6], None,
                  1, 1, 64, 64, 64, 0, 0.0) == -1
    assert status(lib.fa_bwd_dq, 2, P[0], P[1], P[2], P[3], P[4], P[5], P[6],
                  1, 1, 64, 64, 64, 3, 0.0) == -6
    f = lib.fa_bwd_dq_delta
    ok = [2, P[0], P[1], P[2], P[3], P[4], P[5], None, P[6], P[7], 1, 1, 64, 64, 64, 0, 0.0]
    assert status(f, *ok[:4], None, *ok[5:]) == -1                 # o missing
    assert status(f, *ok[:8], None, *ok[9:]) == -1                 # delta missing
    assert status(f, *ok[:7], P[8] + 2, *ok[8:]) == -4             # dlse misaligned
    assert status(f, *ok[:14], 24, *ok[15:]) == -6                 # head dim outside the set
    assert status(f, *ok[:15], 2, *ok[16:]) == -6                  # causal not 0/1
    assert status(f, 5, *ok[1:]) == -3


def test_jvp_and_pw_reject():
    assert status(lib.fa_fwd_jvp, 1, P[0], P[1], P[2], None, P[4], P[5], P[6], P[7], P[8],
                  1, 1, 64, 64, 64, 0, 0.0) == -1
    assert status(lib.fa_fwd_jvp_tlse, 1, P[0], P[1], P[2], P[3], P[4], P[5], P[6], P[7], P[8], P[9] + 2,
                  1, 1, 64, 64, 64, 0, 0.0) == -4
    assert status(lib.fa_fwd_jvp_tlse, 1, P[0], P[1], P[2], P[3], P[4], P[5], P[6], None, P[8], P[9],
                  1, 1, 64, 64, 64, 0, 0.0) == -1
    assert status(lib.pw_bwd, 1, P[0], P[1], P[2], P[3], P[4], P[5], P[6], P[7], P[8], P[9], P[10],
                  P[11], P[12], P[13], 0, 1, 1, 64, 64, 64, 1, 0.0, 10) == -5
    assert status(lib.pw_bwd_dlse, 1, P[0], P[1], P[2], P[3], P[4], P[5], P[6], P[7], P[8] + 1, P[9], P[10],
                  P[11], P[12], P[13], P[14], 1 << 20, 1, 1, 64, 64, 64, 1, 0.0, 10) == -4


def test_merge_rejects():
    f = lib.resmerge_fwd
    ok = [2, P[0], P[1], P[2], P[3], P[4], P[5], 8, 64]
    assert status(f, *ok[:7], 8, 60, 1e-6) == -6          # D not a multiple of 8
    assert status(f, *ok[:7], 0, 64, 1e-6) == -2
    assert status(f, *ok, -1.0) == -6
    assert status(f, *ok, float("nan")) == -6
    assert status(f, 9, *ok[1:], 1e-6) == -3
    assert status(f, 2, P[0] + 4, *ok[2:], 1e-6) == -4
    b = lib.resmerge_bwd
    need = lib.resmerge_bwd_workspace_size(8, 64)
    args = [2, P[0], P[1], P[2], P[3], P[4], None, P[6], P[7], P[8], P[9], P[10], need - 4, 8, 64, 1e-6]
    assert status(b, *args) == -5
    args[12] = need
    args[7] = None  # gx
    assert status(b, *args) == -1
    args[7] = P[7]
    assert status(lib.resmerge_bwd_acc, *args, 2) == -6  # accumulate is 0 or 1
    args[12] = need - 4
    assert status(lib.resmerge_bwd_acc, *args, 1) == -5


def test_load_missing_library_raises():
    with pytest.raises(lib.FAError):
        lib.load("/nonexistent/libfa2tiles.so")


def test_lse_merge_rejects():
    f, b = lib.lse_merge_fwd, lib.lse_merge_bwd
    assert status(f, 2, P[0], P[1], P[2], P[3], 0, 100, 128) == -2      # S = 0
    assert status(f, 2, P[0], P[1], P[2], P[3], 4, 0, 128) == -2        # no rows
    assert status(f, 2, P[0], P[1], P[2], P[3], 4, 100, 60) == -6       # D not a multiple of 8
    assert status(f, 2, P[0], P[1], P[2], P[3], 4, 100, 8192) == -6     # D above 4096
    assert status(f, 5, P[0], P[1], P[2], P[3], 4, 100, 128) == -3      # dtype
    assert status(f, 2, None, P[1], P[2], P[3], 4, 100, 128) == -1
    assert status(f, 2, P[0] + 8, P[1], P[2], P[3], 4, 100, 128) == -4  # ys not 16-byte aligned
    assert status(b, 2, P[0], P[1], None, None, P[4], P[5], 4, 100, 128) == -1
    assert status(b, 2, P[0], P[1], P[2], P[3] + 2, P[4], P[5], 4, 100, 128) == -4  # gl misaligned
    assert status(b, 2, P[0], P[1], P[2], None, P[4], P[5], 4, 100, 12) == -6
