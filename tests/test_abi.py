"""The C ABI library: it loads, exports what include/moe.h declares, and its
host-side checks return the documented status codes (no GPU work)."""
import ctypes

import pytest

import sparse_mixture_experts_histogram_amd as moe
from sparse_mixture_experts_histogram_amd import _lib

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3


def desc(**kw):
    base = dict(T=64, d=256, E=8, k=2, ffn=512, n_shared=0, ffn_shared=0, dtype=1, y_dtype=0,
                path=0, flags=0)
    base.update(kw)
    return _lib.MoeDesc(**base)


def test_exports_every_declared_symbol():
    L = _lib.lib()
    names = _lib.header_symbols()
    assert {"moe_forward", "moe_route", "moe_dispatch", "moe_experts", "moe_combine",
            "moe_workspace_size", "moe_validate"} <= set(names)
    for n in names:
        assert hasattr(L, n), n
    assert L.moe_abi_version() == _lib.ABI_VERSION == 5


def test_desc_struct_size():
    assert ctypes.sizeof(_lib.MoeDesc) == 72
    assert _lib.MoeDesc.capacity_factor.offset == 64
    assert ctypes.sizeof(_lib.MoeMxScales) == 48


@pytest.mark.parametrize("kw,code", [
    ({}, OK),
    (dict(T=0), OK),
    (dict(T=-1), INVALID),
    (dict(k=0), INVALID),
    (dict(k=9), INVALID),
    (dict(E=0), INVALID),
    (dict(E=513, k=2), INVALID),
    (dict(E=64, k=33), INVALID),
    (dict(n_shared=9, ffn_shared=64), INVALID),
    (dict(n_shared=1, ffn_shared=0), INVALID),
    (dict(dtype=2), INVALID),
    (dict(y_dtype=5), INVALID),
    (dict(path=3), INVALID),
    (dict(flags=1), INVALID),                      # line rows with dense experts
    (dict(flags=1, expert_format=1), OK),
    (dict(flags=1, expert_format=2), OK),
    (dict(flags=2, expert_format=1), INVALID),
    (dict(flags=3, expert_format=2), INVALID),
    (dict(scoring=1), OK),
    (dict(scoring=2), INVALID),
    (dict(weighting=1), OK),
    (dict(weighting=-1), INVALID),
    (dict(capacity_factor=1.25), OK),
    (dict(capacity_factor=-0.5), INVALID),
    (dict(capacity_factor=float("nan")), INVALID),
    (dict(capacity_factor=float("inf")), INVALID),
    (dict(expert_format=1), OK),
    (dict(expert_format=2), OK),
    (dict(expert_format=3), INVALID),
    (dict(expert_format=1, dtype=0, d=64, ffn=64), INVALID),   # MXFP4 experts need bf16 x
    (dict(expert_format=2, dtype=0, d=64, ffn=64), INVALID),   # so do MXFP8 experts
    (dict(expert_format=2, d=8192, ffn=8192), OK),
    (dict(expert_format=2, d=8256), UNSUPPORTED),              # MXFP8: K up to 8192
    (dict(expert_format=2, ffn=8256), UNSUPPORTED),
    (dict(expert_format=2, n_shared=1, ffn_shared=8256), UNSUPPORTED),
    (dict(T=2 ** 30, k=2), INVALID),
    (dict(d=96), UNSUPPORTED),
    (dict(ffn=100), UNSUPPORTED),
    (dict(n_shared=1, ffn_shared=96), UNSUPPORTED),
    (dict(dtype=0, d=36, ffn=20), OK),
    (dict(dtype=0, d=34), UNSUPPORTED),
    (dict(E=512, k=32, d=64, ffn=64), OK),
    # bf16 operands are addressed with 32-bit byte offsets
    (dict(T=2 ** 20, d=2048, k=2, ffn=64), UNSUPPORTED),          # x: 4 GiB
    (dict(T=2 ** 18, d=64, k=2, ffn=4096), UNSUPPORTED),          # h: > 4 GiB
    (dict(T=64, d=32768, k=2, ffn=65536), UNSUPPORTED),           # one expert: 4 GiB
    (dict(T=2 ** 20, d=2048, k=2, ffn=64, dtype=0), OK),          # fp32 path: 64-bit offsets
])
def test_validate_codes(kw, code):
    assert moe.moe_validate(desc(**kw)) == code


def test_workspace_and_paths():
    d = desc(T=4096, d=4096, E=8, k=2, ffn=14336)
    ws = moe.moe_workspace_size(d)
    assert ws % 256 == 0
    # grouped rows, h and fp32 expert outputs dominate
    R = 4096 * 2
    assert ws > (R * 14336 * 2 + R * 4096 * 4)
    assert moe.moe_resolve_path(d) == "prefill"
    assert moe.moe_resolve_path(desc(T=16, d=4096, E=8, k=2, ffn=14336)) == "decode"
    assert moe.moe_resolve_path(desc(T=128, d=2880, E=128, k=4, ffn=2880)) == "decode"
    assert moe.moe_resolve_path(desc(T=512, d=2880, E=128, k=4, ffn=2880)) == "prefill"
    assert moe.moe_resolve_path(desc(T=4096, d=7168, E=256, k=8, ffn=2048, n_shared=1,
                                     ffn_shared=2048)) == "prefill"
    assert moe.moe_grouped_rows(desc(T=10, k=3, n_shared=2, ffn_shared=64)) == 50
    # MX-format experts always run the streaming kernels
    assert moe.moe_resolve_path(desc(T=4096, d=4096, E=8, k=2, ffn=14336,
                                     expert_format=1)) == "decode"
    assert moe.moe_resolve_path(desc(T=4096, d=4096, E=8, k=2, ffn=8192,
                                     expert_format=2)) == "decode"


def test_entry_points_reject_before_launch():
    L = _lib.lib()
    d = desc()
    n = ctypes.c_size_t(0)
    assert L.moe_workspace_size(ctypes.byref(d), None) == INVALID
    assert L.moe_workspace_size(ctypes.byref(d), ctypes.byref(n)) == OK
    # missing workspace
    assert L.moe_forward(ctypes.byref(d), *([None] * 13), None, 0, None) == WORKSPACE
    # fake (never dereferenced) aligned workspace, missing tensors
    fake = ctypes.c_void_p(1 << 20)
    assert L.moe_forward(ctypes.byref(d), *([None] * 13), fake, n.value, None) == INVALID
    assert L.moe_forward(ctypes.byref(d), *([None] * 13), fake, n.value - 1, None) == WORKSPACE
    misaligned = ctypes.c_void_p((1 << 20) + 16)
    assert L.moe_route(ctypes.byref(d), None, None, None, None, None, misaligned, n.value,
                       None) == WORKSPACE
    # token / weight arrays must be 16-byte aligned (fake pointers, never dereferenced)
    a = [ctypes.c_void_p((2 << 20) + 4096 * i) for i in range(6)]
    odd = ctypes.c_void_p((3 << 20) + 8)
    args = [a[0], a[1], None, a[2], a[3], a[4], None, None, None, a[5], None, None, None]
    for i in (0, 1, 3, 4, 5):
        bent = list(args)
        bent[i] = odd
        assert L.moe_forward(ctypes.byref(d), *bent, fake, n.value, None) == INVALID, i
    assert L.moe_route(ctypes.byref(d), odd, a[1], None, a[2], a[3], fake, n.value,
                       None) == INVALID
    bad = desc(k=0)
    assert L.moe_combine(ctypes.byref(bad), None, None, None, None, None, None) == INVALID
    assert L.moe_status_str(-3).startswith(b"MOE_ERR_WORKSPACE")


def test_zero_tokens_touch_nothing():
    L = _lib.lib()
    d = desc(T=0)
    assert L.moe_forward(ctypes.byref(d), *([None] * 13), None, 0, None) == OK
    assert L.moe_route(ctypes.byref(d), None, None, None, None, None, None, 0, None) == OK
    assert L.moe_combine(ctypes.byref(d), None, None, None, None, None, None) == OK


def test_noalloc_host_checks():
    """moe_forward_noalloc's checks run on the host before it touches a
    device: an invalid descriptor, an empty batch, and a layer whose
    workspace exceeds the library's scratch (MOE_ERR_TOO_LARGE)."""
    L = _lib.lib()
    args = [None] * 14
    assert L.moe_forward_noalloc(desc(k=0), *args) == INVALID
    assert L.moe_forward_noalloc(desc(T=0), *args) == OK
    big = desc(T=4096, d=4096, E=8, k=2, ffn=14336)
    n = ctypes.c_size_t()
    assert L.moe_workspace_size(big, ctypes.byref(n)) == OK
    assert n.value > _lib.NOALLOC_SCRATCH_BYTES
    assert L.moe_forward_noalloc(big, *args) == -5
    assert b"MOE_ERR_TOO_LARGE" in L.moe_status_str(-5)
    small = desc(T=512, d=2880, E=128, k=4, ffn=2880)
    assert L.moe_workspace_size(small, ctypes.byref(n)) == OK
    assert n.value <= _lib.NOALLOC_SCRATCH_BYTES


def test_mx_line_rows_host_logic():
    """Host side of MOE_FLAG_MX_LINE_ROWS (no GPU): code-row bytes rounded up
    to whole 128-byte lines, the format read from padded code tensors, an
    explicit format where padding makes it ambiguous, and the flag in the
    descriptor."""
    import torch
    from sparse_mixture_experts_histogram_amd import api
    assert api._row_bytes(2880, 2, False) == 1440
    assert api._row_bytes(2880, 2, True) == 1536
    assert api._row_bytes(2880, 1, True) == 2944
    assert api._row_bytes(4096, 2, True) == 2048   # already whole lines
    assert api._row_bytes(64, 2, True) == 128
    u8 = lambda *s: torch.empty(s, dtype=torch.uint8)
    def mxw(code_bytes, d=2880, **kw):
        return api.MxWeights(w_router=torch.empty((4, d), dtype=torch.bfloat16),
                             up=u8(4, 64, code_bytes), up_scale=u8(4, 64, d // 32),
                             gate=u8(4, 64, code_bytes), gate_scale=u8(4, 64, d // 32),
                             down=u8(4, d, 32), down_scale=u8(4, d, 2), **kw)
    assert mxw(1440).format == "mxfp4" and mxw(2880).format == "mxfp8"
    assert mxw(1536, line_rows=True).format == "mxfp4"
    assert mxw(2944, line_rows=True).format == "mxfp8"
    # d = 128: padded FP4 and FP8 rows are both 128 bytes; the explicit format decides
    assert mxw(128, d=128, line_rows=True, expert_format="mxfp4").format == "mxfp4"
    assert mxw(1536, line_rows=True).desc(8, 2).flags == _lib.FLAG_MX_LINE_ROWS
    assert mxw(1440).desc(8, 2).flags == 0
    L = _lib.lib()
    assert L.moe_validate(ctypes.byref(mxw(1536, line_rows=True).desc(8, 2))) == 0
