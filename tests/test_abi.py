"""The C-ABI library loads, exports every declared entry point and rejects bad
arguments before it touches the HIP runtime (CPU only: no call here is valid,
so nothing is ever launched)."""

import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")
LIB = os.path.join(ROOT, "exact_attention_110_amd", "libfa.so")

OK, EINVAL, EUNSUP, EWS, EHIP = 0, -1, -2, -3, -4
F32, F16, BF16 = 0, 1, 2


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.skip("libfa.so not built")
    import torch  # noqa: F401  (the library binds to the HIP runtime torch loads)
    from exact_attention_110_amd import binding
    return binding.load()


def test_header_constants_match_binding():
    from exact_attention_110_amd import binding
    src = open(HEADER).read()
    consts = dict(re.findall(r"#define (FA_[A-Z_0-9]+) \(?(-?\d+)\)?", src))
    assert int(consts["FA_F32"]) == binding.FA_F32
    assert int(consts["FA_F16"]) == binding.FA_F16
    assert int(consts["FA_BF16"]) == binding.FA_BF16
    assert int(consts["FA_MASK_BLOCK"]) == binding.MASK_BLOCK == 128
    assert [int(consts[k]) for k in ("FA_OK", "FA_ERR_INVALID_ARG", "FA_ERR_UNSUPPORTED",
                                     "FA_ERR_WORKSPACE", "FA_ERR_HIP")] == [OK, EINVAL, EUNSUP, EWS, EHIP]


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"fa_forward", "fa_backward", "fa_backward_workspace_size", "fa_backward_stage",
            "fa_status_string", "fa_version", "fa_forward_dropout", "fa_backward_dropout",
            "fa_backward_stage_dropout", "fa_forward_qk", "fa_backward_qk", "fa_forward_varlen",
            "fa_backward_varlen", "fa_forward_fp8"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for st in (OK, EINVAL, EUNSUP, EWS, EHIP, 12345):
        s = lib.fa_status_string(st)
        assert isinstance(s, bytes) and len(s) > 0
    assert lib.fa_status_string(EWS) != lib.fa_status_string(EINVAL)
    assert lib.fa_version() >= 100


P = ctypes.c_void_p
GOOD = P(1 << 20)       # 16- and 256-byte aligned stand-in address; never dereferenced
ODD = P((1 << 20) + 8)  # 8-byte aligned only


def fwd(lib, q=GOOD, k=GOOD, v=GOOD, o=GOOD, lse=GOOD, B=1, H=2, Hkv=1, N=256, d=64, scale=0.125,
        causal=1, mask=None, dtype=BF16):
    return lib.fa_forward(q, k, v, o, lse, B, H, Hkv, N, d, scale, causal, mask, dtype, None)


@pytest.mark.parametrize("bad", [
    dict(q=None), dict(k=None), dict(v=None), dict(o=None), dict(lse=None),
    dict(q=ODD), dict(o=ODD), dict(lse=P((1 << 20) + 2)),
    dict(B=0), dict(H=0), dict(Hkv=0), dict(N=0), dict(N=-5), dict(H=3, Hkv=2),
    dict(d=16), dict(d=96), dict(d=256), dict(dtype=3), dict(dtype=-1),
    dict(scale=float("nan")), dict(scale=float("inf")), dict(scale=-0.5),
    dict(B=70000), dict(B=1 << 16, H=1 << 15, N=8), dict(N=1 << 23, d=128), dict(N=(1 << 24) + 1, d=64),
])
def test_forward_rejects(lib, bad):
    assert fwd(lib, **bad) == EINVAL


def test_forward_mask_too_long_is_unsupported(lib):
    # masks are compacted into on-chip lists of 2048 blocks, so N <= 262144 with a mask;
    # the check returns before any launch
    assert fwd(lib, N=2049 * 128, mask=GOOD) == EUNSUP
    assert bwd(lib, N=2049 * 128, mask=GOOD) == EUNSUP
    assert fwd(lib, N=2049 * 128, mask=GOOD, d=16) == EINVAL   # bad arguments are reported first


def ws_size(lib, B=1, H=2, Hkv=1, N=256, d=64, dtype=BF16):
    return lib.fa_backward_workspace_size(B, H, Hkv, N, d, dtype)


def test_workspace_size_formula(lib):
    def r(x):
        return (x + 255) // 256 * 256
    for B, H, Hkv, N, d in [(1, 2, 1, 256, 64), (8, 12, 12, 1024, 64), (1, 16, 16, 16384, 128),
                            (1, 1, 1, 1, 32), (2, 3, 1, 77, 128)]:
        assert ws_size(lib, B, H, Hkv, N, d) == r(B * H * 2 * ((N + 127) // 128 * 128) * 4)
    # linear in N
    a, b = ws_size(lib, N=4096), ws_size(lib, N=8192)
    assert b == 2 * a
    assert ws_size(lib, dtype=F32) == 0
    assert ws_size(lib, d=48) == 0
    assert ws_size(lib, H=3, Hkv=2) == 0


def bwd(lib, stage=None, ws=GOOD, ws_bytes=None, dtype=BF16, N=256, d=64, mask=None, scale=0.125,
        dq=GOOD, lse=GOOD):
    if ws_bytes is None:
        ws_bytes = ws_size(lib, N=N, d=d) if dtype != F32 else 1 << 30
    args = [GOOD, GOOD, GOOD, GOOD, lse, GOOD, dq, GOOD, GOOD, 1, 2, 1, N, d, scale, 1, mask, dtype,
            ws, ws_bytes, None]
    if stage is None:
        return lib.fa_backward(*args)
    return lib.fa_backward_stage(stage, *args)


def test_backward_rejects(lib):
    assert bwd(lib, dtype=F32) == EUNSUP
    assert bwd(lib, ws=None) == EWS
    assert bwd(lib, ws=P((1 << 20) + 16)) == EWS
    assert bwd(lib, ws_bytes=ws_size(lib) - 1) == EWS
    assert bwd(lib, dq=None) == EINVAL
    assert bwd(lib, lse=None) == EINVAL
    assert bwd(lib, d=100) == EINVAL
    assert bwd(lib, scale=float("nan")) == EINVAL
    for st in (-1, 4, 99):
        assert bwd(lib, stage=st) == EINVAL
    assert bwd(lib, stage=1, ws=None) == EWS
    assert bwd(lib, stage=0, dtype=F32) == EUNSUP
    # stage 3 (dK/dV and dQ in one launch) only where fa_backward uses it
    assert bwd(lib, stage=3, d=128) == EUNSUP
    assert bwd(lib, stage=3, mask=GOOD) == EUNSUP
    assert bwd(lib, stage=3, ws=None) == EWS


def fwd_drop(lib, rate, dtype=BF16, d=64, seed=7):
    return lib.fa_forward_dropout(GOOD, GOOD, GOOD, GOOD, GOOD, 1, 2, 1, 256, d, 0.125, 1, None, dtype,
                                  rate, seed, None)


def bwd_drop(lib, rate, stage=None, dtype=BF16, seed=7):
    ws_bytes = ws_size(lib) if dtype != F32 else 1 << 30
    args = [GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 1, 2, 1, 256, 64, 0.125, 1, None, dtype,
            rate, seed, GOOD, ws_bytes, None]
    if stage is None:
        return lib.fa_backward_dropout(*args)
    return lib.fa_backward_stage_dropout(stage, *args)


@pytest.mark.parametrize("rate", [-0.1, 1.0, 1.5, float("nan"), float("inf"), float("-inf")])
def test_dropout_rate_rejected(lib, rate):
    """A dropout rate outside [0, 1) is an invalid argument, before any launch."""
    assert fwd_drop(lib, rate) == EINVAL
    assert bwd_drop(lib, rate) == EINVAL
    assert bwd_drop(lib, rate, stage=1) == EINVAL


def test_dropout_argument_order(lib):
    assert fwd_drop(lib, 0.5, dtype=F32) == EUNSUP     # no float32 dropout kernel
    assert fwd_drop(lib, 0.5, d=16) == EINVAL          # bad shape reported first
    assert bwd_drop(lib, 0.5, dtype=F32) == EUNSUP
    assert bwd_drop(lib, 0.2, stage=4) == EINVAL
    assert bwd_drop(lib, 0.2, stage=3) == EUNSUP       # no one-launch variant with dropout


def fwd_qk(lib, Nq=256, Nk=512, d=64, mask=None, dtype=BF16, rate=0.0, B=1, H=2, Hkv=1, wl=-1, wr=-1, alibi=None):
    return lib.fa_forward_qk(GOOD, GOOD, GOOD, GOOD, GOOD, B, H, Hkv, Nq, Nk, d, 0.125, 1, wl, wr, alibi, mask, dtype,
                             rate, 3, None)


def bwd_qk(lib, Nq=256, Nk=512, d=64, mask=None, dtype=BF16, ws_bytes=None, rate=0.0, wl=-1, wr=-1, alibi=None):
    if ws_bytes is None:
        ws_bytes = ws_size(lib, N=Nq, d=d)
    return lib.fa_backward_qk(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 1, 2, 1, Nq, Nk, d, 0.125, 1,
                              wl, wr, alibi, mask, dtype, rate, 3, GOOD, ws_bytes, None)


@pytest.mark.parametrize("bad", [dict(Nq=0), dict(Nk=0), dict(Nk=-3), dict(d=48), dict(rate=1.0),
                                 dict(Nq=1 << 23, d=128), dict(Nk=1 << 23, d=128), dict(B=1 << 16),
                                 dict(H=3, Hkv=2), dict(wl=-2), dict(wr=-7)])
def test_forward_qk_rejects(lib, bad):
    assert fwd_qk(lib, **bad) == EINVAL


def test_alibi_slopes_alignment(lib):
    """The slopes are float32 read on the device: a pointer off a 4-byte
    boundary is an invalid argument in every call that takes one."""
    for bad in (P((1 << 20) + 2), P((1 << 20) + 1)):
        assert fwd_qk(lib, alibi=bad) == EINVAL
        assert bwd_qk(lib, alibi=bad) == EINVAL
        assert fwd_var(lib, alibi=bad) == EINVAL
        assert bwd_var(lib, alibi=bad) == EINVAL
    # argument errors elsewhere still come first with well-aligned slopes
    assert fwd_qk(lib, alibi=GOOD, d=48) == EINVAL
    assert bwd_qk(lib, alibi=GOOD, dtype=F32) == EUNSUP


def test_window_limits_rejected_in_backward(lib):
    assert bwd_qk(lib, wl=-2) == EINVAL
    assert bwd_qk(lib, wr=-2) == EINVAL
    assert bwd_var(lib, wl=-5) == EINVAL


def test_qk_mask_and_workspace(lib):
    # a mask longer than the on-chip lists on either side is unsupported
    assert fwd_qk(lib, Nq=256, Nk=2049 * 128, mask=GOOD) == EUNSUP
    assert fwd_qk(lib, Nq=2049 * 128, Nk=256, mask=GOOD) == EUNSUP
    assert bwd_qk(lib, Nq=256, Nk=2049 * 128, mask=GOOD) == EUNSUP
    # the backward workspace follows the query length
    assert bwd_qk(lib, Nq=256, Nk=4096, ws_bytes=ws_size(lib, N=256) - 1) == EWS
    assert bwd_qk(lib, Nq=1000, Nk=10, ws_bytes=ws_size(lib, N=10)) == EWS
    assert bwd_qk(lib, dtype=F32) == EUNSUP


def fwd_var(lib, cu_q=GOOD, cu_k=GOOD, B=3, H=2, Hkv=1, tq=100, tk=200, mq=50, mk=90, d=64, dtype=BF16,
            rate=0.0, wl=-1, wr=-1, alibi=None):
    return lib.fa_forward_varlen(GOOD, GOOD, GOOD, GOOD, GOOD, cu_q, cu_k, B, H, Hkv, tq, tk, mq, mk, d, 0.125, 1,
                                 wl, wr, alibi, dtype, rate, 0, None)


def bwd_var(lib, cu_q=GOOD, cu_k=GOOD, mq=50, ws_bytes=None, dtype=BF16, tq=100, wl=-1, wr=-1, alibi=None):
    if ws_bytes is None:
        ws_bytes = ws_size(lib, B=3, N=mq)
    return lib.fa_backward_varlen(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, cu_q, cu_k, 3, 2, 1, tq,
                                  200, mq, 90, 64, 0.125, 1, wl, wr, alibi, dtype, 0.0, 0, GOOD, ws_bytes, None)


@pytest.mark.parametrize("bad", [dict(cu_q=None), dict(cu_k=None), dict(cu_q=P((1 << 20) + 2)),
                                 dict(cu_k=P((1 << 20) + 1)), dict(tq=-1), dict(tk=-5), dict(mq=0), dict(mk=0),
                                 dict(B=0), dict(d=16), dict(H=1 << 16, tq=1 << 15), dict(rate=-0.5),
                                 dict(dtype=7), dict(wl=-3), dict(wr=-2)])
def test_forward_varlen_rejects(lib, bad):
    assert fwd_var(lib, **bad) == EINVAL


def test_varlen_backward_checks(lib):
    assert bwd_var(lib, cu_q=None) == EINVAL
    assert bwd_var(lib, dtype=F32) == EUNSUP
    assert bwd_var(lib, ws_bytes=ws_size(lib, B=3, N=50) - 1) == EWS
    assert bwd_var(lib, mq=0) == EINVAL


def fwd8(lib, d=128, out=BF16, qd=1.0, kd=1.0, vd=1.0, N=256, q=GOOD, lse=GOOD):
    return lib.fa_forward_fp8(q, GOOD, GOOD, GOOD, lse, 1, 2, 1, N, d, 0.125, qd, kd, vd, 1, out, None)


@pytest.mark.parametrize("bad", [dict(out=F32), dict(out=7), dict(qd=0.0), dict(kd=-1.0), dict(vd=float("nan")),
                                 dict(qd=float("inf")), dict(N=0), dict(d=48), dict(q=None), dict(q=ODD),
                                 dict(lse=P((1 << 20) + 2))])
def test_fp8_rejects(lib, bad):
    assert fwd8(lib, **bad) == EINVAL


def test_fp8_head_sizes(lib):
    assert fwd8(lib, d=32) == EUNSUP   # the FP8 contraction takes 64 values at a time


def test_forward_kernel_rows(lib):
    """The library's forward-kernel choice, as bench.py reads it: 64 rows per
    wave at head size 128 when the 64-row grid (B * H * ceil(Nq / 256)
    workgroups) holds at least 256 and the rows have 4096 keys under a band
    (1024 without) or the grid holds at least 2048; 32 otherwise and
    always with a block mask or score bias, 0 (the float32 kernel) for FA_F32;
    negative statuses for arguments the forward calls reject."""
    rows = lambda *a: lib.fa_forward_kernel_rows(*a)  # noqa: E731
    # B, H, Hkv, Nq, Nk, d, causal, wl, wr, alibi, mask, dtype
    assert rows(1, 16, 16, 16384, 16384, 128, 1, -1, -1, 0, 0, BF16) == 64
    assert rows(1, 16, 16, 16384, 16384, 128, 1, -1, -1, 1, 0, BF16) == 32
    assert rows(1, 16, 16, 16384, 16384, 128, 1, -1, -1, 0, 1, BF16) == 32
    assert rows(4, 32, 8, 8192, 8192, 128, 1, -1, -1, 0, 0, BF16) == 64
    assert rows(8, 12, 12, 1024, 1024, 64, 1, -1, -1, 0, 0, BF16) == 32
    # head size 128, grids of at least 256 workgroups: from 4096 keys with a band
    # (causal, windows), from 1024 without; the shorter side decides
    assert rows(1, 8, 8, 8192, 4095, 128, 1, -1, -1, 0, 0, F16) == 32
    assert rows(1, 8, 8, 8192, 4096, 128, 1, -1, -1, 0, 0, F16) == 64
    assert rows(1, 16, 16, 4096, 4096, 128, 0, 256, -1, 0, 0, BF16) == 64  # a lower window edge is a band
    assert rows(4, 16, 16, 2048, 2048, 128, 0, -1, 64, 0, 0, BF16) == 32   # so is an upper one
    assert rows(4, 8, 8, 2048, 1023, 128, 0, -1, -1, 0, 0, F16) == 32
    assert rows(4, 8, 8, 2048, 1024, 128, 0, -1, -1, 0, 0, F16) == 64
    # smaller grids take the 32-row kernel whatever the length
    assert rows(1, 2, 2, 16384, 16384, 128, 1, -1, -1, 0, 0, BF16) == 32   # 128 workgroups
    assert rows(1, 4, 4, 16384, 16384, 128, 1, -1, -1, 0, 0, BF16) == 64   # 256
    assert rows(1, 16, 16, 2048, 2048, 128, 0, -1, -1, 0, 0, BF16) == 32   # 128
    assert rows(1, 8, 8, 4096, 4096, 128, 0, 256, -1, 0, 0, BF16) == 32    # 128
    # shorter rows in grids of 2048 workgroups or more
    assert rows(64, 16, 16, 512, 512, 128, 0, -1, -1, 0, 0, BF16) == 64    # 2048
    assert rows(32, 16, 16, 512, 512, 128, 0, -1, -1, 0, 0, BF16) == 32    # 1024
    assert rows(64, 16, 16, 2048, 2048, 128, 1, -1, -1, 0, 0, BF16) == 64  # 8192, causal
    assert rows(8, 16, 16, 2048, 2048, 128, 1, -1, -1, 0, 0, BF16) == 32   # 1024, causal
    assert rows(1, 16, 16, 16384, 16384, 64, 1, -1, -1, 0, 0, BF16) == 32  # head size 64: 32 rows
    assert rows(1, 1, 1, 512, 512, 32, 0, -1, -1, 0, 0, F32) == 0
    assert rows(1, 2, 1, 256, 256, 96, 1, -1, -1, 0, 0, BF16) == EINVAL
    assert rows(1, 2, 1, 256, 256, 64, 1, -2, -1, 0, 0, BF16) == EINVAL
    assert rows(1, 3, 2, 256, 256, 64, 1, -1, -1, 0, 0, BF16) == EINVAL


@pytest.mark.parametrize("r,kw,want", [
    (16, {}, EINVAL), (128, {}, EINVAL), (-32, {}, EINVAL),
    (64, dict(mask=GOOD), EUNSUP), (64, dict(alibi=GOOD), EUNSUP), (32, dict(dtype=F32), EUNSUP),
    (64, dict(q=None), EINVAL), (32, dict(d=96), EINVAL),
])
def test_forward_select_rejects(lib, r, kw, want):
    a = dict(q=GOOD, k=GOOD, v=GOOD, o=GOOD, lse=GOOD, mask=None, alibi=None, d=64, dtype=BF16)
    a.update(kw)
    st = lib.fa_forward_select(r, a["q"], a["k"], a["v"], a["o"], a["lse"], 1, 2, 1, 256, 256, a["d"], 0.125, 1,
                               -1, -1, a["alibi"], a["mask"], a["dtype"], 0.0, 0, None)
    assert st == want


def test_backward_launches(lib):
    """Stages fa_backward runs: 0, 3 (one launch for dK/dV and dQ) for d <= 64
    without dropout, slopes or mask; 0, 1, 2 otherwise."""
    n = lambda *a: lib.fa_backward_launches(*a)  # noqa: E731
    # B, H, Hkv, Nq, Nk, d, rate, alibi, mask, dtype
    assert n(8, 12, 12, 1024, 1024, 64, 0.0, 0, 0, BF16) == 2
    assert n(8, 12, 12, 1024, 1024, 64, 0.001, 0, 0, BF16) == 2   # rounds to no dropout
    assert n(8, 12, 12, 1024, 1024, 64, 0.1, 0, 0, BF16) == 3
    assert n(8, 12, 12, 1024, 1024, 64, 0.0, 1, 0, BF16) == 3
    assert n(1, 8, 8, 65536, 65536, 64, 0.0, 0, 1, F16) == 3
    assert n(1, 16, 16, 16384, 16384, 128, 0.0, 0, 0, BF16) == 3
    assert n(1, 1, 1, 512, 512, 32, 0.0, 0, 0, F32) == EUNSUP
    assert n(1, 2, 1, 256, 256, 64, 1.0, 0, 0, BF16) == EINVAL
    assert n(1, 2, 1, 256, 256, 96, 0.0, 0, 0, BF16) == EINVAL


def test_backward_noalloc_rejects(lib):
    """The allocation-free backward checks every argument before it touches
    the runtime: bad arguments as fa_backward, and sizes whose statistics
    exceed the scratch array (FA_NOALLOC_SCRATCH_BYTES) are unsupported."""
    src = open(HEADER).read()
    cap = eval(re.search(r"#define FA_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", src).group(0)
               .split(" ", 2)[2].replace("u", ""))
    assert cap == 16 << 20

    def call(B=1, H=2, Hkv=1, N=256, d=64, dtype=BF16, q=GOOD, lse=GOOD, mask=None, scale=0.125):
        return lib.fa_backward_noalloc(q, GOOD, GOOD, GOOD, lse, GOOD, GOOD, GOOD, GOOD, B, H, Hkv, N, d, scale, 1,
                                       mask, dtype, None)
    assert call(q=None) == EINVAL
    assert call(q=ODD) == EINVAL
    assert call(d=96) == EINVAL
    assert call(H=3, Hkv=2) == EINVAL
    assert call(scale=float("nan")) == EINVAL
    assert call(dtype=F32) == EUNSUP
    # 8 bytes of statistics per (b, h, padded row): 2^21 rows fit, one block more does not
    assert call(B=1, H=64, Hkv=1, N=65536, d=32) == EUNSUP
    assert call(B=1, H=32, Hkv=1, N=65536 + 128, d=32) == EUNSUP


def test_bitmask_rejects(lib):
    """Element-mask entry points: both mask arrays required, aligned, a tile
    count in range, tiles present when counted; all before any HIP call."""
    def fwdm(mask=GOOD, tile=GOOD, bits=GOOD, n=3, dtype=BF16):
        return lib.fa_forward_bitmask(GOOD, GOOD, GOOD, GOOD, GOOD, 1, 2, 1, 256, 256, 64, 0.125, 1, mask, tile,
                                      bits, n, dtype, 0.0, 0, None)

    def bwdm(mask=GOOD, tile=GOOD, bits=GOOD, n=3):
        return lib.fa_backward_bitmask(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 1, 2, 1, 256, 256, 64,
                                       0.125, 1, mask, tile, bits, n, BF16, 0.0, 0, None, 0, None)
    for f in (fwdm, bwdm):
        assert f(mask=None) == EINVAL
        assert f(tile=None) == EINVAL
        assert f(tile=P((1 << 20) + 2)) == EINVAL
        assert f(bits=None) == EINVAL
        assert f(bits=ODD) == EINVAL
        assert f(n=-1) == EINVAL
        assert f(n=(1 << 21) + 1) == EINVAL
    assert fwdm(dtype=5) == EINVAL
    # no workspace: the backward reaches the workspace check only after the mask checks pass
    assert bwdm(n=0, bits=None) == EWS
