"""The C ABI on the CPU: the library loads, exports every declared symbol,
and rejects invalid arguments before any HIP call (no device needed).

Pointers here are fake addresses: every call below fails validation, which
runs before the library touches HIP, so nothing is launched."""
import ctypes
import os
import shutil
import subprocess

import pytest

import transformer_row_normalization_amd as trn

F32, BF16 = trn.F32, trn.BF16
A = 0x10000          # fake, 16-byte aligned addresses
B = 0x20000000
C = 0x40000000


@pytest.fixture(scope="module")
def lib():
    return trn.lib()


def test_exports_every_header_symbol(lib):
    names = trn.header_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/fnorm.h but not exported"
    for n in ("fnorm_rms", "fnorm_layer", "fnorm_dual_head_rms"):
        assert n in names


def test_version_and_status_strings(lib):
    assert lib.fnorm_version() >= 100
    for s in range(8):
        assert lib.fnorm_status_string(s).startswith(b"FNORM_")
    assert b"unknown" in lib.fnorm_status_string(99)


@pytest.mark.parametrize("args,status", [
    # (x, w, y, rows, width, eps, dtype)
    ((A, B, C, 4, 8, 1e-6, 7), 4),                  # bad dtype
    ((A, B, C, -1, 8, 1e-6, F32), 2),               # rows < 0
    ((A, B, C, 4, 0, 1e-6, F32), 2),                # width 0
    ((A, B, C, 4, -3, 1e-6, BF16), 2),              # width < 0
    ((A, B, C, 1 << 40, 1 << 40, 1e-6, F32), 2),    # rows*width overflow
    ((A, B, C, 4, 8, -1e-6, F32), 3),               # eps < 0
    ((A, B, C, 4, 8, float("nan"), F32), 3),        # eps NaN
    ((A, B, C, 4, 8, float("inf"), F32), 3),        # eps inf
    ((None, B, C, 4, 8, 1e-6, F32), 1),             # null x
    ((A, None, C, 4, 8, 1e-6, F32), 1),             # null w
    ((A, B, None, 4, 8, 1e-6, F32), 1),             # null y
    ((A, B, A + 16, 4, 8, 1e-6, F32), 5),           # y partially overlaps x
    ((A, B, B - 16, 4, 8, 1e-6, F32), 5),           # y overlaps w
])
def test_rms_validation(lib, args, status):
    x, w, y, rows, width, eps, dt = args
    got = lib.fnorm_rms(x, w, y, rows, width, eps, dt, None)
    assert got == status, lib.fnorm_last_error()
    assert lib.fnorm_last_error().startswith(b"fnorm_rms: ")


def test_rows_zero_is_noop(lib):
    assert lib.fnorm_rms(None, None, None, 0, 8, 1e-6, F32, None) == 0
    assert lib.fnorm_layer(None, None, None, None, 0, 8, 1e-6, BF16, None) == 0
    assert lib.fnorm_dual_head_rms(None, None, None, None, None, None, 0, 0, 128, 1e-6, BF16,
                                   None) == 0
    assert lib.fnorm_last_error() == b""


def test_layer_validation(lib):
    assert lib.fnorm_layer(A, B, C, A + 32, 4, 8, 1e-5, F32, None) == 5   # y overlaps x
    assert lib.fnorm_layer(A, B, C - 8, C, 4, 8, 1e-5, F32, None) == 5    # y overlaps b
    assert lib.fnorm_layer(A, None, C, B, 4, 8, 1e-5, F32, None) == 1
    assert lib.fnorm_layer(A, B, None, C, 4, 8, -1.0, F32, None) == 3
    assert lib.fnorm_layer(A, B, None, C, 4, 8, 1e-5, 3, None) == 4
    assert lib.fnorm_last_error().startswith(b"fnorm_layer: ")


def test_dual_validation(lib):
    D, E, F, G = 0x1000000, 0x2000000, 0x3000000, 0x4000000
    # (q, k, qw, kw, qy, ky, q_rows, k_rows, head_dim)
    assert lib.fnorm_dual_head_rms(A, B, C, D, E, F, -1, 4, 128, 1e-6, BF16, None) == 2
    assert lib.fnorm_dual_head_rms(A, B, C, D, E, F, 4, -1, 128, 1e-6, BF16, None) == 2
    assert lib.fnorm_dual_head_rms(A, B, C, D, E, F, 4, 4, 0, 1e-6, BF16, None) == 2
    assert lib.fnorm_dual_head_rms(None, B, C, D, E, F, 4, 4, 128, 1e-6, BF16, None) == 1
    assert lib.fnorm_dual_head_rms(A, None, C, D, E, F, 4, 4, 128, 1e-6, BF16, None) == 1
    assert lib.fnorm_dual_head_rms(A, B, C, D, E, E + 64, 4, 4, 128, 1e-6, BF16, None) == 5
    assert lib.fnorm_dual_head_rms(A, B, C, D, E, B + 16, 4, 4, 128, 1e-6, BF16, None) == 5
    assert lib.fnorm_dual_head_rms(A, B, C, D, C, G, 4, 4, 128, 1e-6, BF16, None) == 5
    assert lib.fnorm_dual_head_rms(A, B, C, D, E, F, 4, 4, 128, float("nan"), BF16, None) == 3
    assert lib.fnorm_dual_head_rms(A, B, C, D, E, F, 4, 4, 128, 1e-6, 9, None) == 4
    assert lib.fnorm_last_error().startswith(b"fnorm_dual_head_rms: ")


def test_bench_copy_validation(lib):
    assert lib.fnorm_bench_copy(A, B, 24, None) == 2
    assert lib.fnorm_bench_copy(A + 4, B, 32, None) == 2
    assert lib.fnorm_bench_copy(A, A + 16, 64, None) == 5
    assert lib.fnorm_bench_copy(None, B, 64, None) == 1


def test_device_memory_query(lib):
    # with a device: positive figures; without one (this container): a clean
    # FNORM_ERR_LAUNCH that leaves the outputs alone
    vals = [ctypes.c_int(-1) for _ in range(3)]
    rc = lib.fnorm_device_memory(*(ctypes.byref(v) for v in vals))
    if rc == 0:
        assert all(v.value > 0 for v in vals)
    else:
        assert rc == 7 and all(v.value == -1 for v in vals)
        assert b"device query failed" in lib.fnorm_last_error()
    assert lib.fnorm_device_memory(None, None, None) == rc


def test_dispatch_table_choices():
    # the default kernels of the hot shapes use 16-byte packs, no predicate
    d = trn.describe(trn.OP_RMS, BF16, 8192)
    assert d.startswith("rms.bf16.vec8.") and ".exact" in d, d
    d = trn.describe(trn.OP_LAYER, BF16, 4096)
    assert d.startswith("layer.bf16.vec8.") and ".exact" in d, d
    d = trn.describe(trn.OP_DUAL, BF16, 128)
    assert d.startswith("dual.bf16.vec8.") and ".exact" in d, d
    for w in (1024, 768):
        d = trn.describe(trn.OP_RMS, F32, w)
        assert ".vec4." in d and ".exact" in d, d
    # misaligned data or ragged widths take the scalar-access kernels
    assert ".vec1." in trn.describe(trn.OP_RMS, BF16, 8192, aligned=False)
    assert ".vec1." in trn.describe(trn.OP_RMS, BF16, 8190)
    assert ".vec8." in trn.describe(trn.OP_RMS, BF16, 8184) and "masked" in trn.describe(
        trn.OP_RMS, BF16, 8184)
    # rows wider than the resident capacity take the multi-pass kernel
    assert ".wide." in trn.describe(trn.OP_LAYER, BF16, 1 << 20)
    assert ".wide." in trn.describe(trn.OP_RMS, F32, 40000)
    # the dual form has no multi-pass kernel
    assert trn.variant_count(trn.OP_DUAL, BF16, 1 << 20) == 0
    # every variant index describes; one past the end does not
    n = trn.variant_count(trn.OP_RMS, BF16, 4096)
    assert n >= 6 and n % 2 == 0
    names = {trn.describe(trn.OP_RMS, BF16, 4096, variant=i) for i in range(n)}
    assert len(names) == n
    with pytest.raises(trn.FnormError):
        trn.describe(trn.OP_RMS, BF16, 4096, variant=n)


def test_launch_policy_and_per_kind_order():
    # ragged widths on 16-byte packs default to a plain grid, non-temporal
    # with at most 3-4 workgroups resident per CU (".gridK")
    expect = {2560: 3, 3072: 3, 3584: 3, 5120: 3, 6144: 4, 7168: 4, 12288: 3}
    for w, k in expect.items():
        for op in (trn.OP_RMS, trn.OP_LAYER):
            d = trn.describe(op, BF16, w)
            if op == trn.OP_LAYER and w in (6144, 7168):
                # LayerNorm at 641-896 packs: two rows of 7 packs per lane
                assert ".vpt7.lpr128.blk256.masked.nt.grid3" in d, d
                continue
            assert ".vec8." in d and ".masked.nt." in d and d.endswith(f".grid{k}"), d
            # the other launch form of the same kernel is the odd variant
            d1 = trn.describe(op, BF16, w, variant=1)
            assert d1.rsplit(".", 1)[0] == d.rsplit(".", 1)[0] and ".persistent" in d1, d1
    assert trn.describe(trn.OP_RMS, BF16, 5120).startswith("rms.bf16.vec8.vpt5.lpr128.")
    # the shortest masked rows run without a limit
    assert trn.describe(trn.OP_RMS, BF16, 656).endswith(".masked.nt.grid")
    # 33-64 packs: 2 packs per lane on a plain grid; fewer: one pack, persistent
    for w in (264, 320, 504):
        assert trn.describe(trn.OP_LAYER, BF16, w) == "layer.bf16.vec8.vpt2.lpr32.blk256.masked.nt.grid"
    assert trn.describe(trn.OP_RMS, BF16, 200) == "rms.bf16.vec8.vpt1.lpr32.blk256.masked.persistent"
    for w in (18432, 24576):
        d = trn.describe(trn.OP_RMS, BF16, w)
        assert d.startswith("rms.bf16.vec8.vpt6.lpr512.blk512.masked.nt.") and d.endswith(".grid2"), d
    # LayerNorm with a bias there: exact shapes of 9 and 12 packs per lane
    assert trn.describe(trn.OP_LAYER, BF16, 18432) == "layer.bf16.vec8.vpt9.lpr256.blk256.exact.nt.grid"
    assert trn.describe(trn.OP_LAYER, BF16, 24576) == "layer.bf16.vec8.vpt12.lpr256.blk256.exact.nt.grid"
    # one row per 1024-thread workgroup: persistent first
    for w in (32768, 40000):
        d = trn.describe(trn.OP_RMS, BF16, w)
        assert ".lpr1024.blk1024.masked.nt." in d and ".persistent" in d, d
    assert ".vpt4.lpr1024.blk1024.masked.nt.persistent" in trn.describe(trn.OP_LAYER, BF16, 32768)
    # LayerNorm with a bias at 4097-8192 packs: 16 packs per lane, 512 threads
    for dt, w in ((BF16, 40000), (BF16, 65536), (F32, 32768)):
        d = trn.describe(trn.OP_LAYER, dt, w)
        assert ".vpt16.lpr512.blk512.masked.nt.persistent" in d, d
    # the 96-pack exact shape (bf16 768) defaults to a plain grid too
    assert trn.describe(trn.OP_LAYER, BF16, 768).endswith(".exact.nt.grid")
    # 1024 packs: the same shape, LayerNorm with non-temporal stores first,
    # the RMSNorm family with ordinary stores first; each list has it once
    for dt in (BF16, F32):
        w = 8192 if dt == BF16 else 4096
        ln = trn.describe(trn.OP_LAYER, dt, w)
        rms = trn.describe(trn.OP_RMS, dt, w)
        assert ".vpt4.lpr256.blk256.exact.nt.persistent2" in ln, ln
        assert ".vpt4.lpr256.blk256.exact.ntld.persistent2" in rms, rms
        for op in (trn.OP_RMS, trn.OP_LAYER, trn.OP_RMS_SWIGLU):
            n = trn.variant_count(op, dt, w)
            names = [trn.describe(op, dt, w, variant=i) for i in range(n)]
            assert len(set(names)) == n, names
            assert sum(".vpt4.lpr256.blk256.exact.nt.persistent2" in x for x in names) == 1
            assert sum(".vpt4.lpr256.blk256.exact.ntld.persistent2" in x for x in names) == 1
    # head vectors of 8-32 packs: exact shapes with non-temporal access on a plain grid
    assert trn.describe(trn.OP_DUAL, BF16, 64) == "dual.bf16.vec8.vpt1.lpr8.blk256.exact.nt.grid"
    assert trn.describe(trn.OP_DUAL, BF16, 128) == "dual.bf16.vec8.vpt2.lpr8.blk256.exact.nt.grid"
    assert trn.describe(trn.OP_DUAL, BF16, 256) == "dual.bf16.vec8.vpt2.lpr16.blk256.exact.nt.grid"
    assert trn.describe(trn.OP_DUAL, F32, 128) == "dual.f32.vec4.vpt2.lpr16.blk256.exact.nt.grid"
    assert trn.describe(trn.OP_RMS_SWIGLU, BF16, 256) == \
        "rmsgate.bf16.vec8.vpt1.lpr32.blk256.exact.nt.grid"
    assert trn.describe(trn.OP_DUAL, BF16, 192) == "dual.bf16.vec8.vpt3.lpr8.blk256.exact.nt.grid"
    assert trn.describe(trn.OP_LAYER, BF16, 576) == "layer.bf16.vec8.vpt9.lpr8.blk256.exact.nt.grid"
    assert trn.describe(trn.OP_LAYER, BF16, 640) == "layer.bf16.vec8.vpt5.lpr16.blk256.exact.nt.grid"
    assert trn.describe(trn.OP_DUAL, BF16, 128, variant=1) == "dual.bf16.vec8.vpt2.lpr8.blk256.exact.nt.persistent"
    # 4-8 packs per lane at 128, 256 and 2048 packs
    assert ".vpt4.lpr32." in trn.describe(trn.OP_LAYER, BF16, 1024)
    assert ".vpt4.lpr64." in trn.describe(trn.OP_RMS, F32, 1024)
    assert ".vpt8.lpr256." in trn.describe(trn.OP_LAYER, BF16, 16384)


def test_every_resident_width_has_a_kernel():
    for dt, vec in ((F32, 4), (BF16, 8)):
        for w in list(range(1, 300)) + [767, 768, 769, 1023, 1024, 4095, 4096, 8191, 8192]:
            for aligned in (True, False):
                assert trn.variant_count(trn.OP_RMS, dt, w, aligned) >= 4
                assert trn.variant_count(trn.OP_LAYER, dt, w, aligned) >= 4
                assert trn.variant_count(trn.OP_DUAL, dt, w, aligned) >= 2


def test_composed_validation(lib):
    W = 0x60000000
    need = lib.fnorm_composed_workspace_bytes(0, 4, 8)
    assert need >= 4 * 8 * 4
    assert lib.fnorm_composed_workspace_bytes(1, 4, 8) > need
    assert lib.fnorm_composed_workspace_bytes(2, 4, 8) == -1
    assert lib.fnorm_composed_workspace_bytes(0, 4, 0) == -1
    # workspace missing, too small, misaligned, overlapping
    assert lib.fnorm_rms_composed(A, B, C, 4, 8, 1e-6, F32, None, need, None) == 8
    assert lib.fnorm_rms_composed(A, B, C, 4, 8, 1e-6, F32, W, need - 1, None) == 8
    assert lib.fnorm_rms_composed(A, B, C, 4, 8, 1e-6, F32, W + 4, need, None) == 8
    assert lib.fnorm_rms_composed(A, B, C, 4, 8, 1e-6, F32, A, need, None) == 8
    # the common checks apply too
    assert lib.fnorm_rms_composed(A, B, C, -1, 8, 1e-6, F32, W, need, None) == 2
    assert lib.fnorm_layer_composed(A, B, None, A + 16, 4, 8, 1e-6, F32, W, 1 << 20, None) == 5
    assert lib.fnorm_layer_composed(A, None, None, C, 4, 8, 1e-6, F32, W, 1 << 20, None) == 1
    assert lib.fnorm_rms_composed(None, None, None, 0, 8, 1e-6, BF16, None, 0, None) == 0
    assert lib.fnorm_last_error() == b""


def test_rope_validation(lib):
    D, E, F = 0x1000000, 0x2000000, 0x3000000
    args = lambda **kw: {**dict(tokens=4, qh=2, kh=1, hd=128, eps=1e-6, dims=128, trad=0,
                                base=10000.0, scale=1.0, offset=0, freqs=None, dt=BF16), **kw}

    def call(**kw):
        a = args(**kw)
        return lib.fnorm_dual_head_rms_rope(A, B, C, D, E, F, a["tokens"], a["qh"], a["kh"],
                                            a["hd"], a["eps"], a["dims"], a["trad"], a["base"],
                                            a["scale"], a["offset"], a["freqs"], a["dt"], None)
    assert call(dims=127) == 2
    assert call(dims=0) == 2
    assert call(dims=130) == 2
    assert call(base=0.0) == 2
    assert call(base=float("nan")) == 2
    assert call(scale=float("inf")) == 2
    assert call(offset=-1) == 2
    assert call(tokens=-1) == 2
    assert call(qh=-2) == 2
    assert call(eps=-1.0) == 3
    assert call(dt=5) == 4
    assert call(hd=8192, dims=8192) == 6    # more pairs than the frequency tables carry
    assert call(tokens=0) == 0
    assert lib.fnorm_last_error() == b""
    # head shapes the kernel cannot serve are refused, not run
    assert trn.rope_variant_count(BF16, 1024, 128, False) == 0
    assert trn.rope_variant_count(BF16, 128, 128, False) >= 2
    assert trn.rope_variant_count(BF16, 128, 128, True) >= 2
    assert trn.describe_rope(BF16, 128, 128, False) == "ropesplit.bf16.vec8.vpt2.lpr8.blk256.exact.nt.grid"
    assert trn.describe_rope(BF16, 64, 64, False) == "ropesplit.bf16.vec8.vpt1.lpr8.blk256.exact.nt.persistent"
    assert trn.rope_variant_count(BF16, 128, 127, False) == 0


def test_strided_row_validation(lib):
    # (x, x_stride, w, y, y_stride, rows, width, eps, dtype, stream, variant)
    rms = lambda *a: lib.fnorm_rms_strided(*a, F32, None, 10 ** 6)
    assert rms(A, 7, B, C, 16, 4, 8, 1e-6) == 2           # x stride below width
    assert rms(A, 16, B, C, 7, 4, 8, 1e-6) == 2           # y stride below width
    assert rms(A, 1 << 60, B, C, 16, 4, 8, 1e-6) == 2     # stride overflow
    assert rms(A, 16, B, A, 8, 4, 8, 1e-6) == 5           # y = x but another stride
    assert rms(A, 16, B, A + 16, 16, 4, 8, 1e-6) == 5     # y rows shifted into x's rows
    # y rows in the gaps between x's rows are accepted: variant 10**6 then
    # fails as unsupported, which shows validation passed (nothing launches)
    assert rms(A, 16, B, A + 32, 16, 4, 8, 1e-6) == 6     # x at A+64r, y at A+32+64r
    assert rms(A, 32, B, A + 32, 32, 4, 8, 1e-6) == 6     # x at A+128r, y at A+32+128r
    assert rms(A, 16, B, A, 16, 4, 8, 1e-6) == 6          # in place, same stride
    assert rms(A, 16, B, C, 16, 1, 8, 1e-6) == 6          # one row: strides unused
    assert rms(A, 3, B, C, 3, 1, 8, 1e-6) == 6
    assert lib.fnorm_last_error().startswith(b"fnorm_rms_strided: ")
    # (x, x_stride, w, b, y, y_stride, rows, width, eps)
    lay = lambda *a: lib.fnorm_layer_strided(*a, F32, None, 10 ** 6)
    assert lay(A, 8, B, None, C, 4, 4, 8, 1e-5) == 2      # y stride below width
    assert lay(A, 16, B, A + 40, C, 16, 4, 8, 1e-5) == 6  # inputs may overlap each other
    assert lay(A, 16, B, C + 8, C, 16, 4, 8, 1e-5) == 5   # y overlaps b
    assert lib.fnorm_last_error().startswith(b"fnorm_layer_strided: ")


def test_packed_qkv_layout_is_accepted(lib):
    """q, k and v heads of one token packed back to back (one buffer, token
    stride (qh + 2 kh) * hd): normalizing q and k in place is legal; an
    output that lands on v, or on the other input, is not."""
    hd, qh, kh, tokens = 128, 8, 2, 16
    ts = (qh + 2 * kh) * hd                     # token stride, elements
    eb = 2                                      # bf16
    q = A
    k = A + qh * hd * eb
    v = A + (qh + kh) * hd * eb
    D, E = 0x1000000, 0x2000000                 # weights elsewhere

    def dual(qp, kp, qyp, kyp, qs=ts, ks=ts, qys=ts, kys=ts, variant=10 ** 6):
        return lib.fnorm_dual_head_rms_strided(qp, qs, kp, ks, D, E, qyp, qys, kyp, kys, tokens,
                                               qh, kh, hd, 1e-6, BF16, None, variant)
    assert dual(q, k, q, k) == 6                # in place inside the packed buffer
    assert dual(q, k, B, C, qys=qh * hd, kys=kh * hd) == 6   # to separate buffers
    assert dual(q, k, q, v) == 6                # ky into v's slots: v is not an input
    assert dual(q, k, v, k) == 5                # qy (8 heads) over v (2 heads) and beyond
    assert dual(q, k, k, k) == 5                # qy over k
    assert dual(q, k, q + 16, k) == 5           # qy shifted into q
    assert dual(q, k, q, k, qs=qh * hd - 1) == 2  # q token stride below its heads
    assert dual(q, k, q, k, ks=kh * hd - 1) == 2
    assert lib.fnorm_last_error().startswith(b"fnorm_dual_head_rms_strided: ")

    def rope(qp, kp, qyp, kyp, qs=ts, ks=ts, qys=ts, kys=ts):
        return lib.fnorm_dual_head_rms_rope_strided(
            qp, qs, kp, ks, D, E, qyp, qys, kyp, kys, tokens, qh, kh, hd, 1e-6, hd, 0, 10000.0,
            1.0, 0, None, BF16, None, 10 ** 6)
    assert rope(q, k, q, k) == 6
    assert rope(q, k, k, k) == 5
    assert rope(q, k, q, k, kys=kh * hd - 8) == 2
    assert lib.fnorm_last_error().startswith(b"fnorm_dual_head_rms_rope_strided: ")


def test_dual_heads_times_head_dim_overflow_without_tokens(lib):
    # no tokens: the row count is 0 and bounds nothing, so heads * head_dim
    # itself is checked before any stride is formed from it
    D, E = 0x1000000, 0x2000000
    huge = 1 << 60
    assert lib.fnorm_dual_head_rms_strided(A, 0, B, 0, D, E, C, 0, C + 64, 0, 0, huge, 1,
                                           1 << 10, 1e-6, BF16, None, -1) == 2
    assert b"overflows" in lib.fnorm_last_error()
    assert lib.fnorm_dual_head_rms_strided(A, 0, B, 0, D, E, C, 0, C + 64, 0, 0, 1, huge,
                                           1 << 10, 1e-6, BF16, None, -1) == 2
    assert lib.fnorm_dual_head_rms_rope_strided(A, 0, B, 0, D, E, C, 0, C + 64, 0, 0, huge, 1,
                                                1 << 10, 1e-6, 64, 0, 10000.0, 1.0, 0, None,
                                                BF16, None, -1) == 2
    # a shape that fits stays a no-op
    assert lib.fnorm_dual_head_rms_strided(None, 0, None, 0, None, None, None, 0, None, 0, 0, 32,
                                           8, 128, 1e-6, BF16, None, -1) == 0


def test_rms_swiglu_validation(lib):
    G = 0x60000000
    # (x, g, w, y, rows, width, eps, dtype, stream, variant)
    sw = lambda *a: lib.fnorm_rms_swiglu_v(*a, None, 10 ** 6)
    assert sw(A, None, B, C, 4, 8, 1e-6, BF16) == 1          # gate missing
    assert sw(A, G, B, C, -1, 8, 1e-6, BF16) == 2
    assert sw(A, G, B, C, 4, 8, -1.0, BF16) == 3
    assert sw(A, G, B, C, 4, 8, 1e-6, 7) == 4
    assert sw(A, G, B, G + 16, 4, 8, 1e-6, BF16) == 5         # y partly over the gate
    assert sw(A, G, B, G, 4, 8, 1e-6, BF16) == 6              # in place on the gate: accepted
    assert sw(A, G, B, A, 4, 8, 1e-6, BF16) == 6              # in place on x: accepted
    assert sw(None, None, None, None, 0, 8, 1e-6, BF16) == 0  # no rows: no-op
    st = lambda *a: lib.fnorm_rms_swiglu_strided(*a, BF16, None, 10 ** 6)
    # (x, xs, g, gs, w, y, ys, rows, width, eps)
    assert st(A, 8, G, 7, B, C, 8, 4, 8, 1e-6) == 2           # gate stride below width
    assert st(A, 16, A + 16, 16, B, C, 8, 4, 8, 1e-6) == 6    # x and g interleaved in one buffer
    assert lib.fnorm_last_error().startswith(b"fnorm_rms_swiglu_strided: ")
    assert trn.variant_count(trn.OP_RMS_SWIGLU, BF16, 128) >= 2
    assert trn.describe(trn.OP_RMS_SWIGLU, BF16, 128).startswith("rmsgate.bf16.vec8.vpt2.lpr8")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_header_compiles_as_c_and_links(tmp_path):
    """include/fnorm.h is valid C11; a C program links libfnorm.so and sees
    the documented status codes (validation only, no GPU needed)."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    exe = tmp_path / "abi_check"
    libdir = os.path.dirname(trn.LIB_PATH)
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic",
                    "-I", os.path.join(root, "include"),
                    os.path.join(root, "tests", "c_abi", "abi_check.c"), "-o", str(exe),
                    "-L", libdir, "-lfnorm", "-Wl,-rpath," + libdir], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stderr
    assert "c abi ok" in out.stdout


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """No fallback: without libfnorm.so every entry point raises."""
    monkeypatch.setattr(trn, "LIB_PATH", str(tmp_path / "absent" / "libfnorm.so"))
    monkeypatch.setattr(trn, "_lib", None)
    with pytest.raises(ImportError, match="missing"):
        trn.lib()
    with pytest.raises(ImportError):
        trn.variant_count(trn.OP_RMS, BF16, 128)


def test_prepare_rejects_host_tensors_and_restores_the_library():
    torch = pytest.importorskip("torch")
    x = torch.zeros(4, 8)
    with pytest.raises(ValueError, match="GPU"):
        trn.prepare(trn.rms_norm, x, torch.ones(8), 1e-6)
    assert isinstance(trn.lib(), ctypes.CDLL)      # no recorder left behind


def test_multi_pack_rope_kernels_serve_only_their_pairings():
    """Split-half kernels with two or four packs per lane carry compile-time
    pairings only: two packs serve full rotation only (the partner pack one
    away), four packs a partner one or two packs away.  Every (type,
    head_dim, dims) the library serves is enumerated over every variant it
    offers."""
    import re
    seen = {2: 0, 4: 0}
    for dt in (F32, BF16, trn.F16):
        for hd in list(range(2, 258, 2)) + [384, 512, 640, 768, 1024, 2048]:
            for dims in range(2, hd + 1, 2):
                for v in range(trn.rope_variant_count(dt, hd, dims, False)):
                    name = trn.describe_rope(dt, hd, dims, False, variant=v)
                    m = re.search(r"\.vec(\d+)\.vpt(\d+)\.lpr(\d+)\.", name)
                    vec, vpt, lpr = map(int, m.groups())
                    if vpt not in seen:
                        continue
                    seen[vpt] += 1
                    dp = dims // 2 // vec          # partner distance in packs
                    assert dp % lpr == 0, (dt, hd, dims, name)
                    dv = dp // lpr                 # ... in packs of one lane
                    assert dv == 1 if vpt == 2 else dv in (1, 2), (dt, hd, dims, name)
                    if vpt == 2:
                        assert dims == hd, (dt, hd, dims, name)
    assert seen[2] > 0 and seen[4] > 0


def test_dual_head_dim_limits():
    """The dual serves any head_dim up to 8192, and 16-byte-pack multiples
    with aligned pointers up to 65536 (2-byte types) / 32768 (fp32)."""
    for dt, cap, pack in ((trn.BF16, 65536, 8), (trn.F16, 65536, 8), (trn.F32, 32768, 4)):
        for hd in (1, 7, 100, 8191, 8192):
            for aligned in (True, False):
                assert trn.variant_count(trn.OP_DUAL, dt, hd, aligned=aligned) > 0, (dt, hd)
        for hd in (8192 + pack, 16384, cap):
            assert trn.variant_count(trn.OP_DUAL, dt, hd, aligned=True) > 0, (dt, hd)
            assert trn.variant_count(trn.OP_DUAL, dt, hd, aligned=False) == 0, (dt, hd)
        for hd in (8193, cap + pack, cap + 1):
            assert trn.variant_count(trn.OP_DUAL, dt, hd, aligned=True) == 0, (dt, hd)
