"""C-ABI contract on the CPU: the library loads, exports every function the
header declares, and rejects invalid arguments on the host before any HIP
call (no compute call is made here)."""
import ctypes
import os
import re

import pytest

import paged_kv_gqa_write_amd as pa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pa.h")

INVALID, UNSUPPORTED, OK = pa.PA_ERR_INVALID_ARG, pa.PA_ERR_UNSUPPORTED, pa.PA_OK
FAKE = 0x1000  # never dereferenced: every call below fails validation first


def header_functions():
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^(?:int|int64_t|void|const char\*)\s+(pa_\w+)\s*\(", text,
                                 flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return pa.load_library()


def test_header_declares_the_boundary():
    assert header_functions() == sorted(["pa_write_kv", "pa_decode", "pa_decode_reduce",
                                         "pa_decode_multi", "pa_decode_multi_reduce",
                                         "pa_decode_append",
                                         "pa_prefill", "pa_copy_blocks",
                                         "pa_decode_split_plan", "pa_decode_multi_split_plan",
                                         "pa_decode_split_plan_lens", "pa_decode_noalloc",
                                         "pa_status_string",
                                         "pa_prefix_index_create", "pa_prefix_index_destroy",
                                         "pa_prefix_index_size", "pa_prefix_index_match",
                                         "pa_prefix_index_insert", "pa_prefix_index_remove"])


def test_library_exports_every_declared_symbol(lib):
    for name in header_functions():
        assert hasattr(lib, name), name
    assert set(header_functions()) == set(pa.EXPORTED_SYMBOLS)


def test_exported_symbols_have_c_linkage():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", pa.library_path()],
                         capture_output=True, text=True, check=True).stdout
    names = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    for name in header_functions():
        assert name in names, name


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError, match="no fallback"):
        pa.load_library(str(tmp_path / "nope.so"))


def test_status_strings(lib):
    for code in (OK, INVALID, UNSUPPORTED, pa.PA_ERR_LAUNCH, pa.PA_ERR_NO_MEMORY,
                 pa.PA_ERR_TOO_LARGE):
        s = lib.pa_status_string(code).decode()
        assert s.startswith("PA_")
    assert "unknown" in lib.pa_status_string(7).decode()


def _write(lib, **kw):
    a = dict(k_new=FAKE, v_new=FAKE, slots=FAKE, kc=FAKE, vc=FAKE, T=4, hkv=8, d=128, bs=16,
             nb=64)
    a.update(kw)
    return lib.pa_write_kv(a["k_new"], a["v_new"], a["slots"], a["kc"], a["vc"], a["T"],
                           a["hkv"], a["d"], a["bs"], a["nb"], None)


def test_write_kv_validation(lib):
    assert _write(lib, T=-1) == INVALID
    assert _write(lib, hkv=0) == INVALID
    assert _write(lib, nb=-5) == INVALID
    assert _write(lib, d=96) == UNSUPPORTED
    assert _write(lib, bs=32) == UNSUPPORTED
    assert _write(lib, hkv=65536) == UNSUPPORTED
    assert _write(lib, k_new=None) == INVALID
    assert _write(lib, slots=None) == INVALID
    assert _write(lib, vc=None) == INVALID
    # zero tokens is a no-op that touches nothing (null pointers allowed)
    assert _write(lib, T=0, k_new=None, v_new=None, slots=None, kc=None, vc=None) == OK


def _decode(lib, **kw):
    a = dict(out=FAKE, po=FAKE, pl=FAKE, q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, ctx=FAKE, B=8,
             hq=32, hkv=8, d=128, bs=16, nb=4096, mb=72, ps=256, P=5, scale=0.088)
    a.update(kw)
    return lib.pa_decode(a["out"], a["po"], a["pl"], a["q"], a["kc"], a["vc"], a["bt"], a["ctx"],
                         a["B"], a["hq"], a["hkv"], a["d"], a["bs"], a["nb"], a["mb"], a["ps"],
                         a["P"], a["scale"], None)


def test_decode_validation(lib):
    assert _decode(lib, B=-1) == INVALID
    assert _decode(lib, hq=30) == INVALID           # not a multiple of Hkv
    assert _decode(lib, hq=0) == INVALID
    assert _decode(lib, hq=136, hkv=4) == UNSUPPORTED  # group 34 > 16
    assert _decode(lib, d=80) == UNSUPPORTED
    assert _decode(lib, bs=8) == UNSUPPORTED
    assert _decode(lib, mb=0) == INVALID
    assert _decode(lib, ps=100) == INVALID          # not a multiple of 16
    assert _decode(lib, ps=0) == INVALID
    assert _decode(lib, P=0) == INVALID
    assert _decode(lib, scale=float("nan")) == INVALID
    assert _decode(lib, scale=float("inf")) == INVALID
    assert _decode(lib, scale=-0.5) == INVALID
    assert _decode(lib, q=None) == INVALID
    assert _decode(lib, bt=None) == INVALID
    assert _decode(lib, ctx=None) == INVALID
    assert _decode(lib, P=1, out=None) == INVALID
    assert _decode(lib, P=4, po=None) == INVALID
    assert _decode(lib, P=4, pl=None) == INVALID
    assert _decode(lib, P=0x40000000, hkv=8, B=8) == UNSUPPORTED  # grid too large
    assert _decode(lib, B=0, q=None, kc=None, vc=None, bt=None, ctx=None, out=None) == OK


def _reduce(lib, **kw):
    a = dict(out=FAKE, po=FAKE, pl=FAKE, ctx=FAKE, B=8, hq=32, d=128, ps=256, P=5)
    a.update(kw)
    return lib.pa_decode_reduce(a["out"], a["po"], a["pl"], a["ctx"], a["B"], a["hq"], a["d"],
                                a["ps"], a["P"], None)


def test_reduce_validation(lib):
    assert _reduce(lib, B=-2) == INVALID
    assert _reduce(lib, hq=0) == INVALID
    assert _reduce(lib, d=32) == UNSUPPORTED
    assert _reduce(lib, ps=24) == INVALID
    assert _reduce(lib, P=0) == INVALID
    assert _reduce(lib, out=None) == INVALID
    assert _reduce(lib, po=None) == INVALID
    assert _reduce(lib, pl=None) == INVALID
    assert _reduce(lib, B=0, out=None, po=None, pl=None) == OK


def _append(lib, **kw):
    a = dict(out=FAKE, po=FAKE, pl=FAKE, q=FAKE, kn=FAKE, vn=FAKE, kc=FAKE, vc=FAKE, bt=FAKE,
             ctx=FAKE, B=8, hq=32, hkv=8, d=128, bs=16, nb=4096, mb=72, ps=288, P=4,
             scale=0.088)
    a.update(kw)
    return lib.pa_decode_append(a["out"], a["po"], a["pl"], a["q"], a["kn"], a["vn"], a["kc"],
                                a["vc"], a["bt"], a["ctx"], a["B"], a["hq"], a["hkv"], a["d"],
                                a["bs"], a["nb"], a["mb"], a["ps"], a["P"], a["scale"], None)


def test_decode_append_validation(lib):
    assert _append(lib, B=-1) == INVALID
    assert _append(lib, hq=31) == INVALID
    assert _append(lib, hq=136, hkv=4) == UNSUPPORTED
    assert _append(lib, d=72) == UNSUPPORTED
    assert _append(lib, bs=8) == UNSUPPORTED
    assert _append(lib, mb=0) == INVALID
    assert _append(lib, ps=20) == INVALID
    assert _append(lib, P=0) == INVALID
    assert _append(lib, scale=float("inf")) == INVALID
    assert _append(lib, kn=None) == INVALID
    assert _append(lib, vn=None) == INVALID
    assert _append(lib, kc=None) == INVALID
    assert _append(lib, P=1, out=None) == INVALID
    assert _append(lib, P=4, pl=None) == INVALID
    assert _append(lib, P=0x40000000) == UNSUPPORTED
    assert _append(lib, B=0, q=None, kn=None, vn=None, kc=None, vc=None, bt=None, ctx=None,
                   out=None) == OK


def _multi(lib, **kw):
    a = dict(out=FAKE, po=FAKE, pl=FAKE, q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, ctx=FAKE, B=4, T=8,
             hq=32, hkv=8, d=128, bs=16, nb=4096, mb=72, ps=288, P=4, scale=0.088)
    a.update(kw)
    return lib.pa_decode_multi(a["out"], a["po"], a["pl"], a["q"], a["kc"], a["vc"], a["bt"],
                               a["ctx"], a["B"], a["T"], a["hq"], a["hkv"], a["d"], a["bs"],
                               a["nb"], a["mb"], a["ps"], a["P"], a["scale"], None)


def test_decode_multi_validation(lib):
    assert _multi(lib, T=0) == INVALID
    assert _multi(lib, T=-3) == INVALID
    assert _multi(lib, T=17) == UNSUPPORTED          # more than 16 query tokens
    assert _multi(lib, B=-1) == INVALID
    assert _multi(lib, hq=30) == INVALID
    assert _multi(lib, hq=136, hkv=4) == UNSUPPORTED
    assert _multi(lib, d=96) == UNSUPPORTED
    assert _multi(lib, bs=32) == UNSUPPORTED
    assert _multi(lib, mb=0) == INVALID
    assert _multi(lib, ps=40) == INVALID
    assert _multi(lib, P=0) == INVALID
    assert _multi(lib, scale=float("nan")) == INVALID
    assert _multi(lib, scale=-1.0) == INVALID
    assert _multi(lib, q=None) == INVALID
    assert _multi(lib, ctx=None) == INVALID
    assert _multi(lib, P=1, out=None) == INVALID
    assert _multi(lib, P=4, po=None) == INVALID
    assert _multi(lib, P=0x10000000, B=8) == UNSUPPORTED  # grid too large
    assert _multi(lib, B=0x1000000, T=16, hq=256, hkv=16) == UNSUPPORTED  # rows overflow int32
    assert _multi(lib, B=0, q=None, kc=None, vc=None, bt=None, ctx=None, out=None) == OK


def _multi_reduce(lib, **kw):
    a = dict(out=FAKE, po=FAKE, pl=FAKE, ctx=FAKE, B=4, T=8, hq=32, d=128, ps=288, P=4)
    a.update(kw)
    return lib.pa_decode_multi_reduce(a["out"], a["po"], a["pl"], a["ctx"], a["B"], a["T"],
                                      a["hq"], a["d"], a["ps"], a["P"], None)


def test_decode_multi_reduce_validation(lib):
    assert _multi_reduce(lib, T=0) == INVALID
    assert _multi_reduce(lib, T=17) == UNSUPPORTED
    assert _multi_reduce(lib, B=-1) == INVALID
    assert _multi_reduce(lib, hq=0) == INVALID
    assert _multi_reduce(lib, d=48) == UNSUPPORTED
    assert _multi_reduce(lib, ps=8) == INVALID
    assert _multi_reduce(lib, P=0) == INVALID
    assert _multi_reduce(lib, out=None) == INVALID
    assert _multi_reduce(lib, pl=None) == INVALID
    assert _multi_reduce(lib, B=0x1000000, T=16, hq=256) == UNSUPPORTED
    assert _multi_reduce(lib, B=0, out=None, po=None, pl=None) == OK


def _copy(lib, **kw):
    a = dict(dk=FAKE, dv=FAKE, dnb=4096, di=FAKE, sk=FAKE, sv=FAKE, snb=1024, si=None, n=1024,
             hkv=8, d=128, bs=16)
    a.update(kw)
    return lib.pa_copy_blocks(a["dk"], a["dv"], a["dnb"], a["di"], a["sk"], a["sv"], a["snb"],
                              a["si"], a["n"], a["hkv"], a["d"], a["bs"], None)


def test_copy_blocks_validation(lib):
    assert _copy(lib, n=-1) == INVALID
    assert _copy(lib, hkv=0) == INVALID
    assert _copy(lib, hkv=65536) == UNSUPPORTED
    assert _copy(lib, dnb=-1) == INVALID
    assert _copy(lib, snb=-2) == INVALID
    assert _copy(lib, d=100) == UNSUPPORTED
    assert _copy(lib, bs=32) == UNSUPPORTED
    assert _copy(lib, hkv=70000) == UNSUPPORTED
    assert _copy(lib, n=0x40000000) == UNSUPPORTED        # grid of 2n workgroups too large
    assert _copy(lib, dk=None) == INVALID
    assert _copy(lib, sv=None) == INVALID
    assert _copy(lib, dk=FAKE + 8) == INVALID             # pools must be 16-byte aligned
    assert _copy(lib, sv=FAKE + 4) == INVALID
    # zero copies is a no-op that touches nothing
    assert _copy(lib, n=0, dk=None, dv=None, sk=None, sv=None, di=None) == OK


def _prefill(lib, **kw):
    a = dict(out=FAKE, q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, cu=FAKE, pre=FAKE, S=4, tq=4096,
             mq=1024, hq=32, hkv=8, d=128, bs=16, nb=4096, mb=96, scale=0.088)
    a.update(kw)
    return lib.pa_prefill(a["out"], a["q"], a["kc"], a["vc"], a["bt"], a["cu"], a["pre"], a["S"],
                          a["tq"], a["mq"], a["hq"], a["hkv"], a["d"], a["bs"], a["nb"], a["mb"],
                          a["scale"], None)


def test_prefill_validation(lib):
    assert _prefill(lib, S=-1) == INVALID
    assert _prefill(lib, tq=-1) == INVALID
    assert _prefill(lib, mq=-1) == INVALID
    assert _prefill(lib, hq=33) == INVALID
    assert _prefill(lib, d=512) == UNSUPPORTED
    assert _prefill(lib, bs=64) == UNSUPPORTED
    assert _prefill(lib, hq=65536, hkv=65536) == UNSUPPORTED  # 32-bit block offsets
    assert _prefill(lib, mb=0) == INVALID
    assert _prefill(lib, scale=float("nan")) == INVALID
    assert _prefill(lib, scale=-1.0) == INVALID
    assert _prefill(lib, cu=None) == INVALID
    assert _prefill(lib, out=None) == INVALID
    assert _prefill(lib, S=0) == OK
    assert _prefill(lib, tq=0, q=None, out=None) == OK


def plan(lib, B, hkv, ctx, cus=256):
    ps, npart = ctypes.c_int32(), ctypes.c_int32()
    st = lib.pa_decode_split_plan(B, hkv, ctx, cus, ctypes.byref(ps), ctypes.byref(npart))
    return st, ps.value, npart.value


@pytest.mark.parametrize("B,hkv,ctx", [(8, 8, 1152), (64, 8, 1152), (4, 8, 8192), (8, 2, 8192),
                                       (2, 2, 50), (1, 1, 1), (1, 1, 0), (300, 8, 100000)])
def test_split_plan_covers_context(lib, B, hkv, ctx):
    st, ps, npart = plan(lib, B, hkv, ctx)
    assert st == OK
    assert ps > 0 and ps % 16 == 0 and npart >= 1
    assert ps * npart >= max(ctx, 1)
    if npart > 1:
        assert ps % 32 == 0 and ps >= 128
        assert ps * (npart - 1) < ctx        # no partition is empty at max context


def test_split_plan_fills_the_gpu(lib):
    # small batches are split into about one workgroup per CU
    assert plan(lib, 8, 8, 1152) == (OK, 288, 4)      # Qwen3-4B batch 8: 256 workgroups
    assert plan(lib, 4, 8, 8192) == (OK, 1024, 8)     # batch 4 at 8192: 256 workgroups
    assert plan(lib, 8, 2, 8192) == (OK, 512, 16)     # 2 KV heads, 8192: 256 workgroups
    st, ps, npart = plan(lib, 64, 8, 1152)
    assert npart == 1                       # 512 items already cover 256 CUs
    st, ps, npart = plan(lib, 2, 2, 50)
    assert npart == 1                       # short contexts are never split below 128


def test_split_plan_validation(lib):
    ps, npart = ctypes.c_int32(), ctypes.c_int32()
    assert lib.pa_decode_split_plan(1, 1, 10, 256, None, ctypes.byref(npart)) == INVALID
    assert lib.pa_decode_split_plan(-1, 1, 10, 256, ctypes.byref(ps), ctypes.byref(npart)) == INVALID
    assert lib.pa_decode_split_plan(1, 0, 10, 256, ctypes.byref(ps), ctypes.byref(npart)) == INVALID
    assert lib.pa_decode_split_plan(1, 1, 10, 0, ctypes.byref(ps), ctypes.byref(npart)) == INVALID


def mplan(lib, B, T, hq, hkv, ctx, cus=256):
    ps, npart = ctypes.c_int32(), ctypes.c_int32()
    st = lib.pa_decode_multi_split_plan(B, T, hq, hkv, ctx, cus, ctypes.byref(ps),
                                        ctypes.byref(npart))
    return st, ps.value, npart.value


def _launch_workgroups(B, T, hq, hkv, npart, cus=256):
    """Workgroups pa_decode_multi launches (its tile rule, restated)."""
    tiles = -(-(T * (hq // hkv)) // 16)
    items = B * hkv * npart
    two = tiles >= 2 and items * ((tiles + 1) // 2) >= cus
    return items * (((tiles + 1) // 2) if two else tiles)


def test_multi_split_plan_measured_shapes(lib):
    # Qwen3-4B verify, T = 8, longest context 1110: the partition sizes that
    # were fastest in a sweep of forced sizes on MI355X (batch 1: 128;
    # batch 4: 288, one tile per workgroup in two column chunks; batch 8:
    # 288, two tiles per wave).
    assert mplan(lib, 1, 8, 32, 8, 1110) == (OK, 128, 9)
    assert mplan(lib, 4, 8, 32, 8, 1110) == (OK, 288, 4)
    assert mplan(lib, 8, 8, 32, 8, 1110) == (OK, 288, 4)
    # one token per sequence: the batch-8 decode plan
    assert mplan(lib, 8, 1, 32, 8, 1110) == (OK, 288, 4)


@pytest.mark.parametrize("B,T,hq,hkv,ctx", [(1, 8, 32, 8, 1110), (4, 8, 32, 8, 1110),
                                            (8, 8, 32, 8, 1110), (8, 8, 16, 2, 8192),
                                            (2, 3, 4, 2, 50), (1, 16, 16, 1, 1), (1, 1, 8, 8, 0),
                                            (64, 2, 64, 8, 1152), (3, 5, 12, 4, 3000)])
def test_multi_split_plan_covers_context_within_the_cus(lib, B, T, hq, hkv, ctx):
    st, ps, npart = mplan(lib, B, T, hq, hkv, ctx)
    assert st == OK
    assert ps > 0 and ps % 16 == 0 and npart >= 1
    assert ps * npart >= max(ctx, 1)
    if npart > 1:
        assert ps % 32 == 0 and ps >= 128
        assert ps * (npart - 1) < ctx
        assert _launch_workgroups(B, T, hq, hkv, npart) <= 256


def test_multi_split_plan_validation(lib):
    ps, npart = ctypes.c_int32(), ctypes.c_int32()
    f = lib.pa_decode_multi_split_plan
    assert f(1, 1, 8, 8, 10, 256, None, ctypes.byref(npart)) == INVALID
    assert f(1, 0, 8, 8, 10, 256, ctypes.byref(ps), ctypes.byref(npart)) == INVALID
    assert f(1, 1, 6, 4, 10, 256, ctypes.byref(ps), ctypes.byref(npart)) == INVALID
    assert f(-1, 1, 8, 8, 10, 256, ctypes.byref(ps), ctypes.byref(npart)) == INVALID
    assert f(1, 1, 8, 8, -1, 256, ctypes.byref(ps), ctypes.byref(npart)) == INVALID
    assert f(1, 1, 8, 8, 10, 0, ctypes.byref(ps), ctypes.byref(npart)) == INVALID


def test_partition_cover_must_fit_int32(lib):
    # num_partitions * partition_size indexes positions with 32-bit integers
    # in the kernels: a cover of 2^36 tokens passes every other check.
    big = dict(ps=1 << 24, P=4096)
    assert _decode(lib, **big) == UNSUPPORTED
    assert _append(lib, **big) == UNSUPPORTED
    assert _multi(lib, **big) == UNSUPPORTED
    assert _reduce(lib, **big) == UNSUPPORTED
    assert _multi_reduce(lib, **big) == UNSUPPORTED
    assert _decode(lib, ps=1 << 26, P=32) == UNSUPPORTED      # exactly 2^31


def lplan(lib, hkv, lens, cus=256):
    arr = (ctypes.c_int32 * max(len(lens), 1))(*lens)
    ps, npart = ctypes.c_int32(), ctypes.c_int32()
    st = lib.pa_decode_split_plan_lens(len(lens), hkv, arr if lens else None, cus,
                                       ctypes.byref(ps), ctypes.byref(npart))
    return st, ps.value, npart.value


def _live(hkv, lens, ps):
    return hkv * sum(-(-c // ps) for c in lens if c > 0)


def test_split_plan_lens_mixed_batch(lib):
    # One 8192-token request among seven of ~1100 (8 KV heads): the longest
    # alone gives 4 x 2048 (the long sequence's 32 workgroups each stream
    # 2048 tokens); from the lengths, 15 x 576 keeps 232 live workgroups.
    lens = [8192, 1084, 1038, 1106, 1094, 1090, 1110, 1061]
    assert lplan(lib, 8, lens) == (OK, 576, 15)
    assert _live(8, lens, 576) == 232 and _live(8, lens, 544) > 256
    # hybrid contexts 4097 / 8192 (2 KV heads): 20 x 416 is the smallest
    # partition within the CUs, but 416 > 2/3 * 512 -- the plan from the
    # longest context (16 x 512, one dispatch round) is kept.
    assert lplan(lib, 2, [4097, 8192] * 4) == (OK, 512, 16)


def test_split_plan_lens_matches_uniform_plans(lib):
    # with equal (or nearly equal) lengths the plan is the maximum-based one
    assert lplan(lib, 8, [1084, 1038, 1106, 1094, 1090, 1110, 1061, 1068]) == (OK, 288, 4)
    assert lplan(lib, 8, [8192] * 4) == (OK, 1024, 8)
    assert lplan(lib, 8, [1100] * 64)[2] == 1          # 512 live items: no split
    assert lplan(lib, 2, [50, 37]) == (OK, 64, 1)      # short contexts: one piece
    assert lplan(lib, 8, [100] * 70 + [8192]) == plan(lib, 71, 8, 8192)   # > 64 sequences


@pytest.mark.parametrize("hkv,lens", [(2, [4097, 8192] * 4), (8, [100, 9000, 20, 3000]),
                                      (1, [1, 2, 3, 100000]), (4, [0, -5, 700, 0]),
                                      (8, [1152] * 8 + [64] * 8), (2, [128]),
                                      (8, [8192, 100, 100, 100])])
def test_split_plan_lens_shorter_partition_within_the_cus(lib, hkv, lens):
    st, ps, npart = lplan(lib, hkv, lens)
    top = max(max(lens), 1)
    _, mps, mnp = plan(lib, len(lens), hkv, top)
    assert st == OK
    assert ps > 0 and ps % 16 == 0 and ps * npart >= top
    if (ps, npart) != (mps, mnp):
        # taken from the lengths: at most one live workgroup per CU, the
        # smallest such partition, and at most 2/3 of the longest-based one
        assert npart > 1 and ps % 32 == 0 and ps >= 128
        assert ps * (npart - 1) < top
        assert _live(hkv, lens, ps) <= 256
        assert ps == 128 or _live(hkv, lens, ps - 32) > 256
        assert 3 * ps <= 2 * mps


def test_split_plan_lens_validation(lib):
    ps, npart = ctypes.c_int32(), ctypes.c_int32()
    f = lib.pa_decode_split_plan_lens
    arr = (ctypes.c_int32 * 2)(10, 20)
    assert f(2, 1, None, 256, ctypes.byref(ps), ctypes.byref(npart)) == INVALID
    assert f(2, 0, arr, 256, ctypes.byref(ps), ctypes.byref(npart)) == INVALID
    assert f(2, 1, arr, 0, ctypes.byref(ps), ctypes.byref(npart)) == INVALID
    assert f(-1, 1, arr, 256, ctypes.byref(ps), ctypes.byref(npart)) == INVALID
    assert f(2, 1, arr, 256, None, ctypes.byref(npart)) == INVALID
    assert lplan(lib, 4, []) == (OK, 16, 1)             # empty batch


def _noalloc(lib, **kw):
    a = dict(out=FAKE, q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, ctx=FAKE, B=8, hq=32, hkv=8, d=128,
             bs=16, nb=4096, mb=72, ps=288, P=4, scale=0.088)
    a.update(kw)
    return lib.pa_decode_noalloc(a["out"], a["q"], a["kc"], a["vc"], a["bt"], a["ctx"], a["B"],
                                 a["hq"], a["hkv"], a["d"], a["bs"], a["nb"], a["mb"], a["ps"],
                                 a["P"], a["scale"], None)


def test_decode_noalloc_validation(lib):
    assert _noalloc(lib, B=-1) == INVALID
    assert _noalloc(lib, hq=30) == INVALID
    assert _noalloc(lib, d=80) == UNSUPPORTED
    assert _noalloc(lib, ps=100) == INVALID
    assert _noalloc(lib, P=0) == INVALID
    assert _noalloc(lib, ps=1 << 24, P=4096) == UNSUPPORTED
    assert _noalloc(lib, scale=-1.0) == INVALID
    assert _noalloc(lib, out=None) == INVALID           # out is always written
    assert _noalloc(lib, ctx=None) == INVALID
    assert _noalloc(lib, B=0, out=None, q=None, kc=None, vc=None, bt=None, ctx=None) == OK
    # pieces beyond the 16 MiB static scratch: B*Hq*P*(D+1)*4 bytes
    assert _noalloc(lib, B=64, hq=64, P=8, ps=1024) == pa.PA_ERR_TOO_LARGE   # 16.5 MiB
    assert _noalloc(lib, B=4, hq=64, hkv=8, d=256, P=64, ps=128) == pa.PA_ERR_TOO_LARGE
