"""The Python binding checks every tensor it hands to the library -- inputs,
outputs and the split-K workspace -- before anything reaches the GPU.

These run on the CPU: shapes are checked before where a tensor lives, so a
call whose shapes are all right stops only at the final device check, and a
wrong output or workspace shape is reported by name.  No kernel is launched.
"""
import pytest
import torch

import paged_kv_gqa_write_amd as pa

B, HQ, HKV, D, NB, MB = 3, 8, 2, 64, 16, 4
BF, F32, I32 = torch.bfloat16, torch.float32, torch.int32


def pools():
    return (torch.zeros(NB, HKV, D // 32, 16, 32, dtype=BF), torch.zeros(NB, HKV, D, 16, dtype=BF))


def inputs(T=None):
    q = torch.zeros((B, HQ, D) if T is None else (B, T, HQ, D), dtype=BF)
    return q, torch.zeros(B, MB, dtype=I32), torch.zeros(B, dtype=I32)


def reaches_device_check(fn):
    with pytest.raises(ValueError, match="GPU tensor"):
        fn()


def rejects(fn, name):
    with pytest.raises((ValueError, TypeError), match=name):
        fn()


def test_pool_layout_checked():
    """K must be [NB, Hkv, D/32, 16, 32]: the token-row shape [NB, Hkv, 16, D],
    another slice width, or a K/V head-dim mismatch is refused."""
    kc, vc = pools()
    q, bt, ctx = inputs()
    call = lambda k, v: pa.decode(q, k, v, bt, ctx, 0.1, partition_size=64,  # noqa: E731
                                  num_partitions=1)
    reaches_device_check(lambda: call(kc, vc))
    rejects(lambda: call(torch.zeros(NB, HKV, 16, D, dtype=BF), vc), "k_cache")
    rejects(lambda: call(torch.zeros(NB, HKV, D // 16, 16, 16, dtype=BF), vc), "pools")
    rejects(lambda: call(torch.zeros(NB, HKV, D // 32 + 1, 16, 32, dtype=BF), vc), "pools")
    kn = torch.zeros(B, HKV, D, dtype=BF)
    rejects(lambda: pa.write_kv(kn, kn, torch.zeros(B, dtype=torch.int64),
                                torch.zeros(NB, HKV, 16, D, dtype=BF), vc), "k_cache")
    rejects(lambda: pa.copy_blocks(torch.zeros(NB, HKV, 16, D, dtype=BF), vc, kc, vc), "dst_k")


def test_decode_single_partition_out_shape():
    kc, vc = pools()
    q, bt, ctx = inputs()
    good = torch.zeros(B, HQ, D, dtype=BF)
    call = lambda out: pa.decode(q, kc, vc, bt, ctx, 0.1, partition_size=64,  # noqa: E731
                                 num_partitions=1, out=out)
    reaches_device_check(lambda: call(good))
    rejects(lambda: call(torch.zeros(B, HQ + 1, D, dtype=BF)), "out")
    rejects(lambda: call(torch.zeros(B, HQ, D, dtype=F32)), "out")
    rejects(lambda: call(torch.zeros(B, HQ, 2 * D, dtype=BF)[:, :, :D]), "out")


@pytest.mark.parametrize("which", ["part_out", "part_lse"])
def test_decode_workspace_shapes(which):
    kc, vc = pools()
    q, bt, ctx = inputs()
    P = 3
    ws = {"part_out": torch.zeros(B, HQ, P, D, dtype=F32),
          "part_lse": torch.zeros(B, HQ, P, dtype=F32)}
    call = lambda **kw: pa.decode(q, kc, vc, bt, ctx, 0.1, partition_size=64,  # noqa: E731
                                  num_partitions=P, **{**ws, **kw})
    reaches_device_check(lambda: call())
    # a workspace planned for another partition count would be overrun
    bad = {"part_out": torch.zeros(B, HQ, P - 1, D, dtype=F32),
           "part_lse": torch.zeros(B, HQ, P - 1, dtype=F32)}[which]
    rejects(lambda: call(**{which: bad}), which)
    rejects(lambda: call(**{which: ws[which].double()}), which)
    rejects(lambda: pa.decode_partials(q, kc, vc, bt, ctx, 0.1, 64, P,
                                       **{**ws, which: bad}), which)


def test_decode_append_shapes():
    kc, vc = pools()
    q, bt, ctx = inputs()
    kn = torch.zeros(B, HKV, D, dtype=BF)
    call = lambda kn=kn, vn=kn, **kw: pa.decode_append(  # noqa: E731
        q, kn, vn, kc, vc, bt, ctx, 0.1, partition_size=64, num_partitions=1, **kw)
    reaches_device_check(lambda: call())
    rejects(lambda: call(kn=torch.zeros(B, HKV + 1, D, dtype=BF)), "k_new")
    rejects(lambda: call(vn=torch.zeros(B - 1, HKV, D, dtype=BF)), "v_new")
    rejects(lambda: call(out=torch.zeros(B + 1, HQ, D, dtype=BF)), "out")
    P = 2
    call2 = lambda **kw: pa.decode_append(  # noqa: E731
        q, kn, kn, kc, vc, bt, ctx, 0.1, partition_size=64, num_partitions=P, **kw)
    rejects(lambda: call2(part_out=torch.zeros(B, HQ, P + 1, D, dtype=F32)), "part_out")
    rejects(lambda: call2(part_lse=torch.zeros(B, HQ, 1, dtype=F32)), "part_lse")


def test_decode_reduce_shapes():
    P = 4
    po = torch.zeros(B, HQ, P, D, dtype=F32)
    pl = torch.zeros(B, HQ, P, dtype=F32)
    ctx = torch.zeros(B, dtype=I32)
    reaches_device_check(lambda: pa.decode_reduce(po, pl, ctx, 64))
    rejects(lambda: pa.decode_reduce(po, torch.zeros(B, HQ, P - 1, dtype=F32), ctx, 64),
            "part_lse")
    rejects(lambda: pa.decode_reduce(po, pl, torch.zeros(B + 1, dtype=I32), 64), "context_lens")
    rejects(lambda: pa.decode_reduce(po, pl, ctx, 64, out=torch.zeros(B, HQ, D + 1, dtype=BF)),
            "out")
    rejects(lambda: pa.decode_reduce(po, None, ctx, 64), "part_lse")


def test_decode_multi_shapes():
    T, P = 3, 2
    kc, vc = pools()
    q, bt, ctx = inputs(T)
    ws = {"part_out": torch.zeros(B, T, HQ, P, D, dtype=F32),
          "part_lse": torch.zeros(B, T, HQ, P, dtype=F32)}
    call = lambda **kw: pa.decode_multi(q, kc, vc, bt, ctx, 0.1, partition_size=64,  # noqa: E731
                                        num_partitions=P, **{**ws, **kw})
    reaches_device_check(lambda: call())
    rejects(lambda: call(part_out=torch.zeros(B, T, HQ, P + 1, D, dtype=F32)), "part_out")
    rejects(lambda: call(part_lse=torch.zeros(B, T - 1, HQ, P, dtype=F32)), "part_lse")
    rejects(lambda: call(out=torch.zeros(B, T, HQ, D - 1, dtype=BF)), "out")
    one = lambda out: pa.decode_multi(q, kc, vc, bt, ctx, 0.1, partition_size=64,  # noqa: E731
                                      num_partitions=1, out=out)
    reaches_device_check(lambda: one(torch.zeros(B, T, HQ, D, dtype=BF)))
    rejects(lambda: one(torch.zeros(B, T + 1, HQ, D, dtype=BF)), "out")
    po, pl = ws["part_out"], ws["part_lse"]
    reaches_device_check(lambda: pa.decode_multi_reduce(po, pl, ctx, 64))
    rejects(lambda: pa.decode_multi_reduce(po, pl[:, :, :, :1].contiguous(), ctx, 64), "part_lse")
    rejects(lambda: pa.decode_multi_reduce(po, pl, ctx, 64,
                                           out=torch.zeros(B, T, HQ + 1, D, dtype=BF)), "out")


def test_prefill_shapes():
    kc, vc = pools()
    total = 10
    q = torch.zeros(total, HQ, D, dtype=BF)
    bt = torch.zeros(2, MB, dtype=I32)
    cu = torch.tensor([0, 4, 10], dtype=I32)
    pre = torch.zeros(2, dtype=I32)
    call = lambda out=None, pre=pre: pa.prefill(q, kc, vc, bt, cu, pre, 0.1, 6,  # noqa: E731
                                                out=out)
    reaches_device_check(lambda: call())
    reaches_device_check(lambda: call(out=torch.zeros(total, HQ, D, dtype=BF)))
    rejects(lambda: call(out=torch.zeros(total - 1, HQ, D, dtype=BF)), "out")
    rejects(lambda: call(out=torch.zeros(total, HQ, D, dtype=F32)), "out")
    rejects(lambda: call(pre=torch.zeros(3, dtype=I32)), "prefix_lens")


def test_heads_must_divide():
    kc, vc = pools()
    q = torch.zeros(B, 3, D, dtype=BF)   # 3 query heads over 2 KV heads
    _, bt, ctx = inputs()
    rejects(lambda: pa.decode(q, kc, vc, bt, ctx, 0.1, partition_size=64, num_partitions=1),
            "multiple")
