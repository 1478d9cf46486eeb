"""pa_copy_blocks on the GPU against the CPU oracle: bit-exact over whole
pools, for copies inside a device pool, restores from pinned host memory
and saves to it."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import paged_kv_gqa_write_amd as pa
import workloads
from _gpu_helpers import DEV, announce
from _helpers import bits, from_bits, random_bf16_bits

pytestmark = pytest.mark.gpu


def _pool(gen, nb, hkv, d):
    return (from_bits(random_bf16_bits(gen, (nb, hkv, d // 32, 16, 32))),
            from_bits(random_bf16_bits(gen, (nb, hkv, d, 16))))


def _ids(values):
    return torch.tensor(values, dtype=torch.int32)


@pytest.mark.parametrize("hkv,d", [(1, 64), (8, 128), (2, 256), (3, 128)])
def test_copy_within_device_pool(hkv, d):
    """Duplicating blocks inside one pool (sources and destinations disjoint),
    with one copy naming a source and one a destination outside the pool:
    the whole pool against the oracle, bit for bit."""
    announce(f"copy_blocks in-pool hkv={hkv} d={d}")
    gen = torch.Generator().manual_seed(100 + d + hkv)
    nb = 64
    k, v = _pool(gen, nb, hkv, d)
    perm = torch.randperm(nb, generator=gen)
    src = perm[:20].tolist() + [-1, int(perm[41])]
    dst = perm[20:40].tolist() + [int(perm[42]), nb]
    kd, vd = k.to(DEV), v.to(DEV)
    pa.copy_blocks(kd, vd, kd, vd, dst_ids=_ids(dst).to(DEV), src_ids=_ids(src).to(DEV))
    torch.cuda.synchronize()
    ek, ev = oracle.copy_blocks(bits(k), bits(v), np.array(dst), bits(k), bits(v),
                                np.array(src), len(src))
    assert np.array_equal(bits(kd), ek) and np.array_equal(bits(vd), ev)


def test_restore_from_pinned_host_buffer():
    """A packed host buffer of sealed blocks (pinned memory, read by the
    kernel over the host link) scattered into chosen pool blocks; ids live in
    pinned host memory too."""
    announce("copy_blocks restore from pinned host")
    gen = torch.Generator().manual_seed(7)
    hkv, d, n, nb = 8, 128, 37, 96
    hk, hv = _pool(gen, n, hkv, d)
    host_k = torch.empty(hk.shape, dtype=torch.bfloat16, pin_memory=True)
    host_v = torch.empty(hv.shape, dtype=torch.bfloat16, pin_memory=True)
    host_k.copy_(hk)
    host_v.copy_(hv)
    k, v = _pool(gen, nb, hkv, d)
    dst = torch.randperm(nb, generator=gen)[:n].tolist()
    dst[11] = 9999                                   # skipped: outside the pool
    dst_ids = torch.empty(n, dtype=torch.int32, pin_memory=True)
    dst_ids.copy_(_ids(dst))
    kd, vd = k.to(DEV), v.to(DEV)
    pa.copy_blocks(kd, vd, host_k, host_v, dst_ids=dst_ids)
    torch.cuda.synchronize()
    ek, ev = oracle.copy_blocks(bits(k), bits(v), np.array(dst), bits(hk), bits(hv), None, n)
    assert np.array_equal(bits(kd), ek) and np.array_equal(bits(vd), ev)


def test_save_to_pinned_host_buffer():
    """Blocks gathered from a device pool into a packed pinned host buffer
    (the kernel writes host memory), then read back on the host."""
    announce("copy_blocks save to pinned host")
    gen = torch.Generator().manual_seed(8)
    hkv, d, n, nb = 2, 256, 21, 40
    k, v = _pool(gen, nb, hkv, d)
    src = torch.randperm(nb, generator=gen)[:n].tolist()
    host_k = torch.zeros((n, hkv, d // 32, 16, 32), dtype=torch.bfloat16, pin_memory=True)
    host_v = torch.zeros((n, hkv, d, 16), dtype=torch.bfloat16, pin_memory=True)
    pa.copy_blocks(host_k, host_v, k.to(DEV), v.to(DEV), src_ids=_ids(src).to(DEV))
    torch.cuda.synchronize()
    ek, ev = oracle.copy_blocks(np.zeros((n, hkv, d // 32, 16, 32), np.uint16),
                                np.zeros((n, hkv, d, 16), np.uint16), None, bits(k), bits(v),
                                np.array(src), n)
    assert np.array_equal(bits(host_k), ek) and np.array_equal(bits(host_v), ev)


def test_restored_blocks_decode_identically():
    """Save every block a batch uses to pinned host memory, restore them into
    other blocks of a fresh pool, remap the table: pa_decode through the
    restored pool gives the same bits as through the original."""
    announce("copy_blocks save/restore round trip + decode")
    case = workloads.make_decode_case("rt", context_lens=[300, 77, 1000, 16], num_q_heads=32,
                                      num_kv_heads=8, head_dim=128, num_blocks=160, seed=30,
                                      poison=False)
    bt = case.block_tables
    used = [int(b) for b in bt.reshape(-1).tolist() if b >= 0]
    n = len(used)
    kc, vc = case.k_cache.to(DEV), case.v_cache.to(DEV)
    args = (case.q.to(DEV),)
    base = pa.decode(*args, kc, vc, bt.to(DEV), case.context_lens.to(DEV), case.scale,
                     partition_size=128)
    host_k = torch.empty((n, 8, 4, 16, 32), dtype=torch.bfloat16, pin_memory=True)
    host_v = torch.empty((n, 8, 128, 16), dtype=torch.bfloat16, pin_memory=True)
    pa.copy_blocks(host_k, host_v, kc, vc, src_ids=_ids(used).to(DEV))
    gen = torch.Generator().manual_seed(31)
    nb2 = 400
    fresh = torch.randperm(nb2, generator=gen)[:n]
    k2 = torch.randn((nb2, 8, 4, 16, 32), generator=gen).to(torch.bfloat16).to(DEV)
    v2 = torch.randn((nb2, 8, 128, 16), generator=gen).to(torch.bfloat16).to(DEV)
    pa.copy_blocks(k2, v2, host_k, host_v, dst_ids=fresh.to(torch.int32).to(DEV))
    remap = dict(zip(used, fresh.tolist()))
    bt2 = torch.tensor([[remap.get(int(b), -1) if b >= 0 else -1 for b in row]
                        for row in bt.tolist()], dtype=torch.int32)
    again = pa.decode(*args, k2, v2, bt2.to(DEV), case.context_lens.to(DEV), case.scale,
                      partition_size=128)
    torch.cuda.synchronize()
    assert torch.equal(base.cpu(), again.cpu())


def test_pageable_host_memory_is_rejected_before_launch():
    """Pageable host memory cannot be reached by a kernel: the library says
    so on the host and enqueues nothing; later calls are unaffected."""
    announce("copy_blocks pageable rejected")
    gen = torch.Generator().manual_seed(9)
    k, v = _pool(gen, 8, 2, 64)
    kd, vd = k.to(DEV), v.to(DEV)
    pageable_k, pageable_v = k.clone(), v.clone()
    assert not pageable_k.is_pinned()
    lib = pa.load_library()
    st = lib.pa_copy_blocks(kd.data_ptr(), vd.data_ptr(), 8, None, pageable_k.data_ptr(),
                            pageable_v.data_ptr(), 8, None, 8, 2, 64, 16,
                            torch.cuda.current_stream().cuda_stream)
    assert st == pa.PA_ERR_INVALID_ARG
    with pytest.raises(ValueError):
        pa.copy_blocks(kd, vd, pageable_k, pageable_v)
    torch.cuda.synchronize()
    assert torch.equal(kd.cpu(), k) and torch.equal(vd.cpu(), v)
    # the failed pointer query left no error behind for the next launch
    pa.copy_blocks(kd, vd, kd, vd, dst_ids=_ids([1]).to(DEV), src_ids=_ids([0]).to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(kd[1].cpu(), k[0])


def test_zero_copies_is_a_no_op():
    announce("copy_blocks zero")
    gen = torch.Generator().manual_seed(10)
    k, v = _pool(gen, 4, 1, 64)
    kd, vd = k.to(DEV), v.to(DEV)
    pa.copy_blocks(kd, vd, kd, vd, num_copies=0)
    torch.cuda.synchronize()
    assert torch.equal(kd.cpu(), k) and torch.equal(vd.cpu(), v)
