"""pa_write_kv on the GPU: bit-exact against the oracle over the whole pool."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_gqa_write_amd as pa
import workloads
from _gpu_helpers import DEV, announce
from _helpers import bits

pytestmark = pytest.mark.gpu


def _check_pools(kc_gpu, vc_gpu, k0, v0, k_new, v_new, slots):
    ek, ev = oracle.write_kv(bits(k0), bits(v0), bits(k_new), bits(v_new), slots.numpy())
    assert np.array_equal(bits(kc_gpu), ek)
    assert np.array_equal(bits(vc_gpu), ev)


@pytest.mark.parametrize("name", ["tiny_decode", "qwen3_4b_decode_b8", "hybrid_decode_b8"])
def test_write_kv_decode_tokens_bit_exact(name):
    announce(f"write_kv {name}")
    case = workloads.DECODE_CASES[name]()
    kc, vc = case.k_cache.to(DEV), case.v_cache.to(DEV)
    pa.write_kv(case.k_new.to(DEV), case.v_new.to(DEV), case.slot_mapping.to(DEV), kc, vc)
    torch.cuda.synchronize()
    _check_pools(kc.cpu(), vc.cpu(), case.k_cache, case.v_cache, case.k_new, case.v_new,
                 case.slot_mapping)


@pytest.mark.parametrize("name", ["qwen3_4b_prefill_4x1024", "hybrid_prefill_4097"])
def test_write_kv_prefill_tokens_bit_exact(name):
    announce(f"write_kv {name}")
    case = workloads.PREFILL_CASES[name]()
    kc, vc = case.k_cache.to(DEV), case.v_cache.to(DEV)
    pa.write_kv(case.k_new.to(DEV), case.v_new.to(DEV), case.slot_mapping.to(DEV), kc, vc)
    torch.cuda.synchronize()
    _check_pools(kc.cpu(), vc.cpu(), case.k_cache, case.v_cache, case.k_new, case.v_new,
                 case.slot_mapping)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_write_kv_random_slots_skips_negative_and_out_of_range(d):
    announce(f"write_kv random slots d={d}")
    g = torch.Generator().manual_seed(d)
    nb, hkv, T = 37, 3, 300
    k0 = torch.randn(nb, hkv, d // 32, 16, 32, generator=g).to(torch.bfloat16)
    v0 = torch.randn(nb, hkv, d, 16, generator=g).to(torch.bfloat16)
    kn = torch.randn(T, hkv, d, generator=g).to(torch.bfloat16)
    vn = torch.randn(T, hkv, d, generator=g).to(torch.bfloat16)
    slots = torch.randperm(nb * 16, generator=g)[:T].to(torch.int64)
    slots[::7] = -1
    slots[5] = nb * 16          # out of range: must be skipped, never written
    slots[11] = nb * 16 + 1000
    kc, vc = k0.to(DEV), v0.to(DEV)
    pa.write_kv(kn.to(DEV), vn.to(DEV), slots.to(DEV), kc, vc)
    torch.cuda.synchronize()
    valid = slots.clone()
    valid[valid >= nb * 16] = -1
    _check_pools(kc.cpu(), vc.cpu(), k0, v0, kn, vn, valid)


def test_write_kv_zero_tokens_is_noop():
    kc = torch.zeros(2, 1, 2, 16, 32, dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros(2, 1, 64, 16, dtype=torch.bfloat16, device=DEV)
    e = torch.empty(0, 1, 64, dtype=torch.bfloat16, device=DEV)
    pa.write_kv(e, e, torch.empty(0, dtype=torch.int64, device=DEV), kc, vc)
    torch.cuda.synchronize()
    assert kc.abs().sum().item() == 0


@pytest.mark.parametrize("d", [64, 128, 256])
def test_write_kv_whole_blocks_and_broken_runs(d):
    """Groups of 16 tokens that fill one block in order take the transposed
    whole-block store; everything else the per-element one.  Mixed here:
    whole blocks (including the pool's last block), a block filled in
    reverse order, a run shifted by one slot, a run with one skipped token,
    a group spanning two blocks, and a short final group."""
    announce(f"write_kv whole blocks and broken runs d={d}")
    g = torch.Generator().manual_seed(300 + d)
    nb, hkv = 24, 2
    runs = [torch.arange(16) + 16 * 3,                 # whole block 3
            torch.arange(16).flip(0) + 16 * 5,         # block 5, reverse order
            torch.arange(16) + 16 * 7 + 1,             # shifted by one slot (crosses into block 8)
            torch.cat([torch.arange(7), torch.tensor([-1]), torch.arange(8, 16)]) + 16 * 10,
            torch.arange(16) + 16 * (nb - 1),          # the pool's last block, whole
            torch.cat([torch.arange(8) + 16 * 12 + 8, torch.arange(8) + 16 * 13]),
            torch.arange(16) + 16 * 15,                # whole block 15
            torch.arange(9) + 16 * 20]                 # short last group
    slots = torch.cat(runs).to(torch.int64)
    slots[3 * 16 + 7] = -1 - 16 * 10                   # the -1 inside run 4, kept negative
    T = slots.numel()
    k0 = torch.randn(nb, hkv, d // 32, 16, 32, generator=g).to(torch.bfloat16)
    v0 = torch.randn(nb, hkv, d, 16, generator=g).to(torch.bfloat16)
    kn = torch.randn(T, hkv, d, generator=g).to(torch.bfloat16)
    vn = torch.randn(T, hkv, d, generator=g).to(torch.bfloat16)
    kc, vc = k0.to(DEV), v0.to(DEV)
    pa.write_kv(kn.to(DEV), vn.to(DEV), slots.to(DEV), kc, vc)
    torch.cuda.synchronize()
    _check_pools(kc.cpu(), vc.cpu(), k0, v0, kn, vn, slots)
