"""Pools past 4 GiB and 2^31 elements: every kernel must address blocks with
64-bit offsets.

Each case is drawn as an ordinary seeded, NaN-poisoned compact pool.  Its
blocks are then placed at high ids of a NaN-filled device pool of
LARGE_BLOCKS blocks (Qwen3-4B shapes: 32 KiB per block per pool, 5.24 GB and
2.62e9 bf16 elements each for K and V), and the block tables and slots are
renumbered to match.  The GPU therefore reads and writes byte offsets past
2^32, and element offsets past 2^31, while the oracle runs on the compact
pool.  The mapped blocks must come out bit-exact against the oracle's
write_kv.  The rest of the large pool must still be NaN.  The outputs must
meet the usual bar against the oracle.  Block id 131072 is where offsets
cross both limits; every mapped id lies above 150000."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_gqa_write_amd as pa
import workloads
from _gpu_helpers import DEV, announce, check_tolerance
from _helpers import bits

pytestmark = pytest.mark.gpu

HQ, HKV, D = 32, 8, 128
LARGE_BLOCKS = 160_000
HIGH_BASE = 150_000
assert HIGH_BASE * HKV * 16 * D > 2**31 and HIGH_BASE * HKV * 16 * D * 2 > 2**32


@pytest.fixture(scope="module")
def large_pools():
    announce(f"large pools: 2 x {LARGE_BLOCKS} blocks x {HKV * 16 * D * 2} B")
    k = torch.empty((LARGE_BLOCKS, HKV, D // 32, 16, 32), dtype=torch.bfloat16, device=DEV)
    v = torch.empty((LARGE_BLOCKS, HKV, D, 16), dtype=torch.bfloat16, device=DEV)
    yield k, v
    del k, v
    torch.cuda.empty_cache()


def _high_ids(nb, seed):
    """Distinct high block ids for compact blocks 0..nb-1, in shuffled order."""
    g = torch.Generator().manual_seed(seed)
    span = torch.arange(HIGH_BASE, LARGE_BLOCKS, dtype=torch.int64)
    pick = span[torch.randperm(span.numel(), generator=g)[:nb]]
    return pick


def _place(large_pools, kc, vc, ids):
    """NaN-fill the large pools, then put the compact pools' blocks at ids."""
    bk, bv = large_pools
    bk.fill_(float("nan"))
    bv.fill_(float("nan"))
    dev_ids = ids.to(DEV)
    bk.index_copy_(0, dev_ids, kc.to(DEV))
    bv.index_copy_(0, dev_ids, vc.to(DEV))
    return bk, bv


def _map_table(bt, ids):
    out = bt.to(torch.int64).clone()
    live = out >= 0
    out[live] = ids[out[live]]
    return out.to(torch.int32)


def _map_slots(slots, ids):
    out = slots.clone()
    live = out >= 0
    out[live] = ids[out[live] // 16] * 16 + out[live] % 16
    return out


def _non_nan(t, chunk=8192):
    n = 0
    for i in range(0, t.shape[0], chunk):
        n += int((~torch.isnan(t[i:i + chunk])).sum().item())
    return n


def _check_pools(large_pools, ids, ek, ev):
    """Mapped blocks bit-exact against the oracle's pools; nothing else written."""
    bk, bv = large_pools
    dev_ids = ids.to(DEV)
    assert np.array_equal(bits(bk.index_select(0, dev_ids).cpu()), ek)
    assert np.array_equal(bits(bv.index_select(0, dev_ids).cpu()), ev)
    assert _non_nan(bk) == int((~np.isnan(_bf16_to_f32(ek))).sum())
    assert _non_nan(bv) == int((~np.isnan(_bf16_to_f32(ev))).sum())


def _bf16_to_f32(b):
    return (b.astype(np.uint32) << 16).view(np.float32)


def _decode_case(seed):
    return workloads.make_decode_case("large_pool_decode", context_lens=[1, 700, 1153, 2048, 3001, 16],
                                      num_q_heads=HQ, num_kv_heads=HKV, head_dim=D, num_blocks=560,
                                      seed=seed)


@pytest.mark.parametrize("ps,P", [(None, None), (64, 47), (3008, 1)],
                         ids=["library_plan", "split_64", "one_partition"])
def test_large_pool_decode_append(large_pools, ps, P):
    """pa_decode_append at high block ids, in the library's plan, a split-K
    plan of 47 x 64 (many partitions, each wave's first entries) and one
    partition of 3008 tokens (4 waves with ranges past 32 pairs)."""
    announce(f"large pool decode_append ps={ps} P={P}")
    case = _decode_case(71)
    ids = _high_ids(case.num_blocks, 5)
    bk, bv = _place(large_pools, case.k_cache, case.v_cache, ids)
    bt = _map_table(case.block_tables, ids).to(DEV)
    out = pa.decode_append(case.q.to(DEV), case.k_new.to(DEV), case.v_new.to(DEV), bk, bv, bt,
                           case.context_lens.to(DEV), case.scale,
                           max_context_len=int(case.context_lens.max()),
                           partition_size=ps, num_partitions=P)
    torch.cuda.synchronize()
    ek, ev = oracle.write_kv(bits(case.k_cache), bits(case.v_cache), bits(case.k_new),
                             bits(case.v_new), case.slot_mapping.numpy())
    ref = oracle.decode(bits(case.q), ek, ev, case.block_tables.numpy(), case.context_lens.numpy(),
                        case.scale, HQ, HKV)
    check_tolerance(f"large pool decode_append ps={ps}", out.cpu(), ref)
    _check_pools(large_pools, ids, ek, ev)


def test_large_pool_write_kv_decode_and_noalloc(large_pools):
    """pa_write_kv of the new tokens to renumbered slots past 2^31 elements,
    then pa_decode (split-K + reduce) and pa_decode_noalloc over the same
    pools: outputs against the oracle, the noalloc output bit-identical."""
    announce("large pool write_kv + decode + decode_noalloc")
    case = _decode_case(72)
    ids = _high_ids(case.num_blocks, 6)
    bk, bv = _place(large_pools, case.k_cache, case.v_cache, ids)
    slots = _map_slots(case.slot_mapping, ids).to(DEV)
    assert int(slots.max()) * HKV * D > 2**31
    pa.write_kv(case.k_new.to(DEV), case.v_new.to(DEV), slots, bk, bv)
    bt = _map_table(case.block_tables, ids).to(DEV)
    ctx = case.context_lens.to(DEV)
    out = pa.decode(case.q.to(DEV), bk, bv, bt, ctx, case.scale,
                    max_context_len=int(case.context_lens.max()), partition_size=256)
    out2 = pa.decode_noalloc(case.q.to(DEV), bk, bv, bt, ctx, case.scale, 256, 12)
    torch.cuda.synchronize()
    ek, ev = oracle.write_kv(bits(case.k_cache), bits(case.v_cache), bits(case.k_new),
                             bits(case.v_new), case.slot_mapping.numpy())
    ref = oracle.decode(bits(case.q), ek, ev, case.block_tables.numpy(), case.context_lens.numpy(),
                        case.scale, HQ, HKV)
    check_tolerance("large pool decode", out.cpu(), ref)
    assert torch.equal(out, out2)
    _check_pools(large_pools, ids, ek, ev)


def test_large_pool_decode_multi(large_pools):
    """Multi-token decode (4 query tokens per sequence) at high block ids."""
    announce("large pool decode_multi T=4")
    case = workloads.make_multi_decode_case("large_pool_multi", query_len=4,
                                            context_lens=[4, 517, 1200, 2400], num_q_heads=HQ,
                                            num_kv_heads=HKV, head_dim=D, num_blocks=260, seed=73)
    ids = _high_ids(case.num_blocks, 7)
    bk, bv = _place(large_pools, case.k_cache, case.v_cache, ids)
    pa.write_kv(case.k_new.to(DEV), case.v_new.to(DEV), _map_slots(case.slot_mapping, ids).to(DEV),
                bk, bv)
    out = pa.decode_multi(case.q.to(DEV), bk, bv, _map_table(case.block_tables, ids).to(DEV),
                          case.context_lens.to(DEV), case.scale,
                          max_context_len=int(case.context_lens.max()))
    torch.cuda.synchronize()
    ek, ev = oracle.write_kv(bits(case.k_cache), bits(case.v_cache), bits(case.k_new),
                             bits(case.v_new), case.slot_mapping.numpy())
    ref = oracle.decode_multi(bits(case.q), ek, ev, case.block_tables.numpy(),
                              case.context_lens.numpy(), case.scale, HQ, HKV)
    check_tolerance("large pool decode_multi", out.cpu(), ref)
    _check_pools(large_pools, ids, ek, ev)


def test_large_pool_prefill(large_pools):
    """pa_write_kv + pa_prefill with cached prefixes at high block ids."""
    announce("large pool prefill")
    case = workloads.make_prefill_case("large_pool_prefill", q_lens=[300, 700, 33],
                                       prefix_lens=[100, 0, 517], num_q_heads=HQ,
                                       num_kv_heads=HKV, head_dim=D, num_blocks=120, seed=74)
    ids = _high_ids(case.num_blocks, 8)
    bk, bv = _place(large_pools, case.k_cache, case.v_cache, ids)
    pa.write_kv(case.k_new.to(DEV), case.v_new.to(DEV), _map_slots(case.slot_mapping, ids).to(DEV),
                bk, bv)
    out = pa.prefill(case.q.to(DEV), bk, bv, _map_table(case.block_tables, ids).to(DEV),
                     case.cu_seqlens.to(DEV), case.prefix_lens.to(DEV), case.scale,
                     max(case.q_lens))
    torch.cuda.synchronize()
    ek, ev = oracle.write_kv(bits(case.k_cache), bits(case.v_cache), bits(case.k_new),
                             bits(case.v_new), case.slot_mapping.numpy())
    ref = oracle.prefill(bits(case.q), ek, ev, case.block_tables.numpy(), case.cu_seqlens.numpy(),
                         case.prefix_lens.numpy(), case.scale, HQ, HKV)
    check_tolerance("large pool prefill", out.cpu(), ref)
    _check_pools(large_pools, ids, ek, ev)


def test_large_pool_copy_blocks(large_pools):
    """pa_copy_blocks between high ids, and from high ids to low ones: each
    destination block equals its source block bit for bit; the sources and
    every other block are untouched."""
    announce("large pool copy_blocks")
    gen = torch.Generator().manual_seed(75)
    nb = 48
    kc = workloads._normal_bf16(gen, (nb, HKV, D // 32, 16, 32), 1.0)
    vc = workloads._normal_bf16(gen, (nb, HKV, D, 16), 1.0)
    ids = _high_ids(nb, 9)
    bk, bv = _place(large_pools, kc, vc, ids)
    src = ids[:24]
    taken = set(ids.tolist())
    free_high = [b for b in range(LARGE_BLOCKS - 1, HIGH_BASE, -1) if b not in taken][:12]
    dst = torch.cat([torch.tensor(free_high, dtype=torch.int64),
                     torch.arange(12, dtype=torch.int64) * 3 + 1])
    pa.copy_blocks(bk, bv, bk, bv, dst_ids=dst.to(torch.int32).to(DEV),
                   src_ids=src.to(torch.int32).to(DEV))
    torch.cuda.synchronize()
    dev_dst = dst.to(DEV)
    assert np.array_equal(bits(bk.index_select(0, dev_dst).cpu()), bits(kc[:24]))
    assert np.array_equal(bits(bv.index_select(0, dev_dst).cpu()), bits(vc[:24]))
    all_ids = torch.cat([ids, dst])
    expect_k = np.concatenate([bits(kc), bits(kc[:24])])
    expect_v = np.concatenate([bits(vc), bits(vc[:24])])
    _check_pools(large_pools, all_ids, expect_k, expect_v)
