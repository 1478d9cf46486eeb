"""pa_decode_append (append the new token's K/V and decode, one kernel) on
the GPU: outputs against the oracle's write_kv + decode, the pools bit-exact
against the oracle's write_kv, and bit-identical to pa_write_kv + pa_decode.
The pools are NaN-poisoned at every slot that does not hold a live token --
the new token's own slot included -- so a kernel that read the new token
back from the pool instead of its own copy would return NaN."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_gqa_write_amd as pa
import workloads
from _gpu_helpers import DEV, announce, check_tolerance, decode_gpu, decode_oracle
from _helpers import bits


def _append_gpu(case, partition_size=None, num_partitions=None):
    kc, vc = case.k_cache.to(DEV), case.v_cache.to(DEV)
    out = pa.decode_append(case.q.to(DEV), case.k_new.to(DEV), case.v_new.to(DEV), kc, vc,
                           case.block_tables.to(DEV), case.context_lens.to(DEV), case.scale,
                           max_context_len=max(int(case.context_lens.max()), 1),
                           partition_size=partition_size, num_partitions=num_partitions)
    torch.cuda.synchronize()
    return out.cpu(), kc.cpu(), vc.cpu()


def _oracle_pools(case):
    return oracle.write_kv(bits(case.k_cache), bits(case.v_cache), bits(case.k_new),
                           bits(case.v_new), case.slot_mapping.numpy())


pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", list(workloads.DECODE_CASES))
def test_decode_append_config_parity(name):
    """Every decode workload at full size in the library's split plan."""
    announce(f"decode_append {name}")
    case = workloads.DECODE_CASES[name]()
    out, kc, vc = _append_gpu(case)
    check_tolerance(name, out, decode_oracle(case), literal=True)
    ek, ev = _oracle_pools(case)
    assert np.array_equal(bits(kc), ek) and np.array_equal(bits(vc), ev)


@pytest.mark.parametrize("ps", [None, 16, 32, 64, 1152])
def test_decode_append_equals_write_then_decode_bitwise(ps):
    announce(f"decode_append vs write_kv+decode ps={ps}")
    case = workloads.qwen3_4b_decode()
    out, _, _ = _append_gpu(case, partition_size=ps)
    assert torch.equal(out, decode_gpu(case, partition_size=ps))


@pytest.mark.parametrize("name", ["qwen3_32b_decode_b64", "qwen3_32b_decode_b4_8192",
                                  "hybrid_decode_b8"])
def test_decode_append_equals_write_then_decode_bitwise_full_size(name):
    """The large launches in the library's plan (two workgroups per CU with
    two pairs in flight, one per CU with one pair, head_dim 256): the
    appending kernel gives the bits of pa_write_kv + pa_decode."""
    announce(f"decode_append vs write_kv+decode {name}")
    case = workloads.DECODE_CASES[name]()
    out, _, _ = _append_gpu(case)
    assert torch.equal(out, decode_gpu(case))


@pytest.mark.parametrize("hq,hkv,d", [(4, 2, 64), (32, 8, 128), (16, 2, 256), (16, 1, 128)])
def test_decode_append_new_token_positions(hq, hkv, d):
    """The new token at every kind of place: alone (ctx 1), first and last
    slot of a block, in the first and second block of a 32-key pair, on a
    partition boundary (ps = 64: ctx-1 = 64 starts partition 1), and a
    sequence with nothing to append (ctx 0)."""
    announce(f"decode_append positions hq={hq} hkv={hkv} d={d}")
    lens = [1, 16, 17, 32, 33, 48, 64, 65, 100, 0, 129]
    case = workloads.make_decode_case("pos", context_lens=lens, num_q_heads=hq,
                                      num_kv_heads=hkv, head_dim=d, num_blocks=96,
                                      seed=hq + d)
    ref = decode_oracle(case)
    ek, ev = _oracle_pools(case)
    for ps, P in [(144, 1), (64, 3), (16, 9)]:
        out, kc, vc = _append_gpu(case, partition_size=ps, num_partitions=P)
        check_tolerance(f"positions ps={ps}", out, ref)
        assert out[9].float().abs().sum().item() == 0
        assert np.array_equal(bits(kc), ek) and np.array_equal(bits(vc), ev)


@pytest.mark.parametrize("hq,hkv,d", [(8, 2, 64), (16, 2, 128), (16, 2, 256)])
def test_decode_append_long_wave_ranges(hq, hkv, d):
    """One partition of 8192 tokens, so every wave's range holds 64 pairs:
    the waves reload their table entries after 32 pairs, and the new token
    lies at the start of a wave's range (ctx 4097, 2050, 1), within its first
    64 entries (5000) and past them (8192; at head_dim 256, whose row is
    stored before the loads, that entry is read from the table).  Pools
    bit-exact, output against the oracle and bit-identical to pa_write_kv +
    pa_decode."""
    announce(f"decode_append long wave ranges hq={hq} hkv={hkv} d={d}")
    lens = [8192, 5000, 4097, 2050, 1]
    case = workloads.make_decode_case("longwave", context_lens=lens, num_q_heads=hq,
                                      num_kv_heads=hkv, head_dim=d, num_blocks=1300,
                                      seed=d + 7)
    ref = decode_oracle(case)
    ek, ev = _oracle_pools(case)
    out, kc, vc = _append_gpu(case, partition_size=8192, num_partitions=1)
    check_tolerance(f"long wave ranges d={d}", out, ref)
    assert np.array_equal(bits(kc), ek) and np.array_equal(bits(vc), ev)
    assert torch.equal(out, decode_gpu(case, partition_size=8192))


def test_decode_two_pairs_in_flight_long_wave_ranges():
    """264 workgroups (33 sequences x 8 KV heads, one partition of 4736
    tokens each): more than one per CU, so both forms keep two pairs in
    flight, and each wave's range of ~37 pairs crosses the table-entry
    reload after 32.  The new token falls before and after that point
    depending on the length.  Output against the oracle, pools bit-exact,
    and the appending kernel bit-identical to pa_write_kv + pa_decode."""
    announce("decode_append two pairs in flight, long wave ranges")
    gen = torch.Generator().manual_seed(4736)
    lens = torch.randint(4100, 4737, (33,), generator=gen).tolist()
    lens[0], lens[1] = 4736, 4097
    nb = sum((n + 15) // 16 for n in lens) + 40
    case = workloads.make_decode_case("twopair", context_lens=lens, num_q_heads=16,
                                      num_kv_heads=8, head_dim=128, num_blocks=nb, seed=47)
    ref = decode_oracle(case)
    ek, ev = _oracle_pools(case)
    out, kc, vc = _append_gpu(case, partition_size=4736, num_partitions=1)
    check_tolerance("two pairs in flight", out, ref, literal=True)
    assert np.array_equal(bits(kc), ek) and np.array_equal(bits(vc), ev)
    assert torch.equal(out, decode_gpu(case, partition_size=4736, num_partitions=1))


def test_decode_append_bad_entry_poisons_and_skips_write():
    """A table entry outside the pool for the new token's block: NaN outputs
    for that sequence and nothing written for it; the other sequence's token
    is appended and its output unharmed."""
    announce("decode_append bad entry")
    case = workloads.make_decode_case("bad", context_lens=[40, 40], num_q_heads=8,
                                      num_kv_heads=2, head_dim=128, num_blocks=16, seed=4)
    ref = decode_oracle(case)
    ek, ev = oracle.write_kv(bits(case.k_cache), bits(case.v_cache), bits(case.k_new[:1]),
                             bits(case.v_new[:1]), case.slot_mapping[:1].numpy())
    case.block_tables[1, 2] = 77             # block of position 39 of sequence 1
    for ps in (None, 16):
        out, kc, vc = _append_gpu(case, partition_size=ps)
        assert torch.isnan(out[1].float()).all()
        check_tolerance("good sequence", out[:1], ref[:1])
        assert np.array_equal(bits(kc), ek) and np.array_equal(bits(vc), ev)


def test_decode_append_repeat_runs_bitwise_identical():
    announce("decode_append determinism")
    case = workloads.qwen3_32b_decode_long()
    a, _, _ = _append_gpu(case)
    b, _, _ = _append_gpu(case)
    assert torch.equal(a, b)


@pytest.mark.parametrize("ps,P", [(64, 1), (16, 3)], ids=["one_partition", "split"])
def test_decode_append_negative_context(ps, P):
    """A negative length: NaN output for that sequence in every plan, and its
    token is not written (the pools equal the oracle's write_kv of the other
    sequences' tokens only)."""
    announce(f"decode_append negative context ps={ps} P={P}")
    case = workloads.make_decode_case("negapp", context_lens=[40, 40, 33], num_q_heads=8,
                                      num_kv_heads=2, head_dim=128, num_blocks=16, seed=16)
    ref = decode_oracle(case)
    case.context_lens[1] = -5
    case.slot_mapping[1] = -1
    out, kc, vc = _append_gpu(case, ps, P)
    assert torch.isnan(out[1].float()).all()
    check_tolerance(f"append negative context, others (P={P})", out[[0, 2]], ref[[0, 2]])
    okc, ovc = _oracle_pools(case)
    assert np.array_equal(bits(kc), okc) and np.array_equal(bits(vc), ovc)


def test_decode_append_mixed_lengths_plan_parity():
    """The mixed batch (one 8192-token request among seven of ~1100 tokens)
    appended and decoded in the plan made from its lengths (15 x 576, items
    ranked live first), literal bar; pools bit-exact."""
    announce("decode_append qwen3_32b_decode_mixed_b8, plan from lengths")
    case = workloads.qwen3_32b_decode_mixed()
    ps, P = pa.decode_split_plan_lens(case.num_kv_heads, case.context_lens)
    out, kc, vc = _append_gpu(case, ps, P)
    check_tolerance("append mixed batch, plan from lengths", out, decode_oracle(case),
                    literal=True)
    okc, ovc = _oracle_pools(case)
    assert np.array_equal(bits(kc), okc) and np.array_equal(bits(vc), ovc)
