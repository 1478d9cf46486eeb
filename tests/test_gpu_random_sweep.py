"""Seeded random sweep over the decode, multi-token decode and prefill paths.

Each case draws its head shape (KV heads 1/2/4/8, group sizes 1-16 including
odd ones, head_dim 64/128/256), its batch, ragged lengths (a mix of short,
medium and long contexts; empty prefill sequences; prefixes that end
mid-block), and for decode the split plan (the library's, one partition, or
a random partition size) and the form (pa_decode_append, or pa_write_kv then
pa_decode).  Every output element is compared with the oracle, and the
appending form's pools bit for bit with the oracle's write_kv.  The fixed
cases elsewhere pick shapes by hand; this sweep covers the combinations
between them."""
import numpy as np
import pytest

import oracle
import paged_kv_gqa_write_amd as pa
import torch
import workloads
from _gpu_helpers import (DEV, announce, check_tolerance, decode_gpu, decode_multi_gpu,
                          decode_multi_oracle, decode_oracle, prefill_gpu, prefill_oracle)
from _helpers import bits

pytestmark = pytest.mark.gpu


def _shape(rng, max_hq=64):
    while True:
        hkv = int(rng.choice([1, 2, 4, 8]))
        g = int(rng.choice([1, 2, 3, 4, 5, 8, 16]))
        if hkv * g <= max_hq:
            return hkv * g, hkv, int(rng.choice([64, 128, 256]))


def _lengths(rng, n, lo=1):
    """A mix of short (lo..40), medium (41..700) and long (701..3000) lengths."""
    kind = rng.integers(0, 3, n)
    bounds = np.array([[lo, 40], [41, 700], [701, 3000]])
    return [int(rng.integers(bounds[k, 0], bounds[k, 1] + 1)) for k in kind]


def _blocks(lens):
    return sum((n + 15) // 16 for n in lens) + 8


@pytest.mark.parametrize("i", range(40))
def test_random_decode(i):
    rng = np.random.default_rng(1000 + i)
    hq, hkv, d = _shape(rng)
    lens = _lengths(rng, int(rng.integers(1, 11)))
    longest = max(lens)
    plan = int(rng.integers(0, 3))
    if plan == 0:
        ps = P = None                                  # the library's plan
    elif plan == 1:
        ps, P = (longest + 15) // 16 * 16, 1           # one partition
    else:
        ps = int(rng.choice([16, 32, 48, 64, 96, 128, 256, 512]))
        P = -(-longest // ps)
    append = bool(rng.integers(0, 2))
    announce(f"random decode {i}: hq={hq} hkv={hkv} d={d} lens={lens} ps={ps} P={P} "
             f"append={append}")
    case = workloads.make_decode_case(f"rand{i}", context_lens=lens, num_q_heads=hq,
                                      num_kv_heads=hkv, head_dim=d, num_blocks=_blocks(lens),
                                      seed=2000 + i)
    ref = decode_oracle(case)
    if append:
        kc, vc = case.k_cache.to(DEV), case.v_cache.to(DEV)
        out = pa.decode_append(case.q.to(DEV), case.k_new.to(DEV), case.v_new.to(DEV), kc, vc,
                               case.block_tables.to(DEV), case.context_lens.to(DEV), case.scale,
                               max_context_len=longest, partition_size=ps, num_partitions=P)
        torch.cuda.synchronize()
        ek, ev = oracle.write_kv(bits(case.k_cache), bits(case.v_cache), bits(case.k_new),
                                 bits(case.v_new), case.slot_mapping.numpy())
        assert np.array_equal(bits(kc), ek) and np.array_equal(bits(vc), ev)
        out = out.cpu()
    else:
        out = decode_gpu(case, partition_size=ps, num_partitions=P)
    check_tolerance(f"random decode {i}", out, ref)


@pytest.mark.parametrize("i", range(12))
def test_random_decode_multi(i):
    rng = np.random.default_rng(3000 + i)
    hq, hkv, d = _shape(rng, max_hq=32)
    T = int(rng.integers(2, 9))
    lens = _lengths(rng, int(rng.integers(1, 7)), lo=T)
    announce(f"random multi-token decode {i}: hq={hq} hkv={hkv} d={d} T={T} lens={lens}")
    case = workloads.make_multi_decode_case(f"randm{i}", query_len=T, context_lens=lens,
                                            num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                                            num_blocks=_blocks(lens), seed=4000 + i)
    check_tolerance(f"random multi-token decode {i}", decode_multi_gpu(case),
                    decode_multi_oracle(case))


@pytest.mark.parametrize("i", range(20))
def test_random_prefill(i):
    rng = np.random.default_rng(5000 + i)
    hq, hkv, d = _shape(rng, max_hq=32)
    S = int(rng.integers(1, 6))
    q_lens = [int(x) for x in rng.integers(0, 401, S)]
    if S > 1 and rng.integers(0, 2):
        q_lens[int(rng.integers(0, S))] = 0
    if max(q_lens) == 0:
        q_lens[0] = 1
    prefix = [int(x) for x in rng.integers(0, 601, S)]
    announce(f"random prefill {i}: hq={hq} hkv={hkv} d={d} q_lens={q_lens} prefix={prefix}")
    case = workloads.make_prefill_case(f"randp{i}", q_lens=q_lens, prefix_lens=prefix,
                                       num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                                       num_blocks=_blocks([n + p for n, p in zip(q_lens, prefix)]),
                                       seed=6000 + i)
    check_tolerance(f"random prefill {i}", prefill_gpu(case), prefill_oracle(case),
                    literal=False)
