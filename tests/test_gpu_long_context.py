"""Long contexts: decode over sequences of up to 65,536 tokens and prefill after
a 16,384-token cached prefix, against the oracle.

In decode, each wave fetches its pairs' block-table entries 32 pairs at a
time. A partition covering a whole 64k-token sequence gives every wave 512
pairs, i.e. 16 entry reloads, with the appended token in the last one. The
library's plan and a plan of 64 partitions of 1024 tokens cover the split
forms. The prefill case walks hundreds of key tiles per workgroup through
the table."""
import functools

import numpy as np
import pytest
import torch

import oracle
import paged_kv_gqa_write_amd as pa
import workloads
from _gpu_helpers import (DEV, announce, check_tolerance, decode_gpu, decode_oracle,
                          prefill_gpu, prefill_oracle)
from _helpers import bits

pytestmark = pytest.mark.gpu

LONG_LENS = [65536, 32771, 1, 40000]


@functools.lru_cache(maxsize=2)
def _long_decode_case(hq, hkv, d, seed):
    nb = sum((n + 15) // 16 for n in LONG_LENS) + 16
    return workloads.make_decode_case("long_context", context_lens=LONG_LENS, num_q_heads=hq,
                                      num_kv_heads=hkv, head_dim=d, num_blocks=nb, seed=seed)


@functools.lru_cache(maxsize=2)
def _long_decode_reference(hq, hkv, d, seed):
    """The oracle's output and pools after write_kv (read only by the tests)."""
    case = _long_decode_case(hq, hkv, d, seed)
    ek, ev = oracle.write_kv(bits(case.k_cache), bits(case.v_cache), bits(case.k_new),
                             bits(case.v_new), case.slot_mapping.numpy())
    return decode_oracle(case), ek, ev


@pytest.mark.parametrize("hq,hkv,d", [(16, 2, 128), (16, 2, 256)])
@pytest.mark.parametrize("ps,P", [(None, None), (1024, 64), (65536, 1)],
                         ids=["library_plan", "split_64x1024", "one_partition"])
def test_long_context_decode_append(hq, hkv, d, ps, P):
    """pa_decode_append over contexts up to 65,536 tokens: outputs against the
    oracle, pools bit-exact against the oracle's write_kv."""
    announce(f"long-context decode_append hq={hq} hkv={hkv} d={d} ps={ps} P={P}")
    case = _long_decode_case(hq, hkv, d, seed=d + 11)
    kc, vc = case.k_cache.to(DEV), case.v_cache.to(DEV)
    out = pa.decode_append(case.q.to(DEV), case.k_new.to(DEV), case.v_new.to(DEV), kc, vc,
                           case.block_tables.to(DEV), case.context_lens.to(DEV), case.scale,
                           max_context_len=max(LONG_LENS), partition_size=ps, num_partitions=P)
    torch.cuda.synchronize()
    ref, ek, ev = _long_decode_reference(hq, hkv, d, d + 11)
    check_tolerance(f"long-context decode_append d={d} ps={ps}", out.cpu(), ref)
    assert np.array_equal(bits(kc), ek) and np.array_equal(bits(vc), ev)


def test_long_context_decode_matches_append_bitwise():
    """pa_write_kv + pa_decode over the same long contexts, one partition:
    bit-identical to the appending kernel."""
    announce("long-context decode vs decode_append bitwise")
    case = _long_decode_case(16, 2, 128, seed=139)
    kc, vc = case.k_cache.to(DEV), case.v_cache.to(DEV)
    a = pa.decode_append(case.q.to(DEV), case.k_new.to(DEV), case.v_new.to(DEV), kc, vc,
                         case.block_tables.to(DEV), case.context_lens.to(DEV), case.scale,
                         max_context_len=max(LONG_LENS), partition_size=65536, num_partitions=1)
    torch.cuda.synchronize()
    assert torch.equal(a.cpu(), decode_gpu(case, partition_size=65536, num_partitions=1))


@pytest.mark.parametrize("hq,hkv,d", [(32, 8, 128), (16, 2, 256)])
def test_long_prefix_prefill(hq, hkv, d):
    """Prefill of 256 and 100 new tokens after cached prefixes of 16,384 and
    8,000 tokens (16,640 keys for the last row), against the oracle."""
    announce(f"long-prefix prefill hq={hq} hkv={hkv} d={d}")
    q_lens, prefix = [256, 100], [16384, 8000]
    nb = sum((n + p + 15) // 16 for n, p in zip(q_lens, prefix)) + 16
    case = workloads.make_prefill_case("long_prefix", q_lens=q_lens, prefix_lens=prefix,
                                       num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                                       num_blocks=nb, seed=d + 23)
    check_tolerance(f"long-prefix prefill d={d}", prefill_gpu(case), prefill_oracle(case))
