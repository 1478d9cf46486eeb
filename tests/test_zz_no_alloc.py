"""pa_decode_noalloc (split-K pieces in the library's static per-GPU scratch)
against pa_decode + pa_decode_reduce with a caller workspace: bit-identical
outputs, and both within the literal bar of the oracle.  Two calls in a row,
the second with a smaller input, so the second call runs on scratch that
still holds the first call's (larger) pieces."""
import pytest
import torch

import paged_kv_gqa_write_amd as pa
import workloads
from _gpu_helpers import DEV, announce, check_tolerance, decode_oracle

pytestmark = pytest.mark.gpu


def _run(case, ps, P):
    kc, vc = case.k_cache.to(DEV), case.v_cache.to(DEV)
    pa.write_kv(case.k_new.to(DEV), case.v_new.to(DEV), case.slot_mapping.to(DEV), kc, vc)
    q, bt, ctx = case.q.to(DEV), case.block_tables.to(DEV), case.context_lens.to(DEV)
    ref = pa.decode(q, kc, vc, bt, ctx, case.scale, partition_size=ps, num_partitions=P)
    out = pa.decode_noalloc(q, kc, vc, bt, ctx, case.scale, ps, P)
    torch.cuda.synchronize()
    return out.cpu(), ref.cpu()


def test_noalloc_decode_matches_workspace_decode_on_consecutive_calls():
    big = workloads.hybrid_decode()             # 8 x 16 heads x 20 x 256: 2.6 MiB of pieces
    small = workloads.qwen3_4b_decode()         # 8 x 32 heads x 4 x 128: 0.5 MiB
    for case in (big, small):
        ps, P = pa.decode_split_plan_lens(case.num_kv_heads, case.context_lens)
        assert P > 1
        announce(f"decode_noalloc {case.name} ps={ps} P={P}")
        out, ref = _run(case, ps, P)
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), case.name
        check_tolerance(f"noalloc {case.name}", out, decode_oracle(case), literal=True)


def test_noalloc_one_partition_and_split_small_batch():
    case = workloads.make_decode_case("noalloc_small", context_lens=[37, 50, 1, 0],
                                      num_q_heads=8, num_kv_heads=2, head_dim=64,
                                      num_blocks=16, seed=17)
    for ps, P in ((64, 1), (16, 4)):
        announce(f"decode_noalloc small ps={ps} P={P}")
        out, ref = _run(case, ps, P)
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), (ps, P)
        check_tolerance(f"noalloc small P={P}", out, decode_oracle(case))


def test_noalloc_rejects_pieces_beyond_the_scratch():
    # 64 sequences x 64 heads x 8 partitions x (128 + 1) floats = 16.1 MiB
    announce("decode_noalloc too large")
    kc = torch.zeros(16, 8, 4, 16, 32, dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros(16, 8, 128, 16, dtype=torch.bfloat16, device=DEV)
    q = torch.zeros(64, 64, 128, dtype=torch.bfloat16, device=DEV)
    bt = torch.zeros(64, 1, dtype=torch.int32, device=DEV)
    ctx = torch.ones(64, dtype=torch.int32, device=DEV)
    out = torch.zeros(64, 64, 128, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(pa.PAError, match="TOO_LARGE"):
        pa.decode_noalloc(q, kc, vc, bt, ctx, 0.088, 512, 8, out=out)
    torch.cuda.synchronize()
    assert out.abs().sum().item() == 0          # nothing was enqueued
