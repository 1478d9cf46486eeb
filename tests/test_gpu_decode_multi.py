"""pa_decode_multi / pa_decode_multi_reduce (several query tokens per
sequence: verifying a drafted block) on the GPU against the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_gqa_write_amd as pa
import workloads
from _gpu_helpers import (DEV, announce, check_tolerance, decode_multi_gpu,
                          decode_multi_oracle, decode_multi_oracle_pools)
from _helpers import bits

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("batch", [1, 4, 8])
def test_verify_qwen3_4b_full_parity(batch):
    """The verify workload at full size (T = 8, context ~1.1k), its 8 new
    tokens appended by pa_write_kv first, in the library's split-K plan:
    every output element against the oracle.  Batches 1 and 4 launch fewer
    than 256 (partition, KV head, sequence) items, so the library gives each
    workgroup one 16-column tile; batch 8 reaches 256 and takes the
    two-tiles-per-wave form."""
    announce(f"decode_multi qwen3_4b_verify_b{batch}")
    case = workloads.qwen3_4b_verify(batch=batch)
    out = decode_multi_gpu(case)
    check_tolerance(case.name, out, decode_multi_oracle(case), literal=True)


def test_verify_head_dim_256_group_8_parity():
    """T = 8 on the hybrid models' full-attention shape (16/2 heads, head_dim
    256, contexts 4097 and 8192): 64 columns per KV head, two tiles per wave
    in two column chunks."""
    announce("decode_multi d256 g8 T=8")
    case = workloads.make_multi_decode_case("d256_verify", query_len=8,
                                            context_lens=[4097, 8192] * 4, num_q_heads=16,
                                            num_kv_heads=2, head_dim=256, num_blocks=8192,
                                            sigma=0.5, scale=1.0 / 16.0, seed=77)
    out = decode_multi_gpu(case)
    check_tolerance(case.name, out, decode_multi_oracle(case), literal=True)


# (Hq, Hkv, D, T): column counts T*G of 3..256, one to eight column chunks,
# group 1..16, all head dims.
SHAPES = [(4, 2, 64, 3), (32, 8, 128, 8), (64, 8, 128, 8), (16, 2, 256, 8), (16, 1, 64, 16),
          (8, 8, 128, 5), (12, 4, 128, 7), (32, 8, 128, 2), (16, 1, 256, 4), (6, 1, 128, 16)]


@pytest.mark.parametrize("hq,hkv,d,T", SHAPES)
def test_decode_multi_shapes_ragged(hq, hkv, d, T):
    """Ragged contexts (the shortest equal to T, so token 0 sees one key),
    whole-context and split partitions."""
    announce(f"decode_multi hq={hq} hkv={hkv} d={d} T={T}")
    case = workloads.make_multi_decode_case("ragged", query_len=T,
                                            context_lens=[T, 17 + T, 100, 300, 33],
                                            num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                                            num_blocks=64, seed=hq * 31 + d + T)
    ref = decode_multi_oracle(case)
    for ps, P in [(304, 1), (32, 10), (128, 3)]:
        out = decode_multi_gpu(case, partition_size=ps, num_partitions=P)
        check_tolerance(f"multi {hq}/{hkv}/{d} T={T} ps={ps}", out, ref)


@pytest.mark.parametrize("ps", [16, 64, 288, 1152])
def test_decode_multi_split_invariance(ps):
    announce(f"decode_multi split ps={ps}")
    case = workloads.qwen3_4b_verify(batch=4)
    out = decode_multi_gpu(case, partition_size=ps)
    check_tolerance(f"verify ps={ps}", out, decode_multi_oracle(case), literal=True)


def test_decode_multi_partials_match_oracle():
    """The split-K pieces: a partition holding no key visible to a token
    (past its causal limit, e.g. keys 96..111 for the first five tokens of the
    99-token sequence) must come back as 0 and -inf, the rest against the
    oracle's pieces."""
    announce("decode_multi partials")
    case = workloads.make_multi_decode_case("parts", query_len=8, context_lens=[40, 99, 8],
                                            num_q_heads=16, num_kv_heads=2, head_dim=128,
                                            num_blocks=32, seed=9)
    ps, P = 16, 7
    kc, vc = case.k_cache.to(DEV), case.v_cache.to(DEV)
    pa.write_kv(case.k_new.to(DEV), case.v_new.to(DEV), case.slot_mapping.to(DEV), kc, vc)
    po, pl = pa.decode_multi_partials(case.q.to(DEV), kc, vc, case.block_tables.to(DEV),
                                      case.context_lens.to(DEV), case.scale, ps, P)
    torch.cuda.synchronize()
    okc, ovc = decode_multi_oracle_pools(case)
    rpo, rpl = oracle.decode_multi_partials(bits(case.q), okc, ovc, case.block_tables.numpy(),
                                            case.context_lens.numpy(), case.scale, 16, 2, ps, P)
    gpo, gpl = po.cpu().double().numpy(), pl.cpu().double().numpy()
    fin = np.isfinite(rpl)
    assert np.array_equal(np.isfinite(gpl), fin)
    assert (gpl[~fin] == -np.inf).all() and (gpo[~fin] == 0).all()
    assert np.abs(gpl[fin] - rpl[fin]).max() < 1e-3
    err = np.abs(gpo - rpo)
    assert err.max() < 4e-3 and err.mean() < 5e-4, (err.max(), err.mean())
    out = pa.decode_multi_reduce(po, pl, case.context_lens.to(DEV), ps)
    torch.cuda.synchronize()
    check_tolerance("multi reduce of partials", out.cpu(), oracle.combine_partials(rpo, rpl))
    out_all = pa.decode_multi_reduce(po, pl, None, ps)     # reads every partition
    torch.cuda.synchronize()
    assert torch.equal(out_all.cpu(), out.cpu())


def test_decode_multi_one_token_equals_decode_bitwise():
    """T = 1 runs the same kernel as pa_decode: identical bits."""
    announce("decode_multi T=1 vs decode")
    case = workloads.qwen3_4b_decode()
    kc, vc = case.k_cache.to(DEV), case.v_cache.to(DEV)
    pa.write_kv(case.k_new.to(DEV), case.v_new.to(DEV), case.slot_mapping.to(DEV), kc, vc)
    args = (kc, vc, case.block_tables.to(DEV), case.context_lens.to(DEV), case.scale)
    for ps in (None, 1152):
        a = pa.decode(case.q.to(DEV), *args, max_context_len=1152, partition_size=ps)
        b = pa.decode_multi(case.q.to(DEV)[:, None].contiguous(), *args, max_context_len=1152,
                            partition_size=ps)
        torch.cuda.synchronize()
        assert torch.equal(a.cpu(), b[:, 0].cpu())


def test_decode_multi_matches_gpu_prefill():
    """The same tokens as a prefill after a cached prefix of ctx - T."""
    announce("decode_multi vs prefill")
    case = workloads.qwen3_4b_verify(batch=4)
    out = decode_multi_gpu(case)
    kc, vc = case.k_cache.to(DEV), case.v_cache.to(DEV)
    pa.write_kv(case.k_new.to(DEV), case.v_new.to(DEV), case.slot_mapping.to(DEV), kc, vc)
    T = case.query_len
    cu = (torch.arange(5, dtype=torch.int32) * T).to(DEV)
    pre = pa.prefill(case.q.reshape(4 * T, 32, 128).to(DEV), kc, vc, case.block_tables.to(DEV),
                     cu, (case.context_lens - T).to(DEV), case.scale, T)
    torch.cuda.synchronize()
    diff = (pre.cpu().float().reshape(out.shape) - out.float()).abs().max().item()
    assert diff <= 8e-3, diff


def test_decode_multi_zero_short_and_bad_sequences():
    """ctx == 0 gives zeros; 0 < ctx < T is invalid (NaN); a table entry
    outside the pool poisons only its sequence."""
    announce("decode_multi edge sequences")
    case = workloads.make_multi_decode_case("edge", query_len=6, context_lens=[0, 3, 50, 50],
                                            num_q_heads=8, num_kv_heads=2, head_dim=128,
                                            num_blocks=16, seed=21)
    ref = decode_multi_oracle(case)
    for ps, P in [(64, 1), (16, 4)]:
        out = decode_multi_gpu(case, partition_size=ps, num_partitions=P)
        assert out[0].float().abs().sum().item() == 0
        assert torch.isnan(out[1].float()).all()
        check_tolerance(f"edge ps={ps}", out[2:], ref[2:])
    case.block_tables[3, 1] = 500
    out = decode_multi_gpu(case, partition_size=16, num_partitions=4)
    assert torch.isnan(out[3].float()).all()
    check_tolerance("edge, good sequence", out[2:3], ref[2:3])


def test_decode_multi_repeat_runs_bitwise_identical():
    announce("decode_multi determinism")
    case = workloads.make_multi_decode_case("det", query_len=8, context_lens=[500, 77, 1200],
                                            num_q_heads=64, num_kv_heads=8, head_dim=128,
                                            num_blocks=160, seed=5)
    assert torch.equal(decode_multi_gpu(case, partition_size=128),
                       decode_multi_gpu(case, partition_size=128))
