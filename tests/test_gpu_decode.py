"""pa_decode / pa_decode_reduce on the GPU against the CPU oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
import paged_kv_gqa_write_amd as pa
import workloads
from _gpu_helpers import (DEV, announce, check_tolerance, decode_gpu, decode_oracle, gpu_f64)
from _helpers import bits, contiguous_twin, permuted_case

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", list(workloads.DECODE_CASES))
def test_decode_config_parity(name):
    """Every decode workload at full size, with its new token appended by
    pa_write_kv first, in the split-K plan the library picks (as benchmarked)."""
    announce(f"decode {name}")
    case = workloads.DECODE_CASES[name]()
    out = decode_gpu(case)
    ref = decode_oracle(case)
    check_tolerance(name, out, ref, literal=True)


@pytest.mark.parametrize("ps", [16, 32, 128, 256, 512, 1152])
def test_decode_split_invariance(ps):
    announce(f"decode split ps={ps}")
    case = workloads.qwen3_4b_decode()
    out = decode_gpu(case, partition_size=ps)
    check_tolerance(f"qwen3_4b ps={ps}", out, decode_oracle(case), literal=True)


def test_decode_partials_match_oracle():
    """The split-K pieces themselves (normalised partition outputs and LSEs)."""
    announce("decode partials long")
    case = workloads.qwen3_32b_decode_long()
    ps, P = 512, 16
    kc, vc = case.k_cache.to(DEV), case.v_cache.to(DEV)
    pa.write_kv(case.k_new.to(DEV), case.v_new.to(DEV), case.slot_mapping.to(DEV), kc, vc)
    po, pl = pa.decode_partials(case.q.to(DEV), kc, vc, case.block_tables.to(DEV),
                                case.context_lens.to(DEV), case.scale, ps, P)
    torch.cuda.synchronize()
    okc, ovc = oracle.write_kv(bits(case.k_cache), bits(case.v_cache), bits(case.k_new),
                               bits(case.v_new), case.slot_mapping.numpy())
    rpo, rpl = oracle.decode_partials(bits(case.q), okc, ovc, case.block_tables.numpy(),
                                      case.context_lens.numpy(), case.scale, case.num_q_heads,
                                      case.num_kv_heads, ps, P)
    gpo, gpl = po.cpu().double().numpy(), pl.cpu().double().numpy()
    assert np.abs(gpl - rpl).max() < 1e-3
    err = np.abs(gpo - rpo)
    assert err.max() < 4e-3 and err.mean() < 5e-4, (err.max(), err.mean())
    # the reduce of the GPU pieces equals the oracle's combine of its own pieces
    out = pa.decode_reduce(po, pl, case.context_lens.to(DEV), ps)
    torch.cuda.synchronize()
    check_tolerance("reduce of partials", out.cpu(), oracle.combine_partials(rpo, rpl))


def test_decode_reduce_handles_empty_and_single_partitions():
    announce("decode reduce edge")
    B, hq, P, D = 3, 4, 5, 64
    g = torch.Generator().manual_seed(3)
    po = torch.randn(B, hq, P, D, generator=g)
    pl = torch.randn(B, hq, P, generator=g) * 3
    pl[0, :, 1:] = -math.inf          # only partition 0 non-empty
    pl[1] = -math.inf                 # every partition empty -> zeros
    po[1] = 0
    out = pa.decode_reduce(po.to(DEV), pl.to(DEV), None, 16)
    torch.cuda.synchronize()
    ref = oracle.combine_partials(po.double().numpy(), pl.double().numpy())
    check_tolerance("reduce edge", out.cpu(), ref)
    assert torch.equal(out[0].cpu(), po[0, :, 0].to(torch.bfloat16))
    assert out[1].abs().sum().item() == 0


@pytest.mark.parametrize("hq,hkv,d", [(4, 4, 64), (8, 4, 128), (6, 2, 64), (16, 2, 256),
                                      (32, 8, 128), (16, 1, 128), (12, 4, 256)])
def test_decode_odd_lengths_and_groups(hq, hkv, d):
    announce(f"decode odd lengths hq={hq} hkv={hkv} d={d}")
    lens = [1, 15, 16, 17, 31, 33, 64, 100, 257]
    case = workloads.make_decode_case("odd", context_lens=lens, num_q_heads=hq, num_kv_heads=hkv,
                                      head_dim=d, num_blocks=64, seed=hq * 1000 + d)
    ref = decode_oracle(case)
    for ps in (None, 32, 64):
        out = decode_gpu(case, partition_size=ps)
        check_tolerance(f"odd {hq}/{hkv}/{d} ps={ps}", out, ref)


def test_single_token_context_returns_v_exactly():
    announce("decode ctx=1")
    case = workloads.make_decode_case("one", context_lens=[1] * 6, num_q_heads=16, num_kv_heads=4,
                                      head_dim=128, num_blocks=12, seed=9)
    out = decode_gpu(case)
    G = 4
    for s in range(6):
        for h in range(16):
            assert torch.equal(out[s, h], case.v_new[s, h // G])


def test_zero_context_gives_zeros():
    announce("decode ctx=0")
    case = workloads.make_decode_case("zero", context_lens=[0, 5, 0], num_q_heads=8,
                                      num_kv_heads=2, head_dim=64, num_blocks=4, seed=2)
    out = decode_gpu(case, partition_size=16, num_partitions=1)
    assert out[0].abs().sum().item() == 0 and out[2].abs().sum().item() == 0
    check_tolerance("zero ctx", out, decode_oracle(case))
    out2 = decode_gpu(case, partition_size=16, num_partitions=2)
    assert out2[0].abs().sum().item() == 0
    check_tolerance("zero ctx split", out2, decode_oracle(case))


def test_bad_block_entry_poisons_only_its_sequence():
    announce("decode bad table entry")
    case = workloads.make_decode_case("bad", context_lens=[40, 40, 40], num_q_heads=8,
                                      num_kv_heads=2, head_dim=128, num_blocks=16, seed=4)
    ref = decode_oracle(case)
    case.block_tables[1, 1] = 1000     # outside the 16-block pool
    case.block_tables[2, 0] = -3
    for ps in (None, 16):
        out = decode_gpu(case, partition_size=ps)
        assert torch.isnan(out[1].float()).all() and torch.isnan(out[2].float()).all()
        check_tolerance("bad entry, good sequence", out[:1], ref[:1])


def test_context_beyond_partitions_is_flagged():
    announce("decode ctx > P*ps")
    case = workloads.make_decode_case("cov", context_lens=[100, 20], num_q_heads=4,
                                      num_kv_heads=2, head_dim=64, num_blocks=16, seed=6)
    out = decode_gpu(case, partition_size=32, num_partitions=2)   # covers 64 < 100
    assert torch.isnan(out[0].float()).all()
    check_tolerance("covered sequence", out[1:], decode_oracle(case)[1:])


def test_block_permutation_and_contiguous_twin_bitwise():
    announce("decode permutation invariance")
    case = workloads.make_decode_case("perm", context_lens=[33, 300, 1000, 17], num_q_heads=32,
                                      num_kv_heads=8, head_dim=128, num_blocks=128, seed=12)
    base = decode_gpu(case, partition_size=128)
    g = torch.Generator().manual_seed(1)
    perm = torch.randperm(case.num_blocks, generator=g)
    k2 = torch.empty_like(case.k_cache)
    v2 = torch.empty_like(case.v_cache)
    k2[perm] = case.k_cache
    v2[perm] = case.v_cache
    bt = case.block_tables
    bt2 = torch.where(bt >= 0, perm[bt.clamp(min=0).long()].to(torch.int32), bt)
    slots2 = torch.tensor([int(bt2[s, (int(c) - 1) // 16]) * 16 + (int(c) - 1) % 16
                           for s, c in enumerate(case.context_lens)], dtype=torch.int64)
    case2 = workloads.DecodeCase(**{**case.__dict__, "k_cache": k2, "v_cache": v2,
                                    "block_tables": bt2, "slot_mapping": slots2})
    assert torch.equal(decode_gpu(case2, partition_size=128), base)
    # contiguous twin: identity-ordered blocks
    rows, nxt = [], 0
    k3 = torch.zeros_like(case.k_cache)
    v3 = torch.zeros_like(case.v_cache)
    bt3 = torch.full_like(bt, -1)
    for s, c in enumerate(case.context_lens.tolist()):
        nb = (c + 15) // 16
        for j in range(nb):
            k3[nxt + j] = case.k_cache[bt[s, j]]
            v3[nxt + j] = case.v_cache[bt[s, j]]
            bt3[s, j] = nxt + j
        nxt += nb
    slots3 = torch.tensor([int(bt3[s, (int(c) - 1) // 16]) * 16 + (int(c) - 1) % 16
                           for s, c in enumerate(case.context_lens)], dtype=torch.int64)
    case3 = workloads.DecodeCase(**{**case.__dict__, "k_cache": k3, "v_cache": v3,
                                    "block_tables": bt3, "slot_mapping": slots3})
    assert torch.equal(decode_gpu(case3, partition_size=128), base)


def test_decode_repeat_runs_bitwise_identical():
    announce("decode determinism")
    case = workloads.qwen3_32b_decode()
    a = decode_gpu(case)
    b = decode_gpu(case)
    assert torch.equal(a, b)


@pytest.mark.parametrize("ps,P", [(64, 1), (16, 3)], ids=["one_partition", "split"])
def test_negative_context_gives_nan_in_every_plan(ps, P):
    """A negative length is invalid device data: that sequence's output is
    NaN whether the decode kernel writes it (one partition) or the reduce
    combines split-K pieces; the others are unaffected."""
    announce(f"decode negative context ps={ps} P={P}")
    case = workloads.make_decode_case("neg", context_lens=[40, 40, 33], num_q_heads=8,
                                      num_kv_heads=2, head_dim=128, num_blocks=16, seed=14)
    ref = decode_oracle(case)
    case.context_lens[1] = -5
    case.slot_mapping[1] = -1
    out = decode_gpu(case, partition_size=ps, num_partitions=P)
    assert torch.isnan(out[1].float()).all()
    check_tolerance(f"negative context, others (P={P})", out[[0, 2]], ref[[0, 2]])


def test_decode_mixed_lengths_plan_parity():
    """One 8192-token request among seven of ~1100 tokens (Qwen3-32B heads)
    in the plan made from the batch's lengths: 15 partitions of 576 tokens
    (232 live workgroups of 960, ranked first) instead of 4 x 2048 from the
    longest alone; at the literal bar."""
    announce("decode qwen3_32b_decode_mixed_b8, plan from lengths")
    case = workloads.qwen3_32b_decode_mixed()
    ps, P = pa.decode_split_plan_lens(case.num_kv_heads, case.context_lens)
    assert (ps, P) == (576, 15)
    assert pa.decode_split_plan(case.batch, case.num_kv_heads, 8192, 256) == (2048, 4)
    out = decode_gpu(case, partition_size=ps, num_partitions=P)
    check_tolerance("mixed batch, plan from lengths", out, decode_oracle(case), literal=True)


def test_block_permutation_and_contiguous_twin_bitwise_split_plan_from_lengths():
    """Layout invariance of the mixed-length batch in its length-based plan."""
    announce("decode permutation invariance, mixed lengths")
    case = workloads.make_decode_case("permmix", context_lens=[4097, 300, 8192, 17],
                                      num_q_heads=16, num_kv_heads=2, head_dim=256,
                                      num_blocks=896, sigma=0.5, scale=1 / 16, seed=15)
    ps, P = pa.decode_split_plan_lens(case.num_kv_heads, case.context_lens)
    assert P > 1
    base = decode_gpu(case, partition_size=ps, num_partitions=P)
    assert torch.equal(decode_gpu(permuted_case(case, seed=2), partition_size=ps,
                                  num_partitions=P).view(torch.int16), base.view(torch.int16))
    assert torch.equal(decode_gpu(contiguous_twin(case), partition_size=ps,
                                  num_partitions=P).view(torch.int16), base.view(torch.int16))
    check_tolerance("mixed lengths", base, decode_oracle(case), literal=True)


@pytest.mark.parametrize("hkv,d,lens", [
    (2, 256, [4097, 300, 8192, 17, 0, 1000, 4097, 129]),
    (8, 128, [8192, 100, 100, 100]),                    # one long request among short ones
    (4, 64, [1, 2000, 33, 2000, 700, 64])])
def test_decode_partials_mixed_lengths_every_piece(hkv, d, lens):
    """In a mixed batch the launch ranks the (sequence, partition) pairs
    that hold keys first and the empty ones last; every piece must still be
    written exactly once: each partial output and LSE against the oracle's,
    empty partitions included (0 and -inf), then the reduce."""
    announce(f"decode partials mixed lengths hkv={hkv} d={d}")
    hq = 8 * hkv
    case = workloads.make_decode_case("mixparts", context_lens=lens, num_q_heads=hq,
                                      num_kv_heads=hkv, head_dim=d,
                                      num_blocks=sum(-(-c // 16) for c in lens) + 4,
                                      sigma=0.5, seed=hkv * 10 + d)
    ps, P = pa.decode_split_plan_lens(hkv, case.context_lens)
    assert P > 1
    kc, vc = case.k_cache.to(DEV), case.v_cache.to(DEV)
    pa.write_kv(case.k_new.to(DEV), case.v_new.to(DEV), case.slot_mapping.to(DEV), kc, vc)
    po = torch.full((len(lens), hq, P, d), float("nan"), device=DEV)   # unwritten stays NaN
    pl = torch.full((len(lens), hq, P), float("nan"), device=DEV)
    pa.decode_partials(case.q.to(DEV), kc, vc, case.block_tables.to(DEV),
                       case.context_lens.to(DEV), case.scale, ps, P, part_out=po, part_lse=pl)
    torch.cuda.synchronize()
    okc, ovc = oracle.write_kv(bits(case.k_cache), bits(case.v_cache), bits(case.k_new),
                               bits(case.v_new), case.slot_mapping.numpy())
    rpo, rpl = oracle.decode_partials(bits(case.q), okc, ovc, case.block_tables.numpy(),
                                      case.context_lens.numpy(), case.scale, hq, hkv, ps, P)
    gpo, gpl = po.cpu().double().numpy(), pl.cpu().double().numpy()
    assert np.isfinite(gpo).all()
    empty = np.isneginf(rpl)
    assert np.array_equal(np.isneginf(gpl), empty)
    assert np.abs(gpl[~empty] - rpl[~empty]).max() < 1e-3
    assert (gpo[empty] == 0).all()
    err = np.abs(gpo - rpo)
    assert err.max() < 4e-3 and err.mean() < 5e-4, (err.max(), err.mean())
    out = pa.decode_reduce(po, pl, case.context_lens.to(DEV), ps)
    torch.cuda.synchronize()
    check_tolerance(f"mixed reduce hkv={hkv} d={d}", out.cpu(), decode_oracle(case),
                    literal=True)
