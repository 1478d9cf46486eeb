"""The decode step captured as a HIP graph and replayed ("Qwen3-4B / 8B / 32B",
Architecture Notes: decode runs as graph replay with pre-allocated buffers).

The library allocates, frees and synchronises nothing and issues no memset,
so a layer stack of pa_write_kv + pa_decode + pa_decode_reduce launches (or
pa_decode_append + pa_decode_reduce) can be captured once and replayed.
Each replay, with eager work and host synchronisation in between, must
reproduce the eager result bit for bit."""
import pytest
import torch

import paged_kv_gqa_write_amd as pa
import workloads
from _gpu_helpers import DEV, announce

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fused", [False, True], ids=["write_then_decode", "decode_append"])
def test_graph_replayed_decode_step_matches_eager_bitwise(fused):
    announce(f"graph-captured decode step fused={fused}")
    layers = 3
    case = workloads.qwen3_4b_decode(poison=False)
    B, hq, hkv, d = case.batch, case.num_q_heads, case.num_kv_heads, case.head_dim
    g = torch.Generator(device=DEV)
    g.manual_seed(7)
    base_k = [torch.randn(case.k_cache.shape, generator=g, device=DEV).to(torch.bfloat16)
              for _ in range(layers)]
    base_v = [torch.randn(case.v_cache.shape, generator=g, device=DEV).to(torch.bfloat16)
              for _ in range(layers)]
    q = [torch.randn(case.q.shape, generator=g, device=DEV).to(torch.bfloat16)
         for _ in range(layers)]
    k_new = case.k_new.to(DEV)
    v_new = case.v_new.to(DEV)
    slots, bt, ctx = case.slot_mapping.to(DEV), case.block_tables.to(DEV), case.context_lens.to(DEV)
    ps, P = pa.decode_split_plan(B, hkv, int(case.context_lens.max()))
    assert P > 1  # the step includes the reduce
    kc = [t.clone() for t in base_k]
    vc = [t.clone() for t in base_v]
    outs = [torch.empty(B, hq, d, dtype=torch.bfloat16, device=DEV) for _ in range(layers)]
    po = torch.empty(B, hq, P, d, dtype=torch.float32, device=DEV)
    pl = torch.empty(B, hq, P, dtype=torch.float32, device=DEV)

    def step():
        for i in range(layers):
            if fused:
                pa.decode_append(q[i], k_new, v_new, kc[i], vc[i], bt, ctx, case.scale,
                                 partition_size=ps, num_partitions=P, out=outs[i], part_out=po,
                                 part_lse=pl)
            else:
                pa.write_kv(k_new, v_new, slots, kc[i], vc[i])
                pa.decode(q[i], kc[i], vc[i], bt, ctx, case.scale, partition_size=ps,
                          num_partitions=P, out=outs[i], part_out=po, part_lse=pl)

    step()                                   # eager reference
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    ref_k = [t.clone() for t in kc]

    side = torch.cuda.Stream(device=DEV)     # default priority
    side.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(side):
        step()                               # warm-up on the capture stream
    torch.cuda.current_stream(DEV).wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for r in range(3):
        for o in outs:
            o.fill_(0)                       # eager work between replays
        for i in range(layers):
            kc[i].copy_(base_k[i])
            vc[i].copy_(base_v[i])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i in range(layers):
            assert torch.equal(outs[i].view(torch.int16), ref[i].view(torch.int16)), (r, i)
            assert torch.equal(kc[i].view(torch.int16), ref_k[i].view(torch.int16)), (r, i)
