"""The decode step captured as a HIP graph and replayed ("Qwen3-4B / 8B / 32B",
Architecture Notes: decode runs as graph replay with pre-allocated buffers).

The library allocates, frees and synchronises nothing and issues no memset,
so a layer stack of pa_write_kv + pa_decode + pa_decode_reduce launches (or
pa_decode_append + pa_decode_reduce) can be captured once and replayed.
Every layer has its own seeded pools and queries (NaN in every slot that
holds no live token).  Each replay, with eager work and host
synchronisation in between, is checked against the oracle (write_kv of the
new tokens, then decode) at the literal bar, with both pools bit-exact,
and against the eager run bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_gqa_write_amd as pa
import workloads
from _gpu_helpers import DEV, announce, check_tolerance
from _helpers import bits

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fused", [False, True], ids=["write_then_decode", "decode_append"])
def test_graph_replayed_decode_step_matches_oracle(fused):
    announce(f"graph-captured decode step fused={fused}")
    layers = 3
    base = workloads.qwen3_4b_decode()
    cases = [base] + [workloads.decode_layer(base, seed=1000 + i) for i in range(1, layers)]
    B, hq, hkv, d = base.batch, base.num_q_heads, base.num_kv_heads, base.head_dim
    # the oracle: each layer's new token written, then decode
    ref_pools, ref_out = [], []
    for c in cases:
        okc, ovc = oracle.write_kv(bits(c.k_cache), bits(c.v_cache), bits(c.k_new),
                                   bits(c.v_new), c.slot_mapping.numpy())
        ref_pools.append((okc, ovc))
        ref_out.append(oracle.decode(bits(c.q), okc, ovc, c.block_tables.numpy(),
                                     c.context_lens.numpy(), c.scale, hq, hkv))

    bt, ctx = base.block_tables.to(DEV), base.context_lens.to(DEV)
    slots = base.slot_mapping.to(DEV)
    q = [c.q.to(DEV) for c in cases]
    k_new = [c.k_new.to(DEV) for c in cases]
    v_new = [c.v_new.to(DEV) for c in cases]
    base_k = [c.k_cache.to(DEV) for c in cases]
    base_v = [c.v_cache.to(DEV) for c in cases]
    ps, P = pa.decode_split_plan(B, hkv, int(base.context_lens.max()))
    assert P > 1  # the step includes the reduce
    kc = [t.clone() for t in base_k]
    vc = [t.clone() for t in base_v]
    outs = [torch.empty(B, hq, d, dtype=torch.bfloat16, device=DEV) for _ in range(layers)]
    po = torch.empty(B, hq, P, d, dtype=torch.float32, device=DEV)
    pl = torch.empty(B, hq, P, dtype=torch.float32, device=DEV)

    def step():
        for i in range(layers):
            if fused:
                pa.decode_append(q[i], k_new[i], v_new[i], kc[i], vc[i], bt, ctx, base.scale,
                                 partition_size=ps, num_partitions=P, out=outs[i], part_out=po,
                                 part_lse=pl)
            else:
                pa.write_kv(k_new[i], v_new[i], slots, kc[i], vc[i])
                pa.decode(q[i], kc[i], vc[i], bt, ctx, base.scale, partition_size=ps,
                          num_partitions=P, out=outs[i], part_out=po, part_lse=pl)

    def check(tag):
        for i in range(layers):
            check_tolerance(f"{tag} layer {i}", outs[i].cpu(), ref_out[i], literal=True)
            assert np.array_equal(bits(kc[i]), ref_pools[i][0]), (tag, i)
            assert np.array_equal(bits(vc[i]), ref_pools[i][1]), (tag, i)

    step()                                   # eager reference
    torch.cuda.synchronize()
    check("eager")
    eager = [o.clone() for o in outs]

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
        check(f"replay {r}")
        for i in range(layers):
            assert torch.equal(outs[i].view(torch.int16), eager[i].view(torch.int16)), (r, i)
