"""Benchmark: paged GQA decode KV GB/s and prefill TFLOP/s on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--legs a,b,...]

Headline step: one decode step of a Qwen3-32B-shaped attention stack
("Qwen3-4B / 8B / 32B", sections Architecture Notes and Qwen3-32B Serving
Load: 64 query heads, GQA group 8, head_dim 128, 64 layers; 64 requests in
flight, the server's default decode batch).  For every layer each
sequence's new token is appended and decode runs over contexts of 1024-1152
tokens scattered over an 8192-block pool (pa_decode_append, one kernel).
Every layer has its own pools (512 MiB each, 32 GiB in all), so the step
streams 64 x 286.5 MB of KV from HBM, far more than the 256 MB Infinity
Cache holds.  `value` = the step's KV bytes / step time.

The other workloads are legs of the same JSON line, each with its own
roofline object for its dominant kernel:
  qwen3_32b_decode_b4_8192  batch 4 at 8192 tokens: split-K + reduce, 64 layers
  qwen3_32b_decode_mixed_b8 one 8192-token request among seven of 1024-1152:
                            split plan from the batch's lengths (live work
                            ranked first), beside the plan from the longest
  hybrid_decode_b8          16/2 heads, head_dim 256, contexts 4097/8192, plan
                            from the batch's lengths; 16 layers' pools
  hybrid_prefill_4097       one 4097-token causal prefill (16/2/256); 16 layers
  qwen3_4b_decode_b8        32/8/128 batch 8, 36 layers: the step, the step as
                            a replayed HIP graph, the step with a separate
                            pa_write_kv; per-layer kernel / reduce / gap split
  qwen3_4b_prefill_4x1024   4 x 1024 new tokens (two after 512 cached), 36 layers
  write_kv                  pa_write_kv of those 4096 tokens
  verify                    4 x 8 query tokens (a drafted block) per layer
  kv_restore                host-tier restore of a 16k-token prefix
  prefix_match              the host prefix-block index
Kernel rooflines: algorithmic bytes (or flops) per launch / the average
launch duration of the leg's launches re-issued back to back between HIP
events on the launch stream.  cpu_baseline = the CPU fp64 oracle timed on
a bounded sample of the headline workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
METRIC = "paged GQA decode KV GB/s (% of HBM peak); prefill TFLOP/s (% of MFMA peak)"
HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 matrix peak
HEADLINE = "qwen3_32b_decode_b64"
LEGS = [HEADLINE, "qwen3_32b_decode_b4_8192", "qwen3_32b_decode_mixed_b8", "hybrid_decode_b8",
        "hybrid_prefill_4097",
        "qwen3_4b_decode_b8", "qwen3_4b_prefill_4x1024", "write_kv", "verify", "kv_restore",
        "prefix_match"]
DECODE_SOURCES = ["decode.hip", "pa_device.h"]
PREFILL_SOURCES = ["prefill.hip", "pa_device.h"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--legs", default="all",
                    help="comma-separated legs to run (default: all): " + ", ".join(LEGS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    args = ap.parse_args()
    args.legs = LEGS if args.legs == "all" else [x for x in args.legs.split(",") if x]
    for x in args.legs:
        if x not in LEGS:
            ap.error(f"unknown leg {x}")
    return args


def source_hash(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "paged_kv_gqa_write_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(leg, sources):
    """HBM bytes per launch of the leg's dominant kernel from committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE runs, if they were taken on the
    current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", f"traffic_{leg}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        rec = json.load(f)
    if rec.get("source_hash") != source_hash(sources):
        return None
    return rec.get("hbm_bytes_per_launch")


class Ctx:
    """What every leg needs: the library, the device, the launch stream and a
    seeded device generator for the extra layers' pools."""

    def __init__(self, args):
        import torch
        import paged_kv_gqa_write_amd as pa
        self.torch, self.pa, self.args = torch, pa, args
        self.lib = pa.load_library()
        self.dev = torch.device("cuda:0")
        torch.cuda.set_device(self.dev)
        self.stream = torch.cuda.current_stream(self.dev)
        self.sptr = self.stream.cuda_stream
        self.gen = torch.Generator(device=self.dev)
        self.gen.manual_seed(42)
        self.cus = torch.cuda.get_device_properties(0).multi_processor_count

    def per_call_ms(self, fn, count):
        """fn(i) for i < count between two HIP events on the launch stream."""
        torch = self.torch
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(self.stream)
        for i in range(count):
            fn(i)
        b.record(self.stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / count

    def layer_pools(self, case, layers):
        """Layer 0 holds the seeded case's own pools, the others random bf16
        from the seeded device generator (finite values, same shapes).

        A leg's pools go back to torch's caching allocator when it ends, never
        to the driver (no empty_cache): for a few seconds after tens of GiB
        are released, every kernel on the GPU streams ~5% slower (Qwen3-32B
        4 x 8192 decode: 24.1 us per launch before a 32 GiB release, 25.2 us
        right after it, 24.1 us again after 5 s idle), which would charge one
        leg's teardown to the next leg's timings.  A serving process
        allocates its KV pools once and keeps them."""
        torch = self.torch
        kc, vc = [case.k_cache.to(self.dev)], [case.v_cache.to(self.dev)]
        for _ in range(1, layers):
            kc.append((torch.randn(kc[0].shape, generator=self.gen, device=self.dev)
                       * case.sigma).to(torch.bfloat16))
            vc.append((torch.randn(vc[0].shape, generator=self.gen, device=self.dev)
                       * case.sigma).to(torch.bfloat16))
        return kc, vc


def ok(st, what):
    if st != 0:
        raise RuntimeError(f"{what} failed with status {st}")


def roofline_hbm(nbytes, us, kernel, leg, sources=DECODE_SOURCES):
    gbps = nbytes / (us * 1e-6) / 1e9
    return {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": measured_traffic(leg, sources),
            "kernel": kernel, "algorithmic_bytes_per_launch": int(nbytes),
            "avg_launch_us": round(us, 3)}


def roofline_mfma(flops, us, kernel, leg):
    tf = flops / (us * 1e-6) / 1e12
    return {"bound": "mfma", "achieved": round(tf, 2), "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4),
            "traffic": measured_traffic(leg, PREFILL_SOURCES), "kernel": kernel,
            "algorithmic_flops_per_launch": int(flops), "avg_launch_us": round(us, 3)}


def decode_leg(c, name, case, layers, plan_from_lengths, detail=False, compare_max_plan=False):
    """One decode step = for every layer, pa_decode_append (append each
    sequence's new token and decode) and, with more than one partition,
    pa_decode_reduce.  Reports the step rate and the appending decode
    kernel's roofline; detail=True adds the per-layer split (kernel, reduce,
    launch gaps), the step replayed from a HIP graph and the step with a
    separate pa_write_kv."""
    torch, lib, dev, sptr, args = c.torch, c.lib, c.dev, c.sptr, c.args
    B, hq, hkv, d, nb = case.batch, case.num_q_heads, case.num_kv_heads, case.head_dim, \
        case.num_blocks
    L = layers
    kc, vc = c.layer_pools(case, L)
    q, k_new, v_new = case.q.to(dev), case.k_new.to(dev), case.v_new.to(dev)
    slots, bt, ctx = case.slot_mapping.to(dev), case.block_tables.to(dev), \
        case.context_lens.to(dev)
    if plan_from_lengths:
        ps, P = c.pa.decode_split_plan_lens(hkv, case.context_lens, c.cus)
    else:
        ps, P = c.pa.decode_split_plan(B, hkv, int(case.context_lens.max()), c.cus)
    out = torch.empty(B, hq, d, dtype=torch.bfloat16, device=dev)
    part_out = torch.empty(B, hq, P, d, dtype=torch.float32, device=dev)
    part_lse = torch.empty(B, hq, P, dtype=torch.float32, device=dev)
    mb = bt.shape[1]

    def append_decode(i, s=sptr):
        ok(lib.pa_decode_append(out.data_ptr(), part_out.data_ptr() if P > 1 else 0,
                                part_lse.data_ptr() if P > 1 else 0, q.data_ptr(),
                                k_new.data_ptr(), v_new.data_ptr(), kc[i % L].data_ptr(),
                                vc[i % L].data_ptr(), bt.data_ptr(), ctx.data_ptr(), B, hq, hkv,
                                d, 16, nb, mb, ps, P, case.scale, s), "pa_decode_append")

    def reduce(i, s=sptr):
        ok(lib.pa_decode_reduce(out.data_ptr(), part_out.data_ptr(), part_lse.data_ptr(),
                                ctx.data_ptr(), B, hq, d, ps, P, s), "pa_decode_reduce")

    def step(_=0, s=sptr):
        for i in range(L):
            append_decode(i, s)
            if P > 1:
                reduce(i, s)

    for _ in range(args.warmup):
        step()
    ms = c.per_call_ms(step, args.steps)
    kvb = case.kv_bytes()
    dec_us = c.per_call_ms(append_decode, args.steps * L) * 1e3
    res = {"workload": name, "layers": L, "batch": B, "num_q_heads": hq, "num_kv_heads": hkv,
           "head_dim": d, "context_lens": sorted(set(case.context_lens.tolist()))
           if B > 8 else case.context_lens.tolist(),
           "num_blocks_per_layer": nb, "partition_size": ps, "num_partitions": P,
           "split_plan": "from the batch's lengths" if plan_from_lengths else "from the longest",
           "kv_bytes_per_layer": kvb, "ms_per_step": round(ms, 4),
           "value": round(kvb * L / (ms * 1e-3) / 1e9, 1), "unit": "GB/s",
           "roofline": roofline_hbm(kvb, dec_us, f"decode_kernel<{d}> (appending form)", name)}
    if B > 8:
        res["context_len_range"] = [int(case.context_lens.min()), int(case.context_lens.max())]
        res.pop("context_lens")
    if P > 1:
        red_us = c.per_call_ms(reduce, args.steps * L) * 1e3
        res["reduce_avg_launch_us"] = round(red_us, 3)
    if compare_max_plan:
        mps, mP = c.pa.decode_split_plan(B, hkv, int(case.context_lens.max()), c.cus)
        mpo = torch.empty(B, hq, mP, d, dtype=torch.float32, device=dev)
        mpl = torch.empty(B, hq, mP, dtype=torch.float32, device=dev)

        def append_decode_max(i):
            ok(lib.pa_decode_append(out.data_ptr(), mpo.data_ptr(), mpl.data_ptr(), q.data_ptr(),
                                    k_new.data_ptr(), v_new.data_ptr(), kc[i % L].data_ptr(),
                                    vc[i % L].data_ptr(), bt.data_ptr(), ctx.data_ptr(), B, hq,
                                    hkv, d, 16, nb, mb, mps, mP, case.scale, sptr),
               "pa_decode_append")

        append_decode_max(0)
        m_us = c.per_call_ms(append_decode_max, args.steps * L) * 1e3
        res["plan_from_longest"] = {"partition_size": mps, "num_partitions": mP,
                                    "kernel_avg_launch_us": round(m_us, 3),
                                    "frac": round(kvb / (m_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}
    if detail:
        layer_us = ms * 1e3 / L
        red_us = res.get("reduce_avg_launch_us", 0.0)
        res["per_layer_us"] = {
            "step_per_layer": round(layer_us, 3), "decode_kernel_back_to_back": round(dec_us, 3),
            "reduce_kernel_back_to_back": round(red_us, 3),
            "note": "kernel averages from back-to-back launches of one kernel; the split of "
                    "the step itself (kernel durations and the gaps between them) comes from "
                    "the rocprofv3 kernel trace"}
        # the same step captured once as a HIP graph and replayed
        side = torch.cuda.Stream(device=dev)
        side.wait_stream(c.stream)
        with torch.cuda.stream(side):
            step(0, side.cuda_stream)
        c.stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step(0, torch.cuda.current_stream(dev).cuda_stream)
        for _ in range(args.warmup):
            graph.replay()
        gms = c.per_call_ms(lambda i: graph.replay(), args.steps)
        del graph
        res["step_graph_replay"] = {"ms_per_step": round(gms, 4),
                                    "value": round(kvb * L / (gms * 1e-3) / 1e9, 1),
                                    "unit": "GB/s"}

        # the same step with the append as its own kernel
        def split_step(_=0):
            for i in range(L):
                ok(lib.pa_write_kv(k_new.data_ptr(), v_new.data_ptr(), slots.data_ptr(),
                                   kc[i].data_ptr(), vc[i].data_ptr(), B, hkv, d, 16, nb, sptr),
                   "pa_write_kv")
                ok(lib.pa_decode(out.data_ptr(), part_out.data_ptr() if P > 1 else 0,
                                 part_lse.data_ptr() if P > 1 else 0, q.data_ptr(),
                                 kc[i].data_ptr(), vc[i].data_ptr(), bt.data_ptr(),
                                 ctx.data_ptr(), B, hq, hkv, d, 16, nb, mb, ps, P, case.scale,
                                 sptr), "pa_decode")
                if P > 1:
                    reduce(i)

        split_step()
        sms = c.per_call_ms(split_step, args.steps)
        res["step_separate_write_kv"] = {"ms_per_step": round(sms, 4),
                                         "value": round(kvb * L / (sms * 1e-3) / 1e9, 1),
                                         "unit": "GB/s"}
    del kc, vc
    return res


def prefill_leg(c, name, case, layers, write_kv_leg=False):
    """Per layer: pa_write_kv of the new tokens, then pa_prefill.  Reports
    the step rate and the prefill kernel's roofline (and, optionally, the
    pa_write_kv kernel's)."""
    torch, lib, dev, sptr, args = c.torch, c.lib, c.dev, c.sptr, c.args
    L = layers
    kc, vc = c.layer_pools(case, L)
    q, kn, vn = case.q.to(dev), case.k_new.to(dev), case.v_new.to(dev)
    slots, bt = case.slot_mapping.to(dev), case.block_tables.to(dev)
    cu, pre = case.cu_seqlens.to(dev), case.prefix_lens.to(dev)
    out = torch.empty_like(q)
    T, hq, hkv, d, nb = case.total_q, case.num_q_heads, case.num_kv_heads, case.head_dim, \
        case.num_blocks
    maxq = max(case.q_lens)

    def wkv(i):
        ok(lib.pa_write_kv(kn.data_ptr(), vn.data_ptr(), slots.data_ptr(), kc[i % L].data_ptr(),
                           vc[i % L].data_ptr(), T, hkv, d, 16, nb, sptr), "pa_write_kv")

    def pf(i):
        ok(lib.pa_prefill(out.data_ptr(), q.data_ptr(), kc[i % L].data_ptr(),
                          vc[i % L].data_ptr(), bt.data_ptr(), cu.data_ptr(), pre.data_ptr(),
                          case.num_seqs, T, maxq, hq, hkv, d, 16, nb, bt.shape[1], case.scale,
                          sptr), "pa_prefill")

    def step(_=0):
        for i in range(L):
            wkv(i)
            pf(i)

    for _ in range(args.warmup):
        step()
    ms = c.per_call_ms(step, args.steps)
    flops = case.flops()
    pf_us = c.per_call_ms(pf, args.steps * L) * 1e3
    res = {"workload": name, "layers": L, "q_lens": case.q_lens,
           "prefix_lens": case.prefix_lens_list, "num_q_heads": hq, "num_kv_heads": hkv,
           "head_dim": d, "algorithmic_flops_per_layer": flops, "ms_per_step": round(ms, 4),
           "value": round(flops * L / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
           "roofline": roofline_mfma(flops, pf_us, f"prefill_kernel<{d}>", name)}
    wk = None
    if write_kv_leg:
        wkv_us = c.per_call_ms(wkv, args.steps * L) * 1e3
        wbytes = 2 * 2 * T * hkv * d * 2     # K and V, read and written
        wk = {"workload": f"pa_write_kv of the {T} new tokens of {name} ({hkv} KV heads, "
                          f"head_dim {d}), back to back over {L} layers' pools",
              "roofline": roofline_hbm(wbytes, wkv_us, f"write_kv_kernel<{d}>", "write_kv",
                                       ["write_kv.hip", "pa_device.h"])}
    del kc, vc
    return res, wk


def verify_leg(c):
    """The pass that checks a drafted block ("Qwen3-4B / 8B / 32B", section
    DSpark Speculative Decoding): per layer the T = 8 query tokens' K/V are
    appended (pa_write_kv, 32 tokens), then pa_decode_multi and
    pa_decode_multi_reduce run over contexts of 1024-1152 tokens."""
    torch, lib, dev, sptr, args, pa = c.torch, c.lib, c.dev, c.sptr, c.args, c.pa
    import workloads
    case = workloads.qwen3_4b_verify(batch=4, poison=False)
    B, T, hq, hkv, d = case.batch, case.query_len, case.num_q_heads, case.num_kv_heads, \
        case.head_dim
    nb, L = case.num_blocks, 36
    kc, vc = c.layer_pools(case, L)
    q = case.q.to(dev)
    k_new, v_new, slots = case.k_new.to(dev), case.v_new.to(dev), case.slot_mapping.to(dev)
    bt, ctx = case.block_tables.to(dev), case.context_lens.to(dev)
    ps, P = pa.decode_multi_split_plan(B, T, hq, hkv, int(case.context_lens.max()), c.cus)
    out = torch.empty(B, T, hq, d, dtype=torch.bfloat16, device=dev)
    part_out = torch.empty(B, T, hq, P, d, dtype=torch.float32, device=dev)
    part_lse = torch.empty(B, T, hq, P, dtype=torch.float32, device=dev)

    def multi(i):
        ok(lib.pa_decode_multi(out.data_ptr(), part_out.data_ptr(), part_lse.data_ptr(),
                               q.data_ptr(), kc[i % L].data_ptr(), vc[i % L].data_ptr(),
                               bt.data_ptr(), ctx.data_ptr(), B, T, hq, hkv, d, 16, nb,
                               bt.shape[1], ps, P, case.scale, sptr), "pa_decode_multi")

    def step(_=0):
        for i in range(L):
            ok(lib.pa_write_kv(k_new.data_ptr(), v_new.data_ptr(), slots.data_ptr(),
                               kc[i].data_ptr(), vc[i].data_ptr(), B * T, hkv, d, 16, nb, sptr),
               "pa_write_kv")
            multi(i)
            if P > 1:
                ok(lib.pa_decode_multi_reduce(out.data_ptr(), part_out.data_ptr(),
                                              part_lse.data_ptr(), ctx.data_ptr(), B, T, hq, d,
                                              ps, P, sptr), "pa_decode_multi_reduce")

    for _ in range(args.warmup):
        step()
    ms = c.per_call_ms(step, args.steps)
    k_us = c.per_call_ms(multi, args.steps * L) * 1e3
    kvb = case.kv_bytes()
    del kc, vc
    return {"workload": f"{case.name}: 4 sequences x 8 query tokens (last accepted + 7 "
                        "drafted), context 1024-1152, 32/8 heads, head_dim 128, 36 layers "
                        "(write_kv + decode_multi + reduce per layer)",
            "value": round(kvb * L / (ms * 1e-3) / 1e9, 1), "unit": "GB/s",
            "ms_per_step": round(ms, 4), "partition_size": ps, "num_partitions": P,
            "roofline": roofline_hbm(kvb, k_us, "decode_kernel<128> (multi-token form)",
                                     "verify")}


def restore_leg(c):
    """Host-tier restore ("Qwen3-4B / 8B / 32B", section KV Offload): the
    1024 sealed blocks of a 16384-token Qwen3-4B prefix, per layer, copied by
    pa_copy_blocks from packed pinned host buffers into scattered pool blocks
    (the kernel reads host memory directly).  8 host buffers (64 MiB each)
    rotate over the layers.  Also: the same 1024 blocks duplicated inside
    the device pool (HBM read + write), and a plain 64 MiB host-to-device
    DMA copy of one buffer for the host link's reference rate."""
    torch, lib, dev, sptr, args = c.torch, c.lib, c.dev, c.sptr, c.args
    hkv, d, n, nb, nh = 8, 128, 1024, 4096, 8
    blk = hkv * 16 * d * 2
    kc = torch.empty((nb, hkv, d // 32, 16, 32), dtype=torch.bfloat16, device=dev)
    vc = torch.empty((nb, hkv, d, 16), dtype=torch.bfloat16, device=dev)
    hk = [torch.zeros((n, hkv, d // 32, 16, 32), dtype=torch.bfloat16, pin_memory=True)
          for _ in range(nh)]
    hv = [torch.zeros((n, hkv, d, 16), dtype=torch.bfloat16, pin_memory=True) for _ in range(nh)]
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    perm = torch.randperm(nb, generator=g, device=dev).to(torch.int32)
    dst, cow_src, cow_dst = (perm[:n].contiguous(), perm[n:2 * n].contiguous(),
                             perm[2 * n:3 * n].contiguous())
    stage_k = torch.empty_like(kc[:n])

    def restore(i):
        ok(lib.pa_copy_blocks(kc.data_ptr(), vc.data_ptr(), nb, dst.data_ptr(),
                              hk[i % nh].data_ptr(), hv[i % nh].data_ptr(), n, None, n, hkv, d,
                              16, sptr), "pa_copy_blocks")

    def cow(i):
        ok(lib.pa_copy_blocks(kc.data_ptr(), vc.data_ptr(), nb, cow_dst.data_ptr(),
                              kc.data_ptr(), vc.data_ptr(), nb, cow_src.data_ptr(), n, hkv, d,
                              16, sptr), "pa_copy_blocks")

    def h2d(i):
        stage_k.copy_(hk[i % nh], non_blocking=True)

    layers = 36
    reps = max(1, args.steps // 4)
    for fn in (restore, cow, h2d):
        for i in range(nh):
            fn(i)
    r_us = c.per_call_ms(restore, layers * reps) * 1e3
    c_us = c.per_call_ms(cow, layers * reps) * 1e3
    h_us = c.per_call_ms(h2d, layers * reps) * 1e3
    moved = 2 * n * blk
    del kc, vc, hk, hv, stage_k
    return {"workload": "restore of a 16384-token Qwen3-4B prefix from pinned host memory: "
                        "1024 blocks x 36 layers, 64 MiB per layer, into scattered pool blocks "
                        "(pa_copy_blocks)",
            "ms_per_prefix": round(r_us * layers / 1e3, 3),
            "host_link_GBps": round(moved / r_us / 1e3, 1),
            "h2d_dma_copy_GBps": round(blk * n / h_us / 1e3, 1),
            "in_pool_copy": {"us_per_layer": round(c_us, 2),
                             "roofline": roofline_hbm(2 * moved, c_us, "copy_blocks_kernel",
                                                      "kv_restore", ["copy.hip"])}}


def prefix_match_leg():
    """Host-side prefix-block matching on the warm prefix-cache sweep's prompt
    lengths ("Qwen3-4B / 8B / 32B", section Warm Prefix-Cache TTFT: 256 ..
    16384 tokens): one prompt of each length is registered (2032 blocks in
    all), then the longest is looked up again (a full warm hit).  Reports
    the library's time per lookup of the 16384-token prompt (1024 blocks)
    and the oracle's for the same lookup."""
    import torch
    import paged_kv_gqa_write_amd as pa
    import oracle
    g = torch.Generator().manual_seed(42)
    lengths = [256 << i for i in range(7)]
    prompts = [torch.randint(0, 151_000, (n,), generator=g, dtype=torch.int32).numpy()
               for n in lengths]
    idx, ref = pa.PrefixIndex(1 << 16), oracle.PrefixCache(1 << 16)
    nid = 0
    for pr in prompts:
        ids = list(range(nid, nid + len(pr) // 16))
        nid += len(ids)
        idx.insert(pr, ids)
        ref.insert(pr.tolist(), ids)
    big, big_list = prompts[-1], prompts[-1].tolist()
    assert idx.match(big) == ref.match(big_list)
    reps = 2000
    t0 = time.perf_counter()
    for _ in range(reps):
        idx.match(big)
    lib_us = (time.perf_counter() - t0) / reps * 1e6
    t0 = time.perf_counter()
    oreps = 0
    while time.perf_counter() - t0 < 1.0:
        ref.match(big_list)
        oreps += 1
    ora_us = (time.perf_counter() - t0) / oreps * 1e6
    idx.close()
    return {"workload": "prompts of 256..16384 tokens registered (2032 sealed blocks), then the "
                        "16384-token prompt looked up again: a 1024-block warm hit",
            "us_per_lookup": round(lib_us, 2), "blocks_per_s": round(1024 / lib_us * 1e6),
            "oracle_us_per_lookup": round(ora_us, 1),
            "note": "host CPU, one thread, including the Python binding's marshalling"}


def copy_calibration(c):
    """A plain 512 MiB device-to-device copy: this device's copy bandwidth
    for reference, and the known-size dispatch the HBM traffic counters are
    scaled by."""
    torch = c.torch
    src = torch.empty(512 * 2 ** 20, dtype=torch.uint8, device=c.dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    ms = c.per_call_ms(lambda i: dst.copy_(src), 10)
    del src, dst
    return round(2 * 512 * 2 ** 20 / (ms * 1e-3) / 1e9, 1)


def cpu_baseline(case, seconds):
    """The fp64 oracle (as it stands) decoding the headline workload's layer
    repeatedly for about `seconds`; KV GB/s on the same algorithmic bytes."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    as_bits = lambda t: t.contiguous().view(__import__("torch").int16).numpy().view(np.uint16)  # noqa
    kc, vc, q = as_bits(case.k_cache), as_bits(case.v_cache), as_bits(case.q)
    bt, ctx = case.block_tables.numpy(), case.context_lens.numpy()
    runs, t0 = 0, time.perf_counter()
    while True:
        oracle.decode(q, kc, vc, bt, ctx, case.scale, case.num_q_heads, case.num_kv_heads)
        runs += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    per = el / runs
    return {"value": round(case.kv_bytes() / per / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{runs} oracle decode(s) of one {case.name} layer ({case.kv_bytes()} KV "
                      f"bytes each: batch {case.batch}, {case.num_q_heads}/{case.num_kv_heads} "
                      f"heads, head_dim {case.head_dim}), {el:.1f} s total, {per:.3f} s per "
                      f"layer; numpy BLAS threads {threads} (the block gather is "
                      f"single-threaded); host CPUs {os.cpu_count()}"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(every workload here is one GPU's share; nothing in the path spans GPUs)",
              file=sys.stderr)
        sys.exit(2)
    import workloads
    c = Ctx(args)
    legs = {}
    headline_case = None

    def run(name, fn):
        if name in args.legs:
            print(f"[bench] {name}", file=sys.stderr, flush=True)
            legs[name] = fn()

    if HEADLINE in args.legs or not args.no_cpu_baseline:
        headline_case = workloads.qwen3_32b_decode(poison=False)
    run(HEADLINE, lambda: decode_leg(c, HEADLINE, headline_case, 64, True))
    run("qwen3_32b_decode_b4_8192",
        lambda: decode_leg(c, "qwen3_32b_decode_b4_8192",
                           workloads.qwen3_32b_decode_long(poison=False), 64, True))
    run("qwen3_32b_decode_mixed_b8",
        lambda: decode_leg(c, "qwen3_32b_decode_mixed_b8",
                           workloads.qwen3_32b_decode_mixed(poison=False), 64, True,
                           compare_max_plan=True))
    run("hybrid_decode_b8",
        lambda: decode_leg(c, "hybrid_decode_b8", workloads.hybrid_decode(poison=False), 16,
                           True))
    run("hybrid_prefill_4097",
        lambda: prefill_leg(c, "hybrid_prefill_4097", workloads.hybrid_prefill(poison=False),
                            16)[0])
    run("qwen3_4b_decode_b8",
        lambda: decode_leg(c, "qwen3_4b_decode_b8", workloads.qwen3_4b_decode(poison=False), 36,
                           True, detail=True))
    if "qwen3_4b_prefill_4x1024" in args.legs or "write_kv" in args.legs:
        print("[bench] qwen3_4b_prefill_4x1024 / write_kv", file=sys.stderr, flush=True)
        pres, wk = prefill_leg(c, "qwen3_4b_prefill_4x1024",
                               workloads.qwen3_4b_prefill(poison=False), 36, write_kv_leg=True)
        if "qwen3_4b_prefill_4x1024" in args.legs:
            legs["qwen3_4b_prefill_4x1024"] = pres
        if "write_kv" in args.legs:
            legs["write_kv"] = wk
    run("verify", lambda: verify_leg(c))
    run("kv_restore", lambda: restore_leg(c))
    run("prefix_match", prefix_match_leg)
    copy_gbps = copy_calibration(c)

    head = legs.get(HEADLINE)
    result = {
        "metric": METRIC,
        "value": head["value"] if head else None, "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"] if head else None,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 tensors shaped like the pages' workloads)",
        "config": {"workload": "qwen3_32b_decode_b64: one decode step of a 64-layer Qwen3-32B "
                               "attention stack, 64 sequences in flight (KV append + decode in "
                               "one kernel per layer)",
                   **({k: v for k, v in head.items()
                       if k in ("layers", "batch", "num_q_heads", "num_kv_heads", "head_dim",
                                "context_len_range", "num_blocks_per_layer", "partition_size",
                                "num_partitions", "kv_bytes_per_layer")} if head else {})},
        "roofline": ({**head["roofline"], "copy_GBps_measured": copy_gbps} if head else None),
        "legs": {k: v for k, v in legs.items() if k != HEADLINE},
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu_baseline", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(headline_case, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
