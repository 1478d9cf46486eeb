"""Benchmark: paged GQA decode KV GB/s (and prefill TFLOP/s) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--layers 36]

One step is one decode step of a Qwen3-4B-shaped attention stack (32 query
heads, 8 KV heads, head_dim 128, 36 layers; "Qwen3-4B / 8B / 32B", section
Architecture Notes): for every layer, the 8 new tokens' K/V are appended and
split-K decode runs over contexts of 1024-1152 tokens scattered over a
4096-block pool (pa_decode_append: both in one kernel), then its
log-sum-exp reduce (pa_decode_reduce).  The same step with the append as
its own kernel (pa_write_kv + pa_decode + reduce) is reported beside it.  Every layer has its own pools, so a step streams
36 x ~35.7 MB of KV -- far more than the 256 MB Infinity Cache -- straight
from HBM, as a real decode step does.  The prefill section times the
prefill path (pa_write_kv of 4 x 1024 new tokens + pa_prefill, two of the
sequences after 512 cached tokens) over the same 36-layer stack, and the
verify section the pass that checks drafted blocks (4 sequences x 8 query
tokens: pa_write_kv + pa_decode_multi + pa_decode_multi_reduce per layer).

Prints ONE JSON line.  `value` = whole-step KV bytes / step time.  The
roofline object covers the decode kernel: algorithmic KV bytes per launch /
its average launch duration (the step's decode launches re-issued back to
back between HIP events on the launch stream).
cpu_baseline = the CPU fp64 oracle timed on a bounded sample of the same
workload.
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


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", type=int, default=36)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-verify", action="store_true")
    ap.add_argument("--no-restore", action="store_true")
    ap.add_argument("--no-prefix-match", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    return ap.parse_args()


def source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "paged_kv_gqa_write_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel_file, sources):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", kernel_file)
    if not os.path.exists(p):
        return None
    with open(p) as f:
        rec = json.load(f)
    if rec.get("source_hash") != source_hash(*sources):
        return None
    return rec.get("hbm_bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path has no multi-GPU component)", file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_kv_gqa_write_amd as pa
    import workloads

    pa.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    L = args.layers

    # ---------------- decode: Qwen3-4B shape, batch 8 ------------------------
    case = workloads.qwen3_4b_decode(poison=False)
    B, hq, hkv, d = case.batch, case.num_q_heads, case.num_kv_heads, case.head_dim
    nb = case.num_blocks
    gen = torch.Generator(device=dev)
    gen.manual_seed(42)
    kc = [case.k_cache.to(dev)]
    vc = [case.v_cache.to(dev)]
    for _ in range(1, L):
        kc.append(torch.randn(kc[0].shape, generator=gen, device=dev).to(torch.bfloat16))
        vc.append(torch.randn(vc[0].shape, generator=gen, device=dev).to(torch.bfloat16))
    q = case.q.to(dev)
    k_new, v_new = case.k_new.to(dev), case.v_new.to(dev)
    slots = case.slot_mapping.to(dev)
    bt = case.block_tables.to(dev)
    ctx = case.context_lens.to(dev)
    max_ctx = int(case.context_lens.max())
    ps, npart = pa.decode_split_plan(B, hkv, max_ctx)
    out = torch.empty(B, hq, d, dtype=torch.bfloat16, device=dev)
    part_out = torch.empty(B, hq, npart, d, dtype=torch.float32, device=dev)
    part_lse = torch.empty(B, hq, npart, dtype=torch.float32, device=dev)
    lib = pa.load_library()
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream

    def append_decode(i, sptr=sptr):
        return lib.pa_decode_append(out.data_ptr(), part_out.data_ptr(), part_lse.data_ptr(),
                                    q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(),
                                    kc[i].data_ptr(), vc[i].data_ptr(), bt.data_ptr(),
                                    ctx.data_ptr(), B, hq, hkv, d, 16, nb, bt.shape[1], ps,
                                    npart, case.scale, sptr)

    def decode_layer(i, sptr=sptr):
        # append the 8 new tokens' K/V and decode (one kernel), then the reduce
        st = append_decode(i, sptr)
        if npart > 1:
            st |= lib.pa_decode_reduce(out.data_ptr(), part_out.data_ptr(), part_lse.data_ptr(),
                                       ctx.data_ptr(), B, hq, d, ps, npart, sptr)
        return st

    def decode_step(sptr=sptr):
        for i in range(L):
            if decode_layer(i, sptr) != 0:
                raise RuntimeError("decode step launch failed")

    for _ in range(args.warmup):
        decode_step()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.steps):
        decode_step()
    t1.record(stream)
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps
    kv_bytes_layer = case.kv_bytes()
    value = kv_bytes_layer * L / (ms_step * 1e-3) / 1e9

    # The same step captured once as a HIP graph and replayed (the pages' decode
    # runs as graph replay): launch overhead leaves the host, the GPU work is
    # identical.  Reported beside the eager figure.
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        decode_step(side.cuda_stream)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        decode_step(torch.cuda.current_stream(dev).cuda_stream)
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(args.steps):
        graph.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    graph_ms_step = t0.elapsed_time(t1) / args.steps
    del graph

    # The same step with the append as its own kernel (pa_write_kv, then
    # pa_decode and the reduce), for reference.
    def split_layer(i):
        st = lib.pa_write_kv(k_new.data_ptr(), v_new.data_ptr(), slots.data_ptr(),
                             kc[i].data_ptr(), vc[i].data_ptr(), B, hkv, d, 16, nb, sptr)
        st |= lib.pa_decode(out.data_ptr(), part_out.data_ptr(), part_lse.data_ptr(),
                            q.data_ptr(), kc[i].data_ptr(), vc[i].data_ptr(), bt.data_ptr(),
                            ctx.data_ptr(), B, hq, hkv, d, 16, nb, bt.shape[1], ps, npart,
                            case.scale, sptr)
        if npart > 1:
            st |= lib.pa_decode_reduce(out.data_ptr(), part_out.data_ptr(), part_lse.data_ptr(),
                                       ctx.data_ptr(), B, hq, d, ps, npart, sptr)
        if st != 0:
            raise RuntimeError("decode step launch failed")

    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(args.steps):
        for i in range(L):
            split_layer(i)
    t1.record(stream)
    torch.cuda.synchronize()
    split_ms_step = t0.elapsed_time(t1) / args.steps

    # The step's decode kernel alone (the appending form): the same K steps'
    # launches issued back to back on the launch stream between one pair of
    # HIP events (the reduce is left out), so the average is the kernel's own
    # duration plus the hardware's inter-dispatch gap -- what rocprofv3's
    # kernel trace reports for it, without per-launch event overhead.
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(args.steps):
        for i in range(L):
            append_decode(i)
    b.record(stream)
    torch.cuda.synchronize()
    dec_us = a.elapsed_time(b) / (args.steps * L) * 1e3
    dec_gbps = kv_bytes_layer / (dec_us * 1e-6) / 1e9
    traffic = measured_traffic("decode_kernel_traffic.json", ["decode.hip", "pa_device.h"])
    roofline = {"bound": "hbm", "achieved": round(dec_gbps, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(dec_gbps / HBM_PEAK_GBPS, 4),
                "traffic": traffic, "kernel": "decode_kernel<128> (appending form)",
                "algorithmic_bytes_per_launch": kv_bytes_layer,
                "avg_launch_us": round(dec_us, 3)}

    # plain copy bandwidth of this device, for reference
    src = torch.empty(512 * 2 ** 20, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    c0 = torch.cuda.Event(enable_timing=True)
    c1 = torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(10):
        dst.copy_(src)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbps = 2 * src.numel() * 10 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    roofline["copy_GBps_measured"] = round(copy_gbps, 1)
    del src, dst

    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 tensors shaped like the pages' workloads)",
        "config": {"workload": "qwen3_4b_decode_b8: one decode step of a 36-layer Qwen3-4B "
                               "attention stack (KV append + split-K decode in one kernel, then "
                               "the reduce, per layer)",
                   "layers": L, "batch": B, "num_q_heads": hq, "num_kv_heads": hkv,
                   "head_dim": d, "block_size": 16, "context_lens": case.context_lens.tolist(),
                   "num_blocks_per_layer": nb, "partition_size": ps, "num_partitions": npart},
        "roofline": roofline,
        "decode_step_separate_append": {
            "ms_per_step": round(split_ms_step, 4),
            "value": round(kv_bytes_layer * L / (split_ms_step * 1e-3) / 1e9, 1), "unit": "GB/s",
            "note": "same step with pa_write_kv as its own kernel before pa_decode"},
        "decode_step_graph": {"ms_per_step": round(graph_ms_step, 4),
                              "value": round(kv_bytes_layer * L / (graph_ms_step * 1e-3) / 1e9, 1),
                              "unit": "GB/s",
                              "note": "same step captured once as a HIP graph and replayed"},
    }

    del kc, vc
    torch.cuda.empty_cache()

    # ---------------- prefill: Qwen3-4B shape, 4 x 1024 ----------------------
    if not args.no_prefill:
        pc = workloads.qwen3_4b_prefill(poison=False)
        pkc = [pc.k_cache.to(dev)]
        pvc = [pc.v_cache.to(dev)]
        for _ in range(1, L):
            pkc.append(torch.randn(pkc[0].shape, generator=gen, device=dev).to(torch.bfloat16))
            pvc.append(torch.randn(pvc[0].shape, generator=gen, device=dev).to(torch.bfloat16))
        pq = pc.q.to(dev)
        pkn, pvn = pc.k_new.to(dev), pc.v_new.to(dev)
        pslots = pc.slot_mapping.to(dev)
        pbt = pc.block_tables.to(dev)
        pcu = pc.cu_seqlens.to(dev)
        ppre = pc.prefix_lens.to(dev)
        pout = torch.empty_like(pq)
        T, phq, phkv, pd = pc.total_q, pc.num_q_heads, pc.num_kv_heads, pc.head_dim
        maxq = max(pc.q_lens)

        def prefill_layer(i):
            st = lib.pa_write_kv(pkn.data_ptr(), pvn.data_ptr(), pslots.data_ptr(),
                                 pkc[i].data_ptr(), pvc[i].data_ptr(), T, phkv, pd, 16,
                                 pc.num_blocks, sptr)
            st |= lib.pa_prefill(pout.data_ptr(), pq.data_ptr(), pkc[i].data_ptr(),
                                 pvc[i].data_ptr(), pbt.data_ptr(), pcu.data_ptr(),
                                 ppre.data_ptr(), pc.num_seqs, T, maxq, phq, phkv, pd, 16,
                                 pc.num_blocks, pbt.shape[1], pc.scale, sptr)
            if st != 0:
                raise RuntimeError("prefill launch failed")

        for _ in range(args.warmup):
            for i in range(L):
                prefill_layer(i)
        torch.cuda.synchronize()
        t0.record(stream)
        for _ in range(args.steps):
            for i in range(L):
                prefill_layer(i)
        t1.record(stream)
        torch.cuda.synchronize()
        pms = t0.elapsed_time(t1) / args.steps
        flops = pc.flops()
        # prefill kernel alone, back to back over the layers (see decode above)
        torch.cuda.synchronize()
        t0.record(stream)
        for _ in range(args.steps):
            for i in range(L):
                st = lib.pa_prefill(pout.data_ptr(), pq.data_ptr(), pkc[i].data_ptr(),
                                    pvc[i].data_ptr(), pbt.data_ptr(), pcu.data_ptr(),
                                    ppre.data_ptr(), pc.num_seqs, T, maxq, phq, phkv, pd, 16,
                                    pc.num_blocks, pbt.shape[1], pc.scale, sptr)
        t1.record(stream)
        torch.cuda.synchronize()
        pf_us = t0.elapsed_time(t1) / (args.steps * L) * 1e3
        pf_tflops = flops / (pf_us * 1e-6) / 1e12
        # pa_write_kv of the 4096 new tokens alone, back to back over the layers
        torch.cuda.synchronize()
        t0.record(stream)
        for _ in range(args.steps):
            for i in range(L):
                lib.pa_write_kv(pkn.data_ptr(), pvn.data_ptr(), pslots.data_ptr(),
                                pkc[i].data_ptr(), pvc[i].data_ptr(), T, phkv, pd, 16,
                                pc.num_blocks, sptr)
        t1.record(stream)
        torch.cuda.synchronize()
        wkv_us = t0.elapsed_time(t1) / (args.steps * L) * 1e3
        wkv_bytes = 2 * 2 * T * phkv * pd * 2     # K and V, read and written
        result["prefill"] = {
            "workload": "qwen3_4b_prefill_4x1024: 4 x 1024 new tokens, sequences 1 and 3 after "
                        "512 cached tokens, 32/8 heads, head_dim 128, 36 layers "
                        "(write_kv + prefill per layer)",
            "value": round(flops * L / (pms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
            "ms_per_step": round(pms, 4), "algorithmic_flops_per_layer": flops,
            "roofline": {"bound": "mfma", "achieved": round(pf_tflops, 2),
                         "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(pf_tflops / BF16_PEAK_TFLOPS, 4),
                         "traffic": measured_traffic("prefill_kernel_traffic.json",
                                                     ["prefill.hip", "pa_device.h"]),
                         "kernel": "prefill_kernel<128>", "avg_launch_us": round(pf_us, 3)},
        }
        result["write_kv"] = {
            "workload": "pa_write_kv of the 4096 new tokens of qwen3_4b_prefill_4x1024 (8 KV heads, "
                        "head_dim 128), back to back over 36 layers' pools",
            "avg_launch_us": round(wkv_us, 3), "bytes_per_launch": wkv_bytes,
            "roofline": {"bound": "hbm", "achieved": round(wkv_bytes / (wkv_us * 1e-6) / 1e9, 1),
                         "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": round(wkv_bytes / (wkv_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)},
            "decode_append_note": "the decode step appends its 8 tokens inside pa_decode_append"}
        del pkc, pvc
        torch.cuda.empty_cache()

    # ---------------- verify: Qwen3-4B shape, batch 4, T = 8 -----------------
    if not args.no_verify:
        result["verify"] = verify_leg(args, lib, dev, gen, stream, L)

    # ---------------- block copy: host-tier restore of a 16k-token prefix ----
    if not args.no_restore:
        result["kv_restore"] = restore_leg(args, lib, dev, stream)

    # ---------------- prefix-block matching (host) ---------------------------
    if not args.no_prefix_match:
        result["prefix_match"] = prefix_match_leg()

    # ---------------- CPU baseline: the oracle on a bounded sample -----------
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args.cpu_seconds)

    print(json.dumps(result), flush=True)


def verify_leg(args, lib, dev, gen, stream, L):
    """The pass that checks a drafted block ("Qwen3-4B / 8B / 32B", section
    DSpark Speculative Decoding): per layer the T = 8 query tokens' K/V are
    appended (pa_write_kv, 32 tokens), then pa_decode_multi and
    pa_decode_multi_reduce run over contexts of 1024-1152 tokens.  Reported
    as KV GB/s like the decode step."""
    import torch
    import paged_kv_gqa_write_amd as pa
    import workloads
    case = workloads.qwen3_4b_verify(batch=4, poison=False)
    B, T, hq, hkv, d = case.batch, case.query_len, case.num_q_heads, case.num_kv_heads, case.head_dim
    nb = case.num_blocks
    kc = [case.k_cache.to(dev)]
    vc = [case.v_cache.to(dev)]
    for _ in range(1, L):
        kc.append(torch.randn(kc[0].shape, generator=gen, device=dev).to(torch.bfloat16))
        vc.append(torch.randn(vc[0].shape, generator=gen, device=dev).to(torch.bfloat16))
    q = case.q.to(dev)
    k_new, v_new, slots = case.k_new.to(dev), case.v_new.to(dev), case.slot_mapping.to(dev)
    bt, ctx = case.block_tables.to(dev), case.context_lens.to(dev)
    ps, npart = pa.decode_multi_split_plan(B, T, hq, hkv, int(case.context_lens.max()))
    out = torch.empty(B, T, hq, d, dtype=torch.bfloat16, device=dev)
    part_out = torch.empty(B, T, hq, npart, d, dtype=torch.float32, device=dev)
    part_lse = torch.empty(B, T, hq, npart, dtype=torch.float32, device=dev)
    sptr = stream.cuda_stream

    def multi(i):
        return lib.pa_decode_multi(out.data_ptr(), part_out.data_ptr(), part_lse.data_ptr(),
                                   q.data_ptr(), kc[i].data_ptr(), vc[i].data_ptr(),
                                   bt.data_ptr(), ctx.data_ptr(), B, T, hq, hkv, d, 16, nb,
                                   bt.shape[1], ps, npart, case.scale, sptr)

    def layer(i):
        st = lib.pa_write_kv(k_new.data_ptr(), v_new.data_ptr(), slots.data_ptr(),
                             kc[i].data_ptr(), vc[i].data_ptr(), B * T, hkv, d, 16, nb, sptr)
        st |= multi(i)
        if npart > 1:
            st |= lib.pa_decode_multi_reduce(out.data_ptr(), part_out.data_ptr(),
                                             part_lse.data_ptr(), ctx.data_ptr(), B, T, hq, d,
                                             ps, npart, sptr)
        if st != 0:
            raise RuntimeError("verify launch failed")

    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    for _ in range(args.warmup):
        for i in range(L):
            layer(i)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(args.steps):
        for i in range(L):
            layer(i)
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    t0.record(stream)
    for _ in range(args.steps):
        for i in range(L):
            multi(i)
    t1.record(stream)
    torch.cuda.synchronize()
    k_us = t0.elapsed_time(t1) / (args.steps * L) * 1e3
    kvb = case.kv_bytes()
    del kc, vc
    torch.cuda.empty_cache()
    return {"workload": f"{case.name}: 4 sequences x 8 query tokens (last accepted + 7 drafted), "
                        "context 1024-1152, 32/8 heads, head_dim 128, 36 layers "
                        "(write_kv + decode_multi + reduce per layer)",
            "value": round(kvb * L / (ms * 1e-3) / 1e9, 1), "unit": "GB/s",
            "ms_per_step": round(ms, 4), "partition_size": ps, "num_partitions": npart,
            "kernel_avg_launch_us": round(k_us, 3),
            "kernel_GBps": round(kvb / (k_us * 1e-6) / 1e9, 1),
            "kernel_frac_of_hbm_peak": round(kvb / (k_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}


def restore_leg(args, lib, dev, stream):
    """Host-tier restore ("Qwen3-4B / 8B / 32B", section KV Offload): the
    1024 sealed blocks of a 16384-token Qwen3-4B prefix, per layer, copied by
    pa_copy_blocks from packed pinned host buffers into scattered pool blocks
    (the kernel reads host memory directly).  8 host buffers (64 MiB each)
    rotate over the layers.  Also: the same 1024 blocks duplicated inside
    the device pool (HBM read + write), and a plain 64 MiB host-to-device
    DMA copy of one buffer for the host link's reference rate."""
    import torch
    hkv, d, n, nb, nh = 8, 128, 1024, 4096, 8
    blk = hkv * 16 * d * 2
    kc = torch.empty((nb, hkv, 16, d), dtype=torch.bfloat16, device=dev)
    vc = torch.empty((nb, hkv, d, 16), dtype=torch.bfloat16, device=dev)
    hk = [torch.zeros((n, hkv, 16, d), dtype=torch.bfloat16, pin_memory=True) for _ in range(nh)]
    hv = [torch.zeros((n, hkv, d, 16), dtype=torch.bfloat16, pin_memory=True) for _ in range(nh)]
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    perm = torch.randperm(nb, generator=g, device=dev).to(torch.int32)
    dst, cow_src, cow_dst = perm[:n].contiguous(), perm[n:2 * n].contiguous(), perm[2 * n:3 * n].contiguous()
    stage_k = torch.empty_like(kc[:n])
    sptr = stream.cuda_stream

    def restore(i):
        if lib.pa_copy_blocks(kc.data_ptr(), vc.data_ptr(), nb, dst.data_ptr(), hk[i % nh].data_ptr(),
                              hv[i % nh].data_ptr(), n, None, n, hkv, d, 16, sptr) != 0:
            raise RuntimeError("restore launch failed")

    def cow(i):
        if lib.pa_copy_blocks(kc.data_ptr(), vc.data_ptr(), nb, cow_dst.data_ptr(), kc.data_ptr(),
                              vc.data_ptr(), nb, cow_src.data_ptr(), n, hkv, d, 16, sptr) != 0:
            raise RuntimeError("copy launch failed")

    def h2d(i):
        stage_k.copy_(hk[i % nh], non_blocking=True)

    def timed(fn, count):
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        for i in range(nh):
            fn(i)
        torch.cuda.synchronize()
        t0.record(stream)
        for i in range(count):
            fn(i)
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / count * 1e3

    layers = 36
    reps = max(1, args.steps // 4)
    r_us = timed(restore, layers * reps)
    c_us = timed(cow, layers * reps)
    h_us = timed(h2d, layers * reps)
    moved = 2 * n * blk
    del kc, vc, hk, hv, stage_k
    torch.cuda.empty_cache()
    return {"workload": "restore of a 16384-token Qwen3-4B prefix from pinned host memory: 1024 blocks "
                        "x 36 layers, 64 MiB per layer, into scattered pool blocks (pa_copy_blocks)",
            "ms_per_prefix": round(r_us * layers / 1e3, 3),
            "host_link_GBps": round(moved / r_us / 1e3, 1),
            "h2d_dma_copy_GBps": round(blk * n / h_us / 1e3, 1),
            "in_pool_copy": {"us_per_layer": round(c_us, 2),
                             "roofline": {"bound": "hbm", "achieved": round(2 * moved / c_us / 1e3, 1),
                                          "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                          "frac": round(2 * moved / c_us / 1e3 / HBM_PEAK_GBPS, 4)}}}


def prefix_match_leg():
    """Host-side prefix-block matching on the warm prefix-cache sweep's prompt
    lengths ("Qwen3-4B / 8B / 32B", section Warm Prefix-Cache TTFT: 256 ..
    16384 tokens): one prompt of each length is registered (2032 blocks in
    all), then each is looked up again (a full warm hit).  Reports the
    library's time per lookup of the 16384-token prompt (1024 blocks) and the
    oracle's for the same lookup."""
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


def cpu_baseline(seconds):
    """The fp64 oracle (as it stands) decoding the same Qwen3-4B batch-8 layer
    repeatedly for about `seconds`; KV GB/s on the same algorithmic bytes."""
    import numpy as np
    import oracle
    import workloads
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    case = workloads.qwen3_4b_decode(poison=False)
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
            "sample": f"{runs} oracle decode(s) of one qwen3_4b_decode_b8 layer "
                      f"({case.kv_bytes()} KV bytes each), {el:.1f} s total, "
                      f"{per:.3f} s per layer; BLAS threads {threads}, gather loop single-threaded"}


if __name__ == "__main__":
    main()
