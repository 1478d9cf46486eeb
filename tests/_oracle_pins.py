"""Pins for the CPU oracle: each function raises AssertionError if the oracle
disagrees with something fixed independently of it -- hand-derived golden
cases, 50-digit brute force on tiny inputs, closed forms, invariants, and
library routines for the bf16 conversions.

The functions take no arguments so that tests/test_oracle_mutations.py can
rerun the whole battery against deliberately broken copies of the oracle.
"""
import json
import math
import os

import mpmath
import numpy as np
import torch

import oracle
from _helpers import (bits, exact_bf16_bits, padded_table, random_bf16_bits,
                      scatter_to_pool, k_pool_from_rows)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "closed_form_cases.json")
mpmath.mp.dps = 50


# ---------------------------------------------------------------------------
# Golden, hand-derived cases
# ---------------------------------------------------------------------------

def _scalar(v):
    if isinstance(v, str):
        if v == "-inf":
            return -math.inf
        if v.startswith("ln"):
            return math.log(float(v[2:]))
    return float(v)


def _golden_inputs(case):
    hq, hkv, d = case["num_q_heads"], case["num_kv_heads"], case["head_dim"]
    if case["kind"] == "prefill":
        lens = [p + n for p, n in zip(case["prefix_lens"], case["q_lens"])]
    elif "context_lens" in case:
        lens = case["context_lens"]
    else:
        lens = [len(k) for k in case["keys"]]
    keys, values = [], []
    for s, L in enumerate(lens):
        if case["keys"] == "ones":
            k = np.ones((L, hkv, d))
        else:
            k = np.asarray(case["keys"][s], dtype=np.float64)
        if case["values"] == "position_pm":
            v = np.zeros((L, hkv, d))
            v[:, :, 0] = np.arange(L)[:, None]
            v[:, :, 1] = -np.arange(L)[:, None]
        else:
            v = np.asarray(case["values"][s], dtype=np.float64)
        keys.append(exact_bf16_bits(k))
        values.append(exact_bf16_bits(v))
    bt = padded_table(case["block_table"])
    kc, vc = scatter_to_pool(keys, values, bt, case["num_blocks"])
    return lens, bt, kc, vc


def pin_golden_cases():
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        lens, bt, kc, vc = _golden_inputs(case)
        hq, hkv = case["num_q_heads"], case["num_kv_heads"]
        scale = _scalar(case["scale"])
        exp = np.asarray(case["expected"], dtype=np.float64)
        if case["kind"] == "prefill":
            total = sum(case["q_lens"])
            q = exact_bf16_bits(np.ones((total, hq, case["head_dim"])))
            cu = np.concatenate([[0], np.cumsum(case["q_lens"])]).astype(np.int32)
            out = oracle.prefill(q, kc, vc, bt, cu, case["prefix_lens"], scale, hq, hkv)
        else:
            q = exact_bf16_bits(case["q"])
            out = oracle.decode(q, kc, vc, bt, lens, scale, hq, hkv)
        assert np.allclose(out, exp, rtol=0, atol=1e-12), (case["name"], out, exp)
        if case["kind"] == "partials":
            po, pl = oracle.decode_partials(q, kc, vc, bt, lens, scale, hq, hkv,
                                            case["partition_size"], case["num_partitions"])
            epo = np.asarray(case["expected_part_out"], dtype=np.float64)
            epl = np.vectorize(_scalar)(np.asarray(case["expected_part_lse"], dtype=object)).astype(np.float64)
            assert np.allclose(po, epo, rtol=0, atol=1e-12), (case["name"], po)
            fin = np.isfinite(epl)
            assert np.array_equal(np.isfinite(pl), fin), (case["name"], pl)
            assert np.allclose(pl[fin], epl[fin], rtol=0, atol=1e-12), (case["name"], pl)
            comb = oracle.combine_partials(po, pl)
            assert np.allclose(comb, exp, rtol=0, atol=1e-12), (case["name"], comb)


# ---------------------------------------------------------------------------
# bf16 conversions against known bit patterns and torch's own rounding
# ---------------------------------------------------------------------------

def pin_bf16_conversions():
    known = {0x3F80: 1.0, 0xC000: -2.0, 0x3F81: 1.0 + 2.0 ** -7, 0x0001: 2.0 ** -133,
             0x7F80: math.inf, 0x3E00: 0.125, 0x4049: 3.140625}
    got = oracle.bf16_bits_to_f64(np.array(list(known.keys()), dtype=np.uint16))
    assert np.array_equal(got, np.array(list(known.values()))), got
    # ties to even at 1: 1 + 2^-8 -> 1, 1 + 3*2^-8 -> 1 + 2^-6
    r = oracle.f64_to_bf16_f64([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 0.0])
    assert np.array_equal(r, [1.0, 1 + 2.0 ** -6, -1.0, 0.0]), r
    # agrees with torch's round-to-nearest-even fp32 -> bf16 on fp32 inputs
    g = torch.Generator().manual_seed(7)
    x = (torch.randn(20000, generator=g) * torch.exp(torch.randn(20000, generator=g) * 4))
    ref = x.to(torch.bfloat16).to(torch.float64).numpy()
    mine = oracle.f64_to_bf16_f64(x.to(torch.float64).numpy())
    assert np.array_equal(mine, ref)
    u = oracle.bf16_ulp(np.array([1.0, 1.5, 2.0, 3.9, 0.01]))
    assert np.array_equal(u, [2.0 ** -7, 2.0 ** -7, 2.0 ** -6, 2.0 ** -6, 2.0 ** -14]), u


# ---------------------------------------------------------------------------
# 50-digit brute force on tiny inputs
# ---------------------------------------------------------------------------

def _brute_attention(qv, ks, vs, scale):
    """Softmax attention straight from the definition, in 50-digit floats,
    without max subtraction: sum_j exp(z_j) v_j / sum_j exp(z_j)."""
    sc = mpmath.mpf(scale)
    ws = []
    for k in ks:
        z = sc * mpmath.fsum(mpmath.mpf(a) * mpmath.mpf(b) for a, b in zip(qv, k))
        ws.append(mpmath.exp(z))
    den = mpmath.fsum(ws)
    if not ws:
        return [0.0] * len(qv), -math.inf
    out = [float(mpmath.fsum(w * mpmath.mpf(v[i]) for w, v in zip(ws, vs)) / den) for i in range(len(qv))]
    return out, float(mpmath.log(den))


def _tiny_paged(gen, lens, hq, hkv, d, sigma=1.0, extra_blocks=3):
    """Logical per-sequence K/V, scattered into a pool through a random table."""
    nblk = [(L + 15) // 16 for L in lens]
    nb = sum(nblk) + extra_blocks
    perm = torch.randperm(nb, generator=gen).numpy()
    rows, off = [], 0
    for n in nblk:
        rows.append(list(perm[off:off + n]))
        off += n
    bt = padded_table(rows, max(nblk) + 1)
    keys = [random_bf16_bits(gen, (L, hkv, d), sigma) for L in lens]
    values = [random_bf16_bits(gen, (L, hkv, d), sigma) for L in lens]
    kc, vc = scatter_to_pool(keys, values, bt, nb)
    f = oracle.bf16_bits_to_f64
    return bt, kc, vc, [f(k) for k in keys], [f(v) for v in values]


SHAPES = [(1, 1, 3), (2, 1, 8), (4, 2, 5), (8, 2, 4), (4, 4, 1)]


def pin_brute_decode():
    gen = torch.Generator().manual_seed(1234)
    for hq, hkv, d in SHAPES:
        lens = [1, 16, 17, 40]
        bt, kc, vc, K, V = _tiny_paged(gen, lens, hq, hkv, d)
        q = random_bf16_bits(gen, (len(lens), hq, d))
        qf = oracle.bf16_bits_to_f64(q)
        scale = 1.0 / math.sqrt(d) * 1.7
        out = oracle.decode(q, kc, vc, bt, lens, scale, hq, hkv)
        G = hq // hkv
        for s, L in enumerate(lens):
            for h in range(hq):
                g = h // G
                want, _ = _brute_attention(qf[s, h], K[s][:, g], V[s][:, g], scale)
                assert np.allclose(out[s, h], want, rtol=1e-12, atol=1e-13), (hq, hkv, d, s, h)


def pin_brute_prefill():
    gen = torch.Generator().manual_seed(99)
    for hq, hkv, d in SHAPES[:4]:
        q_lens, prefix = [5, 1, 18], [0, 17, 3]
        lens = [n + p for n, p in zip(q_lens, prefix)]
        bt, kc, vc, K, V = _tiny_paged(gen, lens, hq, hkv, d)
        total = sum(q_lens)
        q = random_bf16_bits(gen, (total, hq, d))
        qf = oracle.bf16_bits_to_f64(q)
        cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
        scale = 0.9 / math.sqrt(d)
        out = oracle.prefill(q, kc, vc, bt, cu, prefix, scale, hq, hkv)
        G = hq // hkv
        for s in range(len(q_lens)):
            for i in range(q_lens[s]):
                row = cu[s] + i
                n_vis = prefix[s] + i + 1
                for h in range(hq):
                    g = h // G
                    want, _ = _brute_attention(qf[row, h], K[s][:n_vis, g], V[s][:n_vis, g], scale)
                    assert np.allclose(out[row, h], want, rtol=1e-12, atol=1e-13), (s, i, h)


def pin_brute_partials():
    gen = torch.Generator().manual_seed(5)
    hq, hkv, d = 4, 2, 3
    lens = [1, 33, 47, 0]
    bt, kc, vc, K, V = _tiny_paged(gen, [max(L, 1) for L in lens], hq, hkv, d)
    q = random_bf16_bits(gen, (len(lens), hq, d))
    qf = oracle.bf16_bits_to_f64(q)
    ps, P = 16, 4
    po, pl = oracle.decode_partials(q, kc, vc, bt, lens, 0.5, hq, hkv, ps, P)
    for s, L in enumerate(lens):
        for h in range(hq):
            g = h // (hq // hkv)
            for p in range(P):
                lo, hi = p * ps, min(L, (p + 1) * ps)
                want, lse = _brute_attention(qf[s, h], K[s][lo:hi, g] if hi > lo else [],
                                             V[s][lo:hi, g] if hi > lo else [], 0.5)
                assert np.allclose(po[s, h, p], want, rtol=1e-12, atol=1e-13), (s, h, p)
                if hi > lo:
                    assert abs(pl[s, h, p] - lse) < 1e-12, (s, h, p, pl[s, h, p], lse)
                else:
                    assert pl[s, h, p] == -math.inf
    out = oracle.decode(q, kc, vc, bt, lens, 0.5, hq, hkv)
    assert np.allclose(oracle.combine_partials(po, pl), out, rtol=1e-12, atol=1e-13)


def pin_write_kv_elementwise():
    """Element by element from the layout contract: K element i of the token
    in slot (b, o) lands at [b, g, i // W, o, i % W] (W = slice width: one
    slice for D = 5, two 32-wide slices for D = 64), V element i at
    [b, g, i, o]."""
    gen = torch.Generator().manual_seed(3)
    for d in (5, 64):
        nb, hkv, T = 6, 3, 9
        w = 32 if d == 64 else d
        kc = k_pool_from_rows(random_bf16_bits(gen, (nb, hkv, 16, d)))
        assert kc.shape == (nb, hkv, d // w, 16, w)
        vc = random_bf16_bits(gen, (nb, hkv, d, 16))
        kn = random_bf16_bits(gen, (T, hkv, d))
        vn = random_bf16_bits(gen, (T, hkv, d))
        slots = np.array([0, 17, 95, -1, 40, 16 * 5 + 15, 33, -7, 2], dtype=np.int64)
        k2, v2 = oracle.write_kv(kc, vc, kn, vn, slots)
        ek, ev = kc.copy(), vc.copy()
        for t in range(T):
            if slots[t] < 0:
                continue
            for g in range(hkv):
                for i in range(d):
                    ek[slots[t] // 16, g, i // w, slots[t] % 16, i % w] = kn[t, g, i]
                    ev[slots[t] // 16, g, i, slots[t] % 16] = vn[t, g, i]
        assert np.array_equal(k2, ek) and np.array_equal(v2, ev)
        assert k2.dtype == np.uint16 and v2.dtype == np.uint16


# ---------------------------------------------------------------------------
# Closed forms
# ---------------------------------------------------------------------------

def pin_closed_forms():
    """Single key, identical keys, zero query and two keys (sigmoid weights),
    at D = 8 (one K slice) and D = 64 (two 32-wide slices, so a slice read
    out of order changes the two-key scores)."""
    gen = torch.Generator().manual_seed(11)
    for d in (8, 64):
        _closed_forms_at(gen, d)


def _closed_forms_at(gen, d):
    hq, hkv = 4, 2
    # single token: output is V exactly
    bt, kc, vc, K, V = _tiny_paged(gen, [1, 1], hq, hkv, d)
    q = random_bf16_bits(gen, (2, hq, d))
    out = oracle.decode(q, kc, vc, bt, [1, 1], 0.3, hq, hkv)
    for s in range(2):
        for h in range(hq):
            assert np.array_equal(out[s, h], V[s][0, h // 2])
    # identical keys -> mean of V; q = 0 -> mean of V
    lens = [23]
    bt, kc, vc, K, V = _tiny_paged(gen, lens, hq, hkv, d)
    kc_same = kc.copy()
    row = kc[bt[0][0], :, :, 0, :].copy()
    for p in range(23):
        kc_same[bt[0][p // 16], :, :, p % 16, :] = row
    out = oracle.decode(q[:1], kc_same, vc, bt, lens, 0.7, hq, hkv)
    for h in range(hq):
        assert np.allclose(out[0, h], V[0][:, h // 2].mean(axis=0), rtol=1e-13, atol=1e-14)
    qz = np.zeros_like(q[:1])
    out = oracle.decode(qz, kc, vc, bt, lens, 0.7, hq, hkv)
    for h in range(hq):
        assert np.allclose(out[0, h], V[0][:, h // 2].mean(axis=0), rtol=1e-13, atol=1e-14)
    # two keys: sigmoid weights
    bt, kc, vc, K, V = _tiny_paged(gen, [2], hq, hkv, d)
    qf = oracle.bf16_bits_to_f64(q[:1])
    out = oracle.decode(q[:1], kc, vc, bt, [2], 0.25, hq, hkv)
    for h in range(hq):
        g = h // 2
        z0, z1 = 0.25 * K[0][0, g] @ qf[0, h], 0.25 * K[0][1, g] @ qf[0, h]
        s0 = 1.0 / (1.0 + math.exp(z1 - z0))
        s1 = 1.0 / (1.0 + math.exp(z0 - z1))
        assert np.allclose(out[0, h], s0 * V[0][0, g] + s1 * V[0][1, g], rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------------------------
# Invariants
# ---------------------------------------------------------------------------

def _case_bits(case):
    return (bits(case.q), bits(case.k_cache), bits(case.v_cache),
            case.block_tables.numpy(), case.context_lens.numpy())


def pin_block_permutation_and_contiguous_twin():
    from workloads import make_decode_case
    c = make_decode_case("inv", context_lens=[1, 15, 16, 17, 40], num_q_heads=8,
                         num_kv_heads=2, head_dim=16, num_blocks=24, seed=21, poison=False)
    q, kc, vc, bt, ctx = _case_bits(c)
    base = oracle.decode(q, kc, vc, bt, ctx, c.scale, 8, 2)
    gen = torch.Generator().manual_seed(8)
    perm = torch.randperm(24, generator=gen).numpy()
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    kc2[perm] = kc
    vc2[perm] = vc
    bt2 = np.where(bt >= 0, perm[np.maximum(bt, 0)], -1).astype(np.int32)
    assert np.array_equal(oracle.decode(q, kc2, vc2, bt2, ctx, c.scale, 8, 2), base)
    # contiguous twin: blocks laid out in logical order behind an identity-like table
    rows, nxt = [], 0
    kc3, vc3 = np.zeros_like(kc), np.zeros_like(vc)
    for s in range(len(ctx)):
        nb = (int(ctx[s]) + 15) // 16
        rows.append(list(range(nxt, nxt + nb)))
        for j in range(nb):
            kc3[nxt + j] = kc[bt[s, j]]
            vc3[nxt + j] = vc[bt[s, j]]
        nxt += nb
    bt3 = padded_table(rows, bt.shape[1])
    assert np.array_equal(oracle.decode(q, kc3, vc3, bt3, ctx, c.scale, 8, 2), base)


def pin_poison_ignored():
    from workloads import make_decode_case
    a = make_decode_case("p", context_lens=[3, 20, 33], num_q_heads=4, num_kv_heads=2,
                         head_dim=8, num_blocks=10, seed=4, poison=False)
    b = make_decode_case("p", context_lens=[3, 20, 33], num_q_heads=4, num_kv_heads=2,
                         head_dim=8, num_blocks=10, seed=4, poison=True)
    # make b's live slots identical to a's (poisoning covers the decoded
    # token's slot too; restore it)
    kb, vb = bits(b.k_cache), bits(b.v_cache)
    ka, va = bits(a.k_cache), bits(a.v_cache)
    kb, vb = oracle.write_kv(kb, vb, np.stack([ka[s // 16, :, :, s % 16, :].reshape(2, -1)
                                       for s in a.slot_mapping.numpy()]),
                             np.stack([va[s // 16, :, :, s % 16] for s in a.slot_mapping.numpy()]),
                             a.slot_mapping.numpy())
    assert np.isnan(oracle.bf16_bits_to_f64(kb)).any()
    q, ctx, bt = bits(a.q), a.context_lens.numpy(), a.block_tables.numpy()
    ra = oracle.decode(q, ka, va, bt, ctx, a.scale, 4, 2)
    rb = oracle.decode(q, kb, vb, bt, ctx, a.scale, 4, 2)
    assert np.isfinite(rb).all() and np.array_equal(ra, rb)


def pin_causal_perturbation_and_prefill_vs_decode():
    from workloads import make_prefill_case
    c = make_prefill_case("c", q_lens=[7, 20], prefix_lens=[0, 18], num_q_heads=4,
                          num_kv_heads=2, head_dim=8, num_blocks=12, seed=17, poison=False)
    kc, vc = oracle.write_kv(bits(c.k_cache), bits(c.v_cache), bits(c.k_new), bits(c.v_new),
                             c.slot_mapping.numpy())
    q, bt = bits(c.q), c.block_tables.numpy()
    cu, pl = c.cu_seqlens.numpy(), c.prefix_lens.numpy()
    base = oracle.prefill(q, kc, vc, bt, cu, pl, c.scale, 4, 2)
    # each row equals a decode of that token over context prefix+i+1
    for s in range(2):
        for i in range(c.q_lens[s]):
            row = cu[s] + i
            dec = oracle.decode(q[row:row + 1], kc, vc, bt[s:s + 1], [pl[s] + i + 1], c.scale, 4, 2)
            assert np.allclose(base[row], dec[0], rtol=1e-13, atol=1e-14), (s, i)
    # perturbing K/V of positions after prefix+i leaves rows <= i unchanged
    s, i = 1, 9
    kc2, vc2 = kc.copy(), vc.copy()
    for p in range(pl[s] + i + 1, pl[s] + c.q_lens[s]):
        b, o = bt[s, p // 16], p % 16
        kc2[b, :, :, o, :] ^= np.uint16(0x0040)
        vc2[b, :, :, o] ^= np.uint16(0x0040)
    pert = oracle.prefill(q, kc2, vc2, bt, cu, pl, c.scale, 4, 2)
    rows = slice(cu[s], cu[s] + i + 1)
    assert np.array_equal(pert[rows], base[rows])
    assert not np.allclose(pert[cu[s] + i + 1], base[cu[s] + i + 1])


def pin_gqa_equals_repeated_mha():
    from workloads import make_decode_case
    hq, hkv, d = 8, 2, 8
    c = make_decode_case("g", context_lens=[5, 31], num_q_heads=hq, num_kv_heads=hkv,
                         head_dim=d, num_blocks=6, seed=23, poison=False)
    q, kc, vc, bt, ctx = _case_bits(c)
    gqa = oracle.decode(q, kc, vc, bt, ctx, c.scale, hq, hkv)
    G = hq // hkv
    kc_m = np.repeat(kc, G, axis=1)     # KV head h' = h // G
    vc_m = np.repeat(vc, G, axis=1)
    mha = oracle.decode(q, kc_m, vc_m, bt, ctx, c.scale, hq, hq)
    assert np.array_equal(gqa, mha)


def pin_partials_combine_equals_unsplit():
    from workloads import make_decode_case
    c = make_decode_case("s", context_lens=[1, 64, 100, 257], num_q_heads=4, num_kv_heads=1,
                         head_dim=8, num_blocks=30, seed=31, poison=False)
    q, kc, vc, bt, ctx = _case_bits(c)
    full = oracle.decode(q, kc, vc, bt, ctx, c.scale, 4, 1)
    for ps, P in [(16, 17), (64, 5), (256, 2), (512, 1)]:
        po, pl = oracle.decode_partials(q, kc, vc, bt, ctx, c.scale, 4, 1, ps, P)
        assert np.allclose(oracle.combine_partials(po, pl), full, rtol=1e-12, atol=1e-14), ps


# ---------------------------------------------------------------------------
# Several query tokens per sequence (verifying a drafted block)
# ---------------------------------------------------------------------------

def pin_brute_decode_multi():
    """Token t of T at position ctx-T+t sees keys 0..ctx-T+t: 50-digit brute
    force per (sequence, token, head); ctx == 0 gives zeros, 0 < ctx < T NaN."""
    gen = torch.Generator().manual_seed(4321)
    for (hq, hkv, d), T in zip(SHAPES, [3, 8, 1, 2, 5]):
        lens = [T, 16, 17 + T, 40]
        bt, kc, vc, K, V = _tiny_paged(gen, lens, hq, hkv, d)
        q = random_bf16_bits(gen, (len(lens), T, hq, d))
        qf = oracle.bf16_bits_to_f64(q)
        scale = 1.3 / math.sqrt(d)
        out = oracle.decode_multi(q, kc, vc, bt, lens, scale, hq, hkv)
        assert out.shape == (len(lens), T, hq, d)
        G = hq // hkv
        for s, L in enumerate(lens):
            for t in range(T):
                n_vis = L - T + t + 1
                for h in range(hq):
                    g = h // G
                    want, _ = _brute_attention(qf[s, t, h], K[s][:n_vis, g], V[s][:n_vis, g], scale)
                    assert np.allclose(out[s, t, h], want, rtol=1e-12, atol=1e-13), (hq, s, t, h)
    bt, kc, vc, K, V = _tiny_paged(gen, [5, 5], 2, 1, 4)
    q = random_bf16_bits(gen, (2, 4, 2, 4))
    out = oracle.decode_multi(q, kc, vc, bt, [0, 3], 0.5, 2, 1)
    assert np.array_equal(out[0], np.zeros((4, 2, 4))), out[0]
    assert np.isnan(out[1]).all()


def pin_closed_forms_decode_multi():
    """Identical keys: token t's output is the mean of V over its window
    0..ctx-T+t exactly; one visible key gives that key's V."""
    gen = torch.Generator().manual_seed(77)
    hq, hkv, d, T = 4, 2, 8, 6
    lens = [6, 29]
    bt, kc, vc, K, V = _tiny_paged(gen, lens, hq, hkv, d)
    row = kc[bt[0][0], :, :, 0, :].copy()
    for s, L in enumerate(lens):
        for p in range(L):
            kc[bt[s][p // 16], :, :, p % 16, :] = row
    q = random_bf16_bits(gen, (2, T, hq, d))
    out = oracle.decode_multi(q, kc, vc, bt, lens, 0.8, hq, hkv)
    for s, L in enumerate(lens):
        for t in range(T):
            n_vis = L - T + t + 1
            for h in range(hq):
                want = V[s][:n_vis, h // 2].mean(axis=0)
                assert np.allclose(out[s, t, h], want, rtol=1e-13, atol=1e-14), (s, t, h)
    # ctx == T: token 0 sees only itself
    for h in range(hq):
        assert np.array_equal(out[0, 0, h], V[0][0, h // 2])


def pin_decode_multi_invariants():
    """T = 1 is decode; every T equals a prefill of the T tokens after a
    cached prefix of ctx - T; the split-K pieces combine to the unsplit result
    and match 50-digit brute force piece by piece."""
    from workloads import make_decode_case
    c = make_decode_case("m", context_lens=[9, 33, 70], num_q_heads=8, num_kv_heads=2,
                         head_dim=8, num_blocks=16, seed=13, poison=False)
    q1, kc, vc, bt, ctx = _case_bits(c)
    got = oracle.decode_multi(q1[:, None], kc, vc, bt, ctx, c.scale, 8, 2)[:, 0]
    assert np.array_equal(got, oracle.decode(q1, kc, vc, bt, ctx, c.scale, 8, 2))
    gen = torch.Generator().manual_seed(14)
    T = 7
    q = random_bf16_bits(gen, (3, T, 8, 8))
    multi = oracle.decode_multi(q, kc, vc, bt, ctx, c.scale, 8, 2)
    cu = np.arange(4, dtype=np.int32) * T
    pre = oracle.prefill(q.reshape(3 * T, 8, 8), kc, vc, bt, cu, ctx - T, c.scale, 8, 2)
    assert np.allclose(multi.reshape(3 * T, 8, 8), pre, rtol=1e-13, atol=1e-14)
    for ps, P in [(16, 5), (32, 3), (80, 1)]:
        po, pl = oracle.decode_multi_partials(q, kc, vc, bt, ctx, c.scale, 8, 2, ps, P)
        assert np.allclose(oracle.combine_partials(po, pl), multi, rtol=1e-12, atol=1e-14), ps
    po, pl = oracle.decode_multi_partials(q, kc, vc, bt, ctx, c.scale, 8, 2, 16, 5)
    qf = oracle.bf16_bits_to_f64(q)
    for s, L in enumerate(ctx):
        Ks, Vs = oracle.gather_sequence(kc, vc, bt[s], int(L))
        for t in (0, T - 1):
            for h in (0, 5):
                g = h // 4
                for p in range(5):
                    lo, hi = p * 16, min(int(L) - T + t + 1, (p + 1) * 16)
                    if hi <= lo:
                        assert pl[s, t, h, p] == -math.inf and not po[s, t, h, p].any()
                        continue
                    want, lse = _brute_attention(qf[s, t, h], Ks[lo:hi, g], Vs[lo:hi, g], c.scale)
                    assert np.allclose(po[s, t, h, p], want, rtol=1e-12, atol=1e-13)
                    assert abs(pl[s, t, h, p] - lse) < 1e-12


# ---------------------------------------------------------------------------
# Block-granular copy (host-tier restore / save, duplicating a shared block)
# ---------------------------------------------------------------------------

def pin_copy_blocks_elementwise():
    """Element by element: destination block d receives source block s for
    every (head, row, d) of K and (head, d, offset) of V; skipped and
    untouched blocks keep their bits; None ids mean blocks 0..n-1."""
    gen = torch.Generator().manual_seed(61)
    hkv, d = 3, 5
    sk = k_pool_from_rows(random_bf16_bits(gen, (7, hkv, 16, d)))
    sv = random_bf16_bits(gen, (7, hkv, d, 16))
    dk0 = k_pool_from_rows(random_bf16_bits(gen, (9, hkv, 16, d)))
    dv0 = random_bf16_bits(gen, (9, hkv, d, 16))
    src = np.array([6, 0, 3, 9, 2, -1], dtype=np.int32)
    dst = np.array([1, 8, 4, 2, 12, 5], dtype=np.int32)
    dk, dv = oracle.copy_blocks(dk0, dv0, dst, sk, sv, src, 6)
    ek, ev = dk0.copy(), dv0.copy()
    for i in range(6):
        if not (0 <= src[i] < 7 and 0 <= dst[i] < 9):
            continue
        for g in range(hkv):
            for r in range(16):
                for e in range(d):
                    ek[dst[i], g, 0, r, e] = sk[src[i], g, 0, r, e]
                    ev[dst[i], g, e, r] = sv[src[i], g, e, r]
    assert np.array_equal(dk, ek) and np.array_equal(dv, ev)
    assert np.array_equal(dk[[0, 2, 3, 5, 6, 7]], dk0[[0, 2, 3, 5, 6, 7]])
    pk, pv = oracle.copy_blocks(np.zeros((3, hkv, 1, 16, d), np.uint16),
                                np.zeros((3, hkv, d, 16), np.uint16), None, sk, sv,
                                np.array([5, 1, 4], dtype=np.int32), 3)
    assert np.array_equal(pk, sk[[5, 1, 4]]) and np.array_equal(pv, sv[[5, 1, 4]])
    rk, rv = oracle.copy_blocks(dk0, dv0, np.array([0, 7], dtype=np.int32), pk, pv, None, 2)
    assert np.array_equal(rk[0], sk[5]) and np.array_equal(rk[7], sk[1])
    assert np.array_equal(rv[0], sv[5]) and np.array_equal(rv[7], sv[1])


def pin_copy_blocks_save_restore_round_trip():
    """Saving a sequence's blocks to a packed buffer and restoring them into
    other blocks of a fresh pool gives the same attention through the new
    table, bit for bit (the host-tier restore replaces a prefill)."""
    from workloads import make_decode_case
    c = make_decode_case("rt", context_lens=[37, 50], num_q_heads=4, num_kv_heads=2,
                         head_dim=8, num_blocks=16, seed=19, poison=False)
    q, kc, vc, bt, ctx = _case_bits(c)
    base = oracle.decode(q, kc, vc, bt, ctx, c.scale, 4, 2)
    used = [int(b) for b in bt.reshape(-1) if b >= 0]
    n = len(used)
    hk, hv = oracle.copy_blocks(np.zeros((n,) + kc.shape[1:], np.uint16),
                                np.zeros((n,) + vc.shape[1:], np.uint16), None, kc, vc,
                                np.array(used, dtype=np.int32), n)
    gen = torch.Generator().manual_seed(20)
    fresh = torch.randperm(40, generator=gen).numpy()[:n].astype(np.int32)
    nk = random_bf16_bits(gen, (40,) + kc.shape[1:])
    nv = random_bf16_bits(gen, (40,) + vc.shape[1:])
    nk, nv = oracle.copy_blocks(nk, nv, fresh, hk, hv, None, n)
    remap = dict(zip(used, fresh))
    bt2 = np.where(bt >= 0, np.vectorize(lambda b: remap.get(int(b), -1))(bt), -1).astype(np.int32)
    assert np.array_equal(oracle.decode(q, nk, nv, bt2, ctx, c.scale, 4, 2), base)


# ---------------------------------------------------------------------------
# Prefix-block matching (host side of the prefix cache)
# ---------------------------------------------------------------------------

def _toks(*parts):
    out = []
    for p in parts:
        out += list(p)
    return out


def pin_prefix_cache_scenario():
    """A scripted sequence of registrations, lookups and removals whose
    results follow by hand from the definition (full blocks only, a block is
    identified by its whole prefix, first sealed copy kept, removal drops
    everything extending the block, reuse of a block id drops its old
    entry, invalid calls change nothing)."""
    a0, a1, a2 = list(range(100, 116)), list(range(200, 216)), list(range(300, 308))
    x0, y1, z2 = list(range(400, 416)), list(range(500, 516)), list(range(600, 616))
    A = _toks(a0, a1, a2)                 # 40 tokens: 2 full blocks + 8
    B = _toks(a0, a1, z2, [7, 7, 7, 7])   # 52 tokens: 3 full blocks
    C = _toks(x0, a1)                     # A's second block after another first block
    D = _toks(a0, y1)
    pc = oracle.PrefixCache(100)
    assert pc.match(A) == []
    assert pc.insert(A, [10, 11]) == 2
    assert pc.match(A) == [10, 11] and len(pc) == 2
    assert pc.match(A[:31]) == [10]       # the partial second block never matches
    assert pc.match(B) == [10, 11]
    assert pc.insert(B, [10, 11, 12]) == 1
    assert pc.match(B) == [10, 11, 12]
    assert pc.match(C) == []              # same block contents, different position in the prefix
    assert pc.match(D) == [10]
    assert pc.insert(B, [90, 91, 92]) == 0  # already cached: first copies kept
    assert pc.match(B) == [10, 11, 12]
    assert pc.remove(11) == 2             # A's block 1 and B's block 2, which extends it
    assert pc.match(B) == [10] and pc.match(A) == [10] and len(pc) == 1
    assert pc.insert(D, [99, 10]) is None  # 10 already holds D's own block 0
    assert pc.insert(D, [10, 13, 13]) is not None  # D has 2 full blocks: the third id is unused
    assert pc.match(D) == [10, 13]
    assert pc.insert(C, [13, 20]) == 2    # block 13 reused: D's entry for it goes first
    assert pc.match(D) == [10] and pc.match(C) == [13, 20] and len(pc) == 3
    assert pc.insert(A, [5, 6, 6]) is not None
    assert pc.match(A) == [10, 6]
    assert pc.insert(B, [1, 2, 2]) == 1   # blocks 0, 1 cached (10, 6): only id 2 for block 2
    assert pc.insert(_toks(x0, y1, z2), [30, 30, 31]) == 2     # block 0 cached: its id unused
    assert pc.insert(_toks(y1, x0, z2), [32, 32, 33]) is None  # duplicate ids to register
    assert pc.insert(_toks(z2, y1, x0), [40, -1, 41]) == 1     # a negative id stops there
    assert pc.match(_toks(z2, y1, x0)) == [40]
    small = oracle.PrefixCache(3)
    assert small.insert(A, [1, 2]) == 2
    assert small.insert(_toks(x0, y1, z2), [5, 6, 7]) == 1      # full after one more
    assert small.insert(_toks(x0, y1, z2), [5, 2, 7]) == 1      # reusing 2 frees A's entry
    assert small.match(_toks(x0, y1, z2)) == [5, 2] and small.match(A) == [1]


def pin_prefix_cache_invariants():
    """Random sequences: a registered sequence matches its own ids; changing
    one token at position p leaves exactly the p // 16 leading blocks
    matched; removing block j of a sequence leaves its j leading blocks."""
    gen = torch.Generator().manual_seed(55)
    pc = oracle.PrefixCache(10_000)
    next_id = 0
    for trial in range(40):
        n = int(torch.randint(0, 200, (1,), generator=gen))
        toks = torch.randint(0, 50, (n,), generator=gen).tolist()
        nb = n // 16
        ids = list(range(next_id, next_id + nb))
        next_id += nb
        got = pc.insert(toks, ids)
        m = pc.match(toks)
        assert len(m) == nb and got == sum(1 for b in m if b in ids)
        if nb:
            p = int(torch.randint(0, n, (1,), generator=gen))
            alt = list(toks)
            alt[p] += 1000
            assert pc.match(alt) == m[:p // 16]
            j = int(torch.randint(0, nb, (1,), generator=gen))
            pc.remove(m[j])
            assert pc.match(toks) == m[:j]


ALL_PINS = [
    pin_golden_cases,
    pin_bf16_conversions,
    pin_brute_decode,
    pin_brute_prefill,
    pin_brute_partials,
    pin_write_kv_elementwise,
    pin_closed_forms,
    pin_block_permutation_and_contiguous_twin,
    pin_poison_ignored,
    pin_causal_perturbation_and_prefill_vs_decode,
    pin_gqa_equals_repeated_mha,
    pin_partials_combine_equals_unsplit,
    pin_brute_decode_multi,
    pin_closed_forms_decode_multi,
    pin_decode_multi_invariants,
    pin_copy_blocks_elementwise,
    pin_copy_blocks_save_restore_round_trip,
    pin_prefix_cache_scenario,
    pin_prefix_cache_invariants,
]
