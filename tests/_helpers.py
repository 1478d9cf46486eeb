"""Shared test-side helpers: tensor <-> numpy bit views and a test-side
builder that scatters logical per-sequence K/V into the pool layout.

The pool layout is the library contract: K [NB, Hkv, D/32, 16, 32] (element
d of the K row of in-block offset o at [b, g, d // 32, o, d % 32]) and
V [NB, Hkv, D, 16] (bf16), token p of a sequence at physical block
block_table[p // 16], offset p % 16.  Tiny oracle-only cases whose D is not a
multiple of 32 use one K slice of width D ([NB, Hkv, 1, 16, D]); the oracle
takes the slice width from the pool's last axis.
"""
import numpy as np
import torch

BLOCK = 16
NAN_BITS = np.uint16(0x7FC0)


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> uint16 numpy bit patterns (CPU copy)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16).copy()


def from_bits(a: np.ndarray) -> torch.Tensor:
    """uint16 numpy bit patterns -> bf16 CPU tensor."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)


def exact_bf16_bits(values) -> np.ndarray:
    """Bit patterns of values that must be exactly representable in bf16."""
    f = np.asarray(values, dtype=np.float32)
    b = f.view(np.uint32)
    if np.any(b & np.uint32(0xFFFF)):
        raise ValueError("value not exactly representable in bf16")
    return (b >> np.uint32(16)).astype(np.uint16)


def random_bf16_bits(gen: torch.Generator, shape, sigma=1.0) -> np.ndarray:
    x = torch.randn(*shape, generator=gen) * sigma
    return bits(x.to(torch.bfloat16))


def k_slice_width(d: int) -> int:
    """Width of a K pool slice: 32 (the library's) or, for D not a multiple
    of 32, D itself."""
    return 32 if d % 32 == 0 else d


def k_pool_from_rows(rows: np.ndarray) -> np.ndarray:
    """Token rows [..., 16, D] -> K pool layout [..., D/W, 16, W]."""
    *lead, bs, d = rows.shape
    w = k_slice_width(d)
    return np.ascontiguousarray(np.moveaxis(rows.reshape(*lead, bs, d // w, w), -2, -3))


def scatter_to_pool(keys_bits, values_bits, block_table, num_blocks, fill=NAN_BITS):
    """Build K/V pools from logical per-sequence K/V.

    keys_bits[s] is [L_s, Hkv, D] uint16 (bf16 bits) in logical order; the
    token at position p goes to block block_table[s][p // 16], offset p % 16.
    Every other slot holds `fill` (NaN by default).
    """
    hkv, d = keys_bits[0].shape[1], keys_bits[0].shape[2]
    w = k_slice_width(d)
    kc = np.full((num_blocks, hkv, d // w, BLOCK, w), fill, dtype=np.uint16)
    vc = np.full((num_blocks, hkv, d, BLOCK), fill, dtype=np.uint16)
    for s, (ks, vs) in enumerate(zip(keys_bits, values_bits)):
        for p in range(ks.shape[0]):
            b = int(block_table[s][p // BLOCK])
            o = p % BLOCK
            for g in range(hkv):
                for j in range(d // w):
                    kc[b, g, j, o, :] = ks[p, g, j * w:(j + 1) * w]
                vc[b, g, :, o] = vs[p, g]
    return kc, vc


def padded_table(rows, width=None):
    width = width or max(len(r) for r in rows)
    bt = np.full((len(rows), width), -1, dtype=np.int32)
    for i, r in enumerate(rows):
        bt[i, :len(r)] = r
    return bt


def bf16_tolerance_report(gpu_f64: np.ndarray, ref_f64: np.ndarray, atol=4e-3):
    """Per-element check: |gpu - ref| <= atol, or gpu is one of the two bf16
    neighbours of the exact value (|gpu - ref| < ulp_bf16(ref)).  Returns a
    dict with the literal max / mean abs error, the error of the exact value
    rounded to bf16 (the floor no bf16 output can beat), and the counts."""
    import oracle
    err = np.abs(gpu_f64 - ref_f64)
    ulp = oracle.bf16_ulp(ref_f64)
    ok_abs = err <= atol
    ok_ulp = err < ulp
    floor = np.abs(oracle.f64_to_bf16_f64(ref_f64) - ref_f64)
    return {
        "max_abs": float(err.max()) if err.size else 0.0,
        "mean_abs": float(err.mean()) if err.size else 0.0,
        "floor_max_abs": float(floor.max()) if floor.size else 0.0,
        "floor_mean_abs": float(floor.mean()) if floor.size else 0.0,
        "n_fail": int(np.count_nonzero(~(ok_abs | ok_ulp))),
        "n_ulp_only": int(np.count_nonzero(ok_ulp & ~ok_abs)),
        "n_nonfinite": int(np.count_nonzero(~np.isfinite(gpu_f64))),
        "n": int(err.size),
    }


def relayout(case, mapping, num_blocks=None):
    """The same case with its pool blocks moved: physical block `old` becomes
    `mapping[old]` for every block the table references (a dict old -> new;
    a full permutation moves every block).  Pools, block table and slot
    mapping are rewritten to match; blocks no one maps to hold bf16 NaN.
    Works for decode, multi-token and prefill cases (any dataclass with
    k_cache, v_cache, block_tables and slot_mapping)."""
    import dataclasses
    nb = num_blocks or case.k_cache.shape[0]
    olds = torch.tensor(sorted(mapping), dtype=torch.long)
    news = torch.tensor([mapping[int(o)] for o in olds], dtype=torch.long)
    nan = torch.tensor(int(NAN_BITS), dtype=torch.int32).to(torch.int16)
    k2 = torch.empty((nb,) + tuple(case.k_cache.shape[1:]), dtype=torch.int16).fill_(nan)
    v2 = torch.empty((nb,) + tuple(case.v_cache.shape[1:]), dtype=torch.int16).fill_(nan)
    k2[news] = case.k_cache.view(torch.int16)[olds]
    v2[news] = case.v_cache.view(torch.int16)[olds]
    lut = torch.full((case.k_cache.shape[0],), -1, dtype=torch.long)
    lut[olds] = news
    bt = case.block_tables.long()
    bt2 = torch.where(bt >= 0, lut[bt.clamp(min=0)], bt).to(torch.int32)
    sl = case.slot_mapping
    sl2 = torch.where(sl >= 0, lut[(sl // BLOCK).clamp(min=0)] * BLOCK + sl % BLOCK, sl)
    kw = dict(k_cache=k2.view(torch.bfloat16), v_cache=v2.view(torch.bfloat16),
              block_tables=bt2, slot_mapping=sl2)
    if hasattr(case, "num_blocks"):
        kw["num_blocks"] = nb
    return dataclasses.replace(case, **kw)


def permuted_case(case, seed=1):
    """Every physical block moved by a seeded random permutation of the pool."""
    nb = case.k_cache.shape[0]
    perm = torch.randperm(nb, generator=torch.Generator().manual_seed(seed))
    return relayout(case, {b: int(perm[b]) for b in range(nb)})


def contiguous_twin(case):
    """The case with each sequence's blocks laid out one after another from
    block 0, in logical order (identity-like table), other blocks NaN."""
    mapping, nxt = {}, 0
    for row in case.block_tables.tolist():
        for b in row:
            if b >= 0 and b not in mapping:
                mapping[b] = nxt
                nxt += 1
    return relayout(case, mapping)
