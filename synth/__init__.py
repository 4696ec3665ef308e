"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic (no normalisation, no rotation, no rounding rule of the
method).  Both sides read the exact arrays it returns.

Every tensor comes from its own PCG64 stream, keyed by (seed, *stream), so the
same (seed, stream) gives the same values on any machine and in any order of
calls.  Stream keys are small integer tuples: (workload id, layer, tensor id).

Recipe (shapes and distributions follow the workloads the Flint pages imply:
GQA with 32 query and 4 KV heads of dim 128, bf16 KV, learned sinks):
  * raw q, k, v            ~ N(0,1) fp32
  * sink logits            ~ N(0,1) fp32, one per query head
  * norm weights           1.0 (workloads) or ~ 1 + 0.1 N(0,1) (tests)
  * bf16 cache contents    N(0,1) fp32 draws truncated to their top 16 bits
                           (a way to draw bf16 values; not the method's rounding);
                           multi-GB caches use torch's generator on the GPU
                           (normal_bf16_bits_torch) instead of PCG64
  * fp8 cache contents     uniform random E4M3 codes: a random sign and a
                           magnitude code uniform in [0, max_code] (default
                           0x3F, |x| < 2), so no NaN code is ever drawn
  * MoE weights            N(0, 1/fan_in) bf16, drawn like the bf16 caches
                           (x ~ N(0,1), so router logits and FFN
                           activations are O(1))
  * page tables            a seeded permutation of the physical pages
  * ragged lengths         uniform integers in [lo, hi], inclusive
"""
from __future__ import annotations

import numpy as np

# tensor ids for stream keys
Q, K, V, SINK, QW, KW, PERM, LENS, KC, VC, POS = range(1, 12)


def rng(seed: int, *stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), *map(int, stream)])))


def normal(seed: int, stream: tuple, shape) -> np.ndarray:
    """N(0,1) fp32 array of `shape` from stream (seed, *stream)."""
    return rng(seed, *stream).standard_normal(size=shape, dtype=np.float32)


def normal_bf16_bits(seed: int, stream: tuple, shape) -> np.ndarray:
    """uint16 bf16 bit patterns: N(0,1) fp32 draws truncated to their top 16 bits."""
    x = normal(seed, stream, shape)
    return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def torch_seed(seed: int, stream: tuple) -> int:
    """63-bit seed for a torch.Generator, derived from (seed, *stream)."""
    st = np.random.SeedSequence([int(seed), *map(int, stream)]).generate_state(1, np.uint64)[0]
    return int(st) & ((1 << 63) - 1)


def normal_bf16_bits_torch(seed: int, stream: tuple, shape, device="cpu", std: float = 1.0):
    """Like normal_bf16_bits but drawn by torch's generator on `device` (for
    multi-GB caches and weights: fast on the GPU).  Returns an int16 tensor of
    bf16 bit patterns: N(0, std^2) fp32 draws truncated to their top 16 bits."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(torch_seed(seed, stream))
    x = torch.randn(tuple(shape), generator=g, dtype=torch.float32, device=device)
    if std != 1.0:
        x *= std
    return (x.view(torch.int32) >> 16).to(torch.int16)


def fp8_codes(seed: int, stream: tuple, shape, max_code: int = 0x3F) -> np.ndarray:
    """uint8 fp8 E4M3 codes: a random sign bit over a magnitude code uniform in
    [0, max_code]; max_code < 0x7F keeps the NaN codes out."""
    r = rng(seed, *stream)
    mag = r.integers(0, max_code, size=shape, endpoint=True).astype(np.uint8)
    sign = (r.integers(0, 1, size=shape, endpoint=True).astype(np.uint8) << np.uint8(7))
    return mag | sign


def fp8_codes_torch(seed: int, stream: tuple, shape, device="cpu", max_code: int = 0x3F):
    """Like fp8_codes, drawn by torch's generator on `device`; uint8 tensor."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(torch_seed(seed, stream))
    mag = torch.randint(0, max_code + 1, tuple(shape), generator=g, dtype=torch.uint8, device=device)
    sign = torch.randint(0, 2, tuple(shape), generator=g, dtype=torch.uint8, device=device)
    return mag | (sign << 7)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact: bf16 is the top half of fp32)."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def permutation(seed: int, stream: tuple, n: int) -> np.ndarray:
    return rng(seed, *stream).permutation(n).astype(np.int32)


def uniform_ints(seed: int, stream: tuple, n: int, lo: int, hi: int) -> np.ndarray:
    """n integers uniform in [lo, hi] (both ends included)."""
    return rng(seed, *stream).integers(lo, hi, size=n, endpoint=True).astype(np.int32)


def norm_weight(seed: int, stream: tuple, d: int, ones: bool) -> np.ndarray:
    if ones:
        return np.ones(d, dtype=np.float32)
    return (1.0 + 0.1 * rng(seed, *stream).standard_normal(d)).astype(np.float32)


# ---------------------------------------------------------------------------
# page tables
# ---------------------------------------------------------------------------

def shuffled_block_table(seed: int, stream: tuple, num_seqs: int, pages_per_seq,
                         bt_stride: int):
    """Give request b pages_per_seq[b] distinct physical pages, all requests drawn
    from one seeded permutation of sum(pages_per_seq) pages.

    Returns (block_tables [num_seqs, bt_stride] int32 with unused entries -1,
    num_blocks)."""
    pages = np.asarray(pages_per_seq, dtype=np.int64)
    total = int(pages.sum())
    perm = permutation(seed, stream, total)
    bt = np.full((num_seqs, bt_stride), -1, dtype=np.int32)
    off = 0
    for b in range(num_seqs):
        n = int(pages[b])
        bt[b, :n] = perm[off:off + n]
        off += n
    return bt, total


def ring_block_table(seed: int, stream: tuple, num_seqs: int, logical_pages: int,
                     ring_pages: int, bt_stride: int):
    """Sliding-window tables: logical page p of request b maps to physical page
    ring_b[p mod ring_pages], with each request's ring a distinct seeded set of
    physical pages.  Entries beyond `logical_pages` are -1.

    Returns (block_tables, num_blocks = num_seqs * ring_pages)."""
    total = num_seqs * ring_pages
    perm = permutation(seed, stream, total)
    bt = np.full((num_seqs, bt_stride), -1, dtype=np.int32)
    p = np.arange(logical_pages)
    for b in range(num_seqs):
        ring = perm[b * ring_pages:(b + 1) * ring_pages]
        bt[b, :logical_pages] = ring[p % ring_pages]
    return bt, total
