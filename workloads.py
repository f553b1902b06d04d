"""Seeded synthetic inputs for the prefix-scan primitives.

This module only draws random numbers and fills arrays; it holds none of the
arithmetic of the method, so both sides of a parity check (the HIP library
and the CPU oracle) can take their inputs from it without sharing any code of
the computation.  Every generator is a ``numpy.random.Generator`` over
``PCG64(seed)``, so the same seed gives the same array on every machine.

The workloads (sizes, value ranges, seeds):

  scan_small      n = 2^16 uniform u32 (seed 101), checked at fork depths 0..8
  scan_mid        n = 2^24 uniform u32 (seed 201), plus all-ones / all-0xFFFFFFFF
  scan_large      n = 2^28 uniform u32 (seed 202), plus all-ones / all-0xFFFFFFFF
  compact_p*      n = 2^26 int32 0/1 flags, Bernoulli keep probability
                  p = 0.5 / 0.01 / 0.99 (seeds 301 / 302 / 303)
  segscan         n = 2^26 u32 uniform over [0, 2^16) (seed 401), regular
                  segments of length 16 and 2^20
  radix_uniform   n = 2^25 uniform u32 keys (seed 501)
  radix_distinct  n = 2^25 keys drawn from 256 distinct uniform u32 values
                  (seed 502)
  scan_u64        n = 2^27 uniform u64 (seed 601): the byte size of scan_large
  runs_uniform    n = 2^24 owners, entry counts uniform over [0, 8) (seed 701):
                  about 5.9e7 entries, one owner in eight empty
  runs_sparse     n = 2^24 owners, nine in ten empty, the rest uniform over
                  [1, 64) (seed 702): long stretches of empty runs
  segflags        n = 2^26 u32 values uniform over [0, 2^16) (seed 401, as
                  segscan) with head flags: segment lengths geometric with
                  mean 16 (seed 801), and geometric with mean 2^20 (seed 802)
"""
import numpy as np

U32_MAX = 0xFFFFFFFF

SEED_SCAN_SMALL = 101
SEED_SCAN_MID = 201
SEED_SCAN_LARGE = 202
SEED_COMPACT = {0.5: 301, 0.01: 302, 0.99: 303}
SEED_SEGSCAN = 401
SEED_RADIX_UNIFORM = 501
SEED_RADIX_DISTINCT = 502
SEED_SCAN_U64 = 601
SEED_RUNS_UNIFORM = 701
SEED_RUNS_SPARSE = 702
SEED_SEGFLAGS = {16: 801, 1 << 20: 802}

N_SCAN_SMALL = 1 << 16
N_SCAN_MID = 1 << 24
N_SCAN_LARGE = 1 << 28
N_COMPACT = 1 << 26
N_SEGSCAN = 1 << 26
SEG_LENS = (16, 1 << 20)
N_RADIX = 1 << 25
N_SCAN_U64 = 1 << 27
N_RUNS = 1 << 24


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def uniform_u32(n: int, seed: int) -> np.ndarray:
    """n values uniform over [0, 2^32)."""
    return rng(seed).integers(0, 1 << 32, size=n, dtype=np.uint32)


def uniform_u64(n: int, seed: int) -> np.ndarray:
    """n values uniform over [0, 2^64)."""
    return rng(seed).integers(0, 1 << 64, size=n, dtype=np.uint64)


def ones_u32(n: int) -> np.ndarray:
    return np.ones(n, dtype=np.uint32)


def all_ff_u32(n: int) -> np.ndarray:
    """Every entry 0xFFFFFFFF: the sums wrap at every step."""
    return np.full(n, U32_MAX, dtype=np.uint32)


def iota_u32(n: int) -> np.ndarray:
    return np.arange(n, dtype=np.uint32)


def bernoulli_flags(n: int, p: float, seed: int) -> np.ndarray:
    """int32 flags, 1 with probability p, else 0."""
    return (rng(seed).random(n) < p).astype(np.int32)


def compact_flags(p: float, n: int = N_COMPACT) -> np.ndarray:
    return bernoulli_flags(n, p, SEED_COMPACT[p])


def seg_values(n: int = N_SEGSCAN, seed: int = SEED_SEGSCAN) -> np.ndarray:
    """u32 values uniform over [0, 2^16)."""
    return rng(seed).integers(0, 1 << 16, size=n, dtype=np.uint32)


def radix_keys_uniform(n: int = N_RADIX, seed: int = SEED_RADIX_UNIFORM) -> np.ndarray:
    return uniform_u32(n, seed)


def radix_keys_distinct(n: int = N_RADIX, distinct: int = 256,
                        seed: int = SEED_RADIX_DISTINCT) -> np.ndarray:
    """Keys drawn uniformly from `distinct` distinct uniform u32 values."""
    g = rng(seed)
    while True:
        vals = g.integers(0, 1 << 32, size=distinct, dtype=np.uint32)
        if np.unique(vals).size == distinct:
            break
    return vals[g.integers(0, distinct, size=n)]


def small_random_u32(n: int, seed: int, high: int = 1 << 32) -> np.ndarray:
    """Generic seeded u32 array for the small parity cases."""
    return rng(seed).integers(0, high, size=n, dtype=np.uint32)


def runs_counts_uniform(n: int = N_RUNS, seed: int = SEED_RUNS_UNIFORM) -> np.ndarray:
    """Per-owner entry counts, uniform over [0, 8)."""
    return rng(seed).integers(0, 8, size=n, dtype=np.uint32)


def runs_counts_sparse(n: int = N_RUNS, seed: int = SEED_RUNS_SPARSE) -> np.ndarray:
    """Per-owner entry counts: 0 with probability 0.9, else uniform over [1, 64)."""
    g = rng(seed)
    c = g.integers(1, 64, size=n, dtype=np.uint32)
    c[g.random(n) < 0.9] = 0
    return c


def segment_heads(n: int, mean_len: int, seed: int = None) -> np.ndarray:
    """int32 head flags for irregular segments: each element starts a new
    segment with probability 1 / mean_len (geometric lengths), and element 0
    always does."""
    if seed is None:
        seed = SEED_SEGFLAGS[mean_len]
    f = (rng(seed).random(n) < 1.0 / mean_len).astype(np.int32)
    if n:
        f[0] = 1
    return f
