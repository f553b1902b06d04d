"""Brute-force definitions in pure Python big integers, for tiny inputs.

These are the plain definitions of each result, independent of the C oracle,
used to pin the oracle on small cases.  Every sum is taken exactly and reduced
mod 2^32 only at the end.
"""
M = 1 << 32


def exclusive(a):
    return [sum(a[:j]) % M for j in range(len(a))]


def inclusive(a):
    return [sum(a[:j + 1]) % M for j in range(len(a))]


def total(a):
    return sum(a) % M


def segscan(a, L):
    out = []
    for j in range(len(a)):
        h = (j // L) * L
        out.append(sum(a[h:j + 1]) % M)
    sums = [sum(a[s:s + L]) % M for s in range(0, len(a), L)]
    return out, sums


def compact(flags):
    kept = [i for i, f in enumerate(flags) if f != 0]
    return kept + [-1] * (len(flags) - len(kept)), len(kept)


def stable_perm(keys):
    return sorted(range(len(keys)), key=lambda i: (keys[i], i))
