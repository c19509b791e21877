"""Host-side model of the bf16 scatter's launch grid (k_scatter / scatter()
in combine_ep_dispatch_amd/csrc/move.hip): the index arithmetic of the
kernel and its launcher, written out in Python.

Checked: the reciprocal multiplies, in 64-bit arithmetic as the kernel
does them, equal integer division for every numerator tried below 2^31
(the kernel's numerators stay below 2^26); every (token, piece,
slot) of a batch is taken by exactly one wave; the K' waves of a (token,
piece) run on one XCD (workgroup index mod 8); launches stay within 2^32 - 1
work-items.  The GPU parity tests run the kernel itself on the same shapes
and more.
"""

import itertools

import pytest

WAVES = 8                      # EPX_SCATTER_WAVES
MAX_BLOCKS = 0xFFFFFFFF // (WAVES * 64)


def reciprocal(d):
    l = 0
    while (1 << l) < d:
        l += 1
    return ((1 << (32 + l)) // d) + 1, 32 + l


def launches(T, pieces, Kp):
    chunk = ((MAX_BLOCKS - 8) // Kp * WAVES - 8) // pieces
    assert chunk >= 1
    out, t0 = [], 0
    while t0 < T:
        tokens = min(chunk, T - t0)
        pairs_per_xcd = ((tokens * pieces + 7) & ~7) >> 3
        n = (pairs_per_xcd * Kp + WAVES - 1) // WAVES * 8
        out.append((t0, t0 + tokens, n))
        t0 += tokens
    return out


U64 = 2 ** 64 - 1


def div64(q, m, s):
    """(uint64)q * m >> s, as the kernel computes it."""
    return ((q * m) & U64) >> s


def waves(T, pieces, Kp):
    dm, ds = reciprocal(pieces)
    km, ks = reciprocal(Kp)
    for t0, t1, n in launches(T, pieces, Kp):
        for b in range(n):
            for w in range(WAVES):
                j = (b >> 3) * WAVES + w
                assert j < 2 ** 26
                pair = div64(j, km, ks)
                k = j - pair * Kp
                rest = (pair << 3) | (b & 7)
                assert rest < 2 ** 26
                tr = div64(rest, dm, ds)
                p = rest - tr * pieces
                t = t0 + tr
                if t < t1:
                    yield b, w, t, p, k


@pytest.mark.parametrize("T,pieces,Kp", list(itertools.product([1, 7, 13, 129], [1, 3, 7], [1, 2, 6, 8, 9, 16, 64])))
def test_every_triple_once_and_slots_share_an_xcd(T, pieces, Kp):
    seen = {}
    for b, _, t, p, k in waves(T, pieces, Kp):
        assert 0 <= k < Kp and 0 <= p < pieces
        assert (t, p, k) not in seen
        seen[(t, p, k)] = b & 7
    assert len(seen) == T * pieces * Kp
    for (t, p, k), xcd in seen.items():
        assert seen[(t, p, 0)] == xcd


def test_k8_is_one_workgroup_per_pair():
    for b, w, t, p, k in waves(50, 7, 8):
        assert b == t * 7 + p and k == w  # workgroup b holds pair b, wave w its slot w


@pytest.mark.parametrize("d", list(range(1, 70)) + [127, 128, 1000, 2 ** 20 + 3])
def test_reciprocal_division_is_exact(d):
    m, s = reciprocal(d)
    assert m < 2 ** 33  # so q * m < 2^64 for q < 2^31
    qs = [0, 1, d - 1, d, d + 1, 2 ** 26, 2 ** 31 - 1]
    qs += [d * i - 1 for i in range(1, 50)] + [(2 ** 31 // d) * d + r for r in range(-2, 2)]
    for q in qs:
        if 0 <= q < 2 ** 31:
            assert div64(q, m, s) == q // d


@pytest.mark.parametrize("T,pieces,Kp", [(2 ** 24, 7, 8), (2 ** 22, 56, 9), (2 ** 26, 1, 64)])
def test_launches_fit_the_grid_limit(T, pieces, Kp):
    L = launches(T, pieces, Kp)
    assert sum(t1 - t0 for t0, t1, _ in L) == T
    assert all(n <= MAX_BLOCKS for _, _, n in L)
