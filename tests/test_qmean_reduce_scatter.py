"""The Q-mean reduce-scatter of the attention kernel, emulated on the host.

Where the attention kernel sums the region's Q means itself, lane li of a
row of 16 lanes holds its own sums of 8 dims (one query each).  Four DPP
steps then reduce-scatter those sums over the row: partners 15 - li
(row_mirror), 7 - li within each half (row_half_mirror), li ^ 2 and li ^ 1
(quad permutations); at each of the first three a lane keeps half of the
dims it still holds and adds the partner's copy of them, and the last adds
the partner's whole value.  Lane li ends with dim 4 [li >= 8] + 2 [li & 4] +
[li & 2], written by the even lanes.

This test replays the lane exchanges (the same keep/send choices and DPP
partner maps) in Python and checks that every dim's written value is the sum
over all 16 lanes -- exactly, with integer data -- and that each dim is
written once.  A wrong partner map, keep/send choice or output index would
fail it; the GPU parity tests check the same path end to end.
"""
import numpy as np


def row_mirror(i):          # DPP row_mirror: lane 15 - i of the row
    return 15 - i


def row_half_mirror(i):     # DPP row_half_mirror: lane 7 - i within each half
    return (i & 8) | (7 - (i & 7))


def quad_xor2(i):           # quad_perm [2, 3, 0, 1]
    return i ^ 2


def quad_xor1(i):           # quad_perm [1, 0, 3, 2]
    return i ^ 1


def reduce_scatter(sd):
    """sd[li][e]: lane li's sums of dims e = 0..7.  Returns {dim: value}
    as the even lanes write them."""
    ha = [li >= 8 for li in range(16)]
    hb = [(li & 4) != 0 for li in range(16)]
    hc = [(li & 2) != 0 for li in range(16)]
    # step A: keep dims 0..3 (li < 8) or 4..7, add the mirror lane's copy
    send = [[sd[li][j] if ha[li] else sd[li][4 + j] for j in range(4)] for li in range(16)]
    a = [[(sd[li][4 + j] if ha[li] else sd[li][j]) + send[row_mirror(li)][j]
          for j in range(4)] for li in range(16)]
    # step B: keep two of those four
    send = [[a[li][j] if hb[li] else a[li][2 + j] for j in range(2)] for li in range(16)]
    b = [[(a[li][2 + j] if hb[li] else a[li][j]) + send[row_half_mirror(li)][j]
          for j in range(2)] for li in range(16)]
    # step C: keep one
    send = [b[li][0] if hc[li] else b[li][1] for li in range(16)]
    c = [(b[li][1] if hc[li] else b[li][0]) + send[quad_xor2(li)] for li in range(16)]
    # step D: the pair's total
    c = [c[li] + c[quad_xor1(li)] for li in range(16)]
    out = {}
    for li in range(16):
        if li % 2 == 0:
            d = 4 * ha[li] + 2 * hb[li] + hc[li]
            assert d not in out, f"dim {d} written twice"
            out[d] = c[li]
    return out


def test_partner_maps_are_involutions():
    for f in (row_mirror, row_half_mirror, quad_xor2, quad_xor1):
        assert all(f(f(i)) == i and f(i) != i and 0 <= f(i) < 16 for i in range(16))


def test_every_dim_is_the_sum_over_the_row():
    rng = np.random.default_rng(7)
    for _ in range(50):
        sd = rng.integers(-2**40, 2**40, size=(16, 8)).tolist()
        out = reduce_scatter(sd)
        assert sorted(out) == list(range(8))
        for d in range(8):
            assert out[d] == sum(sd[li][d] for li in range(16))


def test_single_lane_contributions_reach_their_dim():
    # one nonzero entry at a time: it must appear in its own dim only
    for li in range(16):
        for e in range(8):
            sd = [[0] * 8 for _ in range(16)]
            sd[li][e] = 1
            out = reduce_scatter(sd)
            assert out == {d: int(d == e) for d in range(8)}
