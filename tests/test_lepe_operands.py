"""The MFMA LePE's operand construction, emulated on the host.

The pool kernel writes each channel's 25 weights as one 64-byte row of bf16
(taps in order 5i + j, then 7 zeros).  In the attention kernel the four
lanes n = 0..3 of a channel load words 4n .. 4n + 3 of that row, share them
by DPP quad broadcasts, and each lane builds, for tap row i, the 8 bf16
[0]*n, w[i][0..4], 0, .. by 16-bit funnel shifts: its B operands for column
steps ks = 0 and 1.  This test replays those word operations (the same
shifts, masks and selects, in Python integers) and checks every lane's ten
operands against the banded Toeplitz definition B[kk][n] = w[i][4 ks + kk - n]
(zero outside 0..4).  A wrong shift direction, word index or mask would fail
it; the GPU parity tests check the same path end to end.
"""
import numpy as np

M32 = 0xFFFFFFFF


def bf16_bits(x):
    """Round-to-nearest-even fp32 -> bf16 bits (finite values)."""
    u = np.float32(x).view(np.uint32).item()
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) & 0xFFFF


def table_row(w25):
    """The 16 words of one channel's row: taps 2m, 2m + 1 in word m."""
    h = [bf16_bits(v) for v in w25] + [0] * 7
    return [h[2 * m] | (h[2 * m + 1] << 16) for m in range(16)]


def alignbit(hi, lo, sh):
    """v_alignbit_b32: the low 32 bits of (hi:lo) >> sh."""
    return (((hi << 32) | lo) >> sh) & M32


def lane_operands(row, n):
    """Lane n's ten operands (row i, ks) as 4-element bf16 lists, built the way
    the kernel builds them: each lane holds words 4n .. 4n + 3, and word m of
    the row comes from lane m // 4 of the quad."""
    held = [row[4 * q:4 * q + 4] for q in range(4)]  # what each quad lane loaded

    def row_word(m):
        return held[m >> 2][m & 3]

    half, word = (n & 1) != 0, n >= 2
    out = {}
    for i in range(5):
        if (5 * i) % 2 == 0:
            m = 5 * i // 2
            z = [row_word(m), row_word(m + 1), row_word(m + 2) & 0xFFFF, 0]
        else:
            m = (5 * i - 1) // 2
            a, b, c = row_word(m), row_word(m + 1), row_word(m + 2)
            z = [alignbit(b, a, 16), alignbit(c, b, 16), c >> 16, 0]
        e = [((z[0] << 16) & M32) if half else z[0]]
        for k in range(1, 4):
            e.append(alignbit(z[k], z[k - 1], 16) if half else z[k])
        o = [0 if word else e[0], e[0] if word else e[1], e[1] if word else e[2],
             e[2] if word else e[3]]
        for ks in range(2):
            w0, w1 = o[2 * ks], o[2 * ks + 1]
            out[(i, ks)] = [w0 & 0xFFFF, w0 >> 16, w1 & 0xFFFF, w1 >> 16]
    return out


def test_operands_match_the_toeplitz_definition():
    rng = np.random.default_rng(2024)
    for _ in range(50):
        w = rng.standard_normal((5, 5)).astype(np.float32)
        row = table_row(w.reshape(-1))
        for n in range(4):
            ops = lane_operands(row, n)
            for i in range(5):
                for ks in range(2):
                    expect = []
                    for kk in range(4):
                        j = 4 * ks + kk - n
                        expect.append(bf16_bits(w[i, j]) if 0 <= j <= 4 else 0)
                    assert ops[(i, ks)] == expect, (n, i, ks, ops[(i, ks)], expect)


def test_row_padding_is_zero_and_taps_in_order():
    w = np.arange(1, 26, dtype=np.float32)
    row = table_row(w)
    halves = [(row[m] >> (16 * s)) & 0xFFFF for m in range(16) for s in range(2)]
    assert halves[:25] == [bf16_bits(v) for v in w]
    assert halves[25:] == [0] * 7
