"""Brute-force reference for tiny inputs (pure Python, independent of the C oracle).

It computes the routing results from their plain meaning rather than from the running
counts the oracle uses:
  * the packed expand_x order is one global stable sort of every routed pick by
    (expert, source rank, token, pick), so a pick's row is its position in that list;
  * a pick's expand_idx is the number of earlier picks of the same source rank that chose
    the same expert;
  * the receive counts are plain counts over that list.
E4M3 and E5M2 rounding is a nearest-value search over the finite magnitudes of the format
(127 for E4M3, 124 for E5M2), built from the formats' field definitions.
"""
from fractions import Fraction


def routed_picks(W, E, BS, K, ids, mask=None, mask_kind=0):
    picks = []
    for s in range(W):
        for i in range(BS):
            for k in range(K):
                if mask_kind == 1 and not mask[s][i]:
                    continue
                if mask_kind == 2 and not mask[s][i][k]:
                    continue
                e = int(ids[s][i][k])
                if e < E:
                    picks.append((e, s, i, k))
    return picks


def route(W, E, BS, K, ids, mask=None, mask_kind=0):
    """Returns (rows, expand_idx, ep_recv_count, etn_counts, etn_cumsum, recv_offsets)."""
    L = E // W
    picks = sorted(routed_picks(W, E, BS, K, ids, mask, mask_kind))
    rows = {(s, i, k): pos for pos, (e, s, i, k) in enumerate(picks)}
    eidx = [[[-1] * K for _ in range(BS)] for _ in range(W)]
    for (e, s, i, k) in picks:
        eidx[s][i][k] = sum(1 for (e2, s2, i2, k2) in picks
                            if e2 == e and s2 == s and (i2, k2) < (i, k))
    erc = [[0] * (L * W) for _ in range(W)]
    etn_counts = [[0] * L for _ in range(W)]
    etn_cumsum = [[0] * L for _ in range(W)]
    for r in range(W):
        for j in range(L):
            for s in range(W):
                erc[r][j * W + s] = sum(1 for (e2, s2, _, _) in picks
                                        if r * L <= e2 and (e2, s2) <= (r * L + j, s))
            etn_counts[r][j] = sum(1 for p in picks if p[0] == r * L + j)
            etn_cumsum[r][j] = sum(1 for p in picks if r * L <= p[0] <= r * L + j)
    recv_offsets = [sum(1 for p in picks if p[0] < r * L) for r in range(W + 1)]
    return rows, eidx, erc, etn_counts, etn_cumsum, recv_offsets


def e4m3_values():
    """(code, exact value) for the 127 finite non-negative E4M3FN codes 0x00..0x7E."""
    out = []
    for code in range(0x7F):
        ex, m = code >> 3, code & 7
        v = Fraction(m, 8) * Fraction(2) ** -6 if ex == 0 else \
            (1 + Fraction(m, 8)) * Fraction(2) ** (ex - 7)
        out.append((code, v))
    return out


_E4M3 = e4m3_values()


def e4m3_nearest(v: Fraction) -> int:
    """Nearest finite E4M3FN code to the exact value v (ties to the even code), with
    magnitudes at or above 448 clamped to 448; the sign bit follows v's sign."""
    sign = 0x80 if v < 0 else 0
    a = abs(v)
    if a >= 448:
        return sign | 0x7E
    best = min(_E4M3, key=lambda cv: (abs(cv[1] - a), cv[0] & 1))
    return sign | best[0]


def e5m2_values():
    """(code, exact value) for the 124 finite non-negative E5M2 codes 0x00..0x7B."""
    out = []
    for code in range(0x7C):
        ex, m = code >> 2, code & 3
        v = Fraction(m, 4) * Fraction(2) ** -14 if ex == 0 else \
            (1 + Fraction(m, 4)) * Fraction(2) ** (ex - 15)
        out.append((code, v))
    return out


_E5M2 = e5m2_values()


def e5m2_nearest(v: Fraction) -> int:
    """Nearest finite E5M2 code to the exact value v (ties to the even code), with
    magnitudes at or above 57344 clamped to 57344; the sign bit follows v's sign."""
    sign = 0x80 if v < 0 else 0
    a = abs(v)
    if a >= 57344:
        return sign | 0x7B
    best = min(_E5M2, key=lambda cv: (abs(cv[1] - a), cv[0] & 1))
    return sign | best[0]


def fp8_nearest(kind: str, v: Fraction) -> int:
    return e4m3_nearest(v) if kind == "e4m3" else e5m2_nearest(v)
