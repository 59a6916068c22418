"""Pure-Python brute-force twins of the oracle, for tiny inputs.

TEST INFRASTRUCTURE ONLY (same rule as mdc_oracle: only tests/, smoke() and
the cpu_baseline leg of bench.py may use it).  Written as independent
formulations of the same definitions, so that a mistake in one does not hide
in the other:

  * dispatch: sorted() of (local expert, src, token, k) tuples instead of a
    stable bucket pass; counts by dictionary; prefix sums by running total;
  * fp32 arithmetic: Python floats (binary64) rounded to binary32 through
    struct after every operation.  A product or sum of two binary32 values
    computed in binary64 and then rounded to binary32 equals the correctly
    rounded binary32 result (binary64 carries more than 2*24+2 bits);
  * bf16 rounding: exact rational comparison of the two neighbouring bf16
    values (fractions.Fraction), ties to the even significand.
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction


def f32(v: float) -> float:
    return struct.unpack("<f", struct.pack("<f", v))[0]


def bits_to_float_bf16(b: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (b & 0xFFFF) << 16))[0]


def _bf16_value(b: int) -> Fraction:
    return Fraction(bits_to_float_bf16(b))


def bf16_round(v: float) -> int:
    """Nearest bf16 to a binary32 value v, ties to even significand, by exact comparison."""
    if math.isnan(v):
        return 0x7FC0 | (0x8000 if math.copysign(1.0, v) < 0 else 0)
    if v == 0.0:
        return 0x8000 if math.copysign(1.0, v) < 0 else 0x0000
    sign = 0x8000 if v < 0 else 0
    mag = abs(v)
    # candidates: largest bf16 <= mag (by truncating the binary32 pattern) and the next one up
    u = struct.unpack("<I", struct.pack("<f", mag))[0]
    lo = u >> 16
    hi = lo + 1
    fv = Fraction(mag)
    dlo = fv - _bf16_value(lo)
    if hi >= 0x7F80:          # next one up is inf: compare against the overflow threshold
        dhi = Fraction(2) ** 128 - fv
    else:
        dhi = _bf16_value(hi) - fv
    if dlo < dhi:
        pick = lo
    elif dhi < dlo:
        pick = hi
    else:
        pick = lo if lo % 2 == 0 else hi
    return sign | pick


def dropped(ids, mask, n_ids):
    """Active routes whose id is below 0 or at least n_ids, counted one by one over a flat list of routes."""
    flat = []
    for s, rank_ids in enumerate(ids):
        for t, tok in enumerate(rank_ids):
            for k, e in enumerate(tok):
                flat.append((s, t, k, int(e)))
    n = 0
    for s, t, k, e in flat:
        if mask is not None:
            m = mask[s][t]
            if not (m[k] if isinstance(m, (list, tuple)) else m):
                continue
        if not (0 <= e < n_ids):
            n += 1
    return n


def expand_scales(rows, scales):
    """Weight of each received row's route, looked up by its (s, t, k) triplet."""
    return [f32(float(scales[s][t][k])) for (s, t, k) in rows]


def dispatch(ids, mask, d, experts, capacity, x=None):
    """Brute-force dispatch: returns (rows list of (s,t,k), counts dict, epRecvCounts list, expertTokenNums list, expand rows)."""
    W = len(ids)
    BS = len(ids[0])
    K = len(ids[0][0])
    L = experts // W
    tuples = []
    for s in range(W):
        for t in range(BS):
            for k in range(K):
                if mask is not None:
                    m = mask[s][t]
                    if not (m[k] if isinstance(m, (list, tuple)) else m):
                        continue
                e = int(ids[s][t][k])
                if e < 0 or e >= experts:
                    continue
                if e // L != d:
                    continue
                tuples.append((e - d * L, s, t, k))
    tuples = sorted(tuples)
    cnt = {}
    for le, s, _, _ in tuples:
        cnt[(le, s)] = cnt.get((le, s), 0) + 1
    ep = []
    run = 0
    for le in range(L):
        for s in range(W):
            run += cnt.get((le, s), 0)
            ep.append(run)
    etn = [sum(cnt.get((le, s), 0) for s in range(W)) for le in range(L)]
    rows = [(s, t, k) for (_, s, t, k) in tuples][:capacity]
    expand = None
    if x is not None:
        expand = [list(x[s][t]) for (s, t, k) in rows]
    return rows, cnt, ep, etn, expand


def combine(segments, r, ids_r, mask_r, scales_r, shared_r, hidden, experts=None, zero=0, copy=0, ori=None):
    """segments: list of (y rows [list of bf16 ints], triplets [list of (s,t,k)]); returns list of bf16 rows.

    Special experts: id in [experts, experts+zero) -> output row of zeros;
    [experts+zero, experts+zero+copy) -> the token's own row ori[t].
    """
    BS = len(ids_r)
    K = len(ids_r[0])
    found = {}
    for j, (yrows, trip) in enumerate(segments):
        for row, (s, t, k) in enumerate(trip):
            if s == r:
                found[(t, k)] = yrows[row]
    out = []
    for t in range(BS):
        acc = [0.0] * hidden
        for k in range(K):
            if mask_r is not None:
                m = mask_r[t]
                if not (m[k] if isinstance(m, (list, tuple)) else m):
                    continue
            y = found.get((t, k))
            if y is None and experts is not None:
                e = int(ids_r[t][k])
                if experts <= e < experts + zero:
                    y = [0] * hidden
                elif experts + zero <= e < experts + zero + copy:
                    y = list(ori[t])
            if y is None:
                continue
            sc = f32(float(scales_r[t][k]))
            for h in range(hidden):
                a = f32(sc * bits_to_float_bf16(int(y[h])))
                if shared_r is not None:
                    b = f32(sc * bits_to_float_bf16(int(shared_r[t][h])))
                    acc[h] = f32(acc[h] + f32(a + b))
                else:
                    acc[h] = f32(acc[h] + a)
        out.append([bf16_round(v) for v in acc])
    return out


def int_matmul(a, b_t):
    """Exact integer a[m][k] . b_t[n][k]^T with Python ints."""
    return [[sum(int(x) * int(y) for x, y in zip(row, col)) for col in b_t] for row in a]
