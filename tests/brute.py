"""Pure-Python brute force for tiny inputs, written separately from the C oracle.

It works from Python floats, exact rationals (fractions.Fraction) and
exhaustive subset search, and shares nothing with the oracle or the HIP path.
Only sizes of a few hundred tokens are practical.

Layout: arrays are nested lists of Python floats: q[b][h][t], K[b][j][i][t].
"""
from __future__ import annotations

import itertools
import math
import struct
from fractions import Fraction


def bits_to_float_bf16(bits: int) -> float:
    return struct.unpack(">f", struct.pack(">I", (bits & 0xFFFF) << 16))[0]


def round_to_bf16_bits(x: Fraction | float) -> int:
    """Exact rational -> nearest bfloat16 (ties to even), by exact comparison."""
    x = Fraction(x)
    sign = 0x8000 if x < 0 else 0
    a = abs(x)
    if a == 0:
        return sign
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    ulp = Fraction(2) ** (e - 7) if e >= -126 else Fraction(2) ** -133
    quot = a / ulp
    fl = quot.numerator // quot.denominator
    rem = quot - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    if e < -126:  # subnormal (fl == 128 is the smallest normal, bit pattern 0x0080)
        return sign | fl
    if fl == 256:
        fl, e = 128, e + 1
    if e > 127:
        return sign | 0x7F80
    return sign | ((e + 127) << 7) | (fl - 128)


def round_to_f32(x: Fraction) -> float:
    """Exact rational -> nearest binary32 (ties to even), by exact comparison."""
    x = Fraction(x)
    sign = -1 if x < 0 else 1
    a = abs(x)
    if a == 0:
        return 0.0
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    ulp = Fraction(2) ** (e - 23) if e >= -126 else Fraction(2) ** -149
    quot = a / ulp
    fl = quot.numerator // quot.denominator
    rem = quot - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * float(fl * ulp)


def n_blocks(n: int, L: int) -> int:
    return (n + L - 1) // L


def block_tokens(n: int, L: int, b: int) -> range:
    return range(b * L, min(n, (b + 1) * L))


def mean_rows(rows, dtype: str):
    """Exact mean of stored rows, rounded once to the storage dtype (returns float values)."""
    d = len(rows[0])
    out = []
    for t in range(d):
        m = sum(Fraction(r[t]) for r in rows) / len(rows)
        out.append(bits_to_float_bf16(round_to_bf16_bits(m)) if dtype == "bf16" else round_to_f32(m))
    return out


def dot(a, b) -> float:
    return math.fsum(x * y for x, y in zip(a, b))


def lse(vals) -> float:
    m = max(vals)
    return m + math.log(math.fsum(math.exp(v - m) for v in vals))


def softmax_avg(logits, values):
    m = max(logits)
    w = [math.exp(l - m) for l in logits]
    z = math.fsum(w)
    d = len(values[0])
    out = [math.fsum(w[e] * values[e][t] for e in range(len(w))) / z for t in range(d)]
    return out, m + math.log(z)


def summaries(K, L, dtype):
    n = len(K)
    return [mean_rows([K[i] for i in block_tokens(n, L, b)], dtype) for b in range(n_blocks(n, L))]


def head_block_logits(qh, K, Kbar, L, scale, mode):
    n = len(K)
    nb = n_blocks(n, L)
    if mode == "summary":
        return [scale * dot(qh, Kbar[b]) + math.log(len(block_tokens(n, L, b))) for b in range(nb)]
    return [lse([scale * dot(qh, K[i]) for i in block_tokens(n, L, b)]) for b in range(nb)]


def group_scores(logits_per_head):
    """COBS Eq. (5) in the log domain: ln sum_g m_b^(g) / Z^(g)."""
    G = len(logits_per_head)
    if G == 1:
        return list(logits_per_head[0])
    nb = len(logits_per_head[0])
    Z = [math.fsum(math.exp(x) for x in row) for row in logits_per_head]
    return [math.log(math.fsum(math.exp(logits_per_head[g][b]) / Z[g] for g in range(G))) for b in range(nb)]


def best_subset(scores, k):
    """Exhaustive search: the k-subset with the largest exact score sum; among equal sums the
    lexicographically smallest sorted index tuple (i.e. ties go to lower indices)."""
    nb = len(scores)
    k = min(k, nb)
    exact = [Fraction(s) for s in scores]
    best, best_sum = None, None
    for S in itertools.combinations(range(nb), k):  # lexicographic order
        tot = sum((exact[b] for b in S), Fraction(0))
        if best_sum is None or tot > best_sum:
            best, best_sum = S, tot
    return list(best)


def attend_head(qh, K, V, Kbar, Vbar, L, scale, sel, proxies, tok=()):
    """Softmax over exact tokens of sel, weighted tokens (idx, logw) and proxies."""
    n = len(K)
    logits, values = [], []
    for b in sel:
        for i in block_tokens(n, L, b):
            logits.append(scale * dot(qh, K[i]))
            values.append(V[i])
    for idx, lw in tok:
        logits.append(scale * dot(qh, K[idx]) + lw)
        values.append(V[idx])
    if proxies:
        for b in range(n_blocks(n, L)):
            if b not in sel:
                logits.append(scale * dot(qh, Kbar[b]) + math.log(len(block_tokens(n, L, b))))
                values.append(Vbar[b])
    return softmax_avg(logits, values)


def pipeline(q, K, V, L, k, mode, proxies, dtype, scale=None, tok=None):
    """The whole path for q[b][h], K/V[b][j]: returns (Kbar, Vbar, scores, sel, out, lse)."""
    B, Hq, Hkv = len(q), len(q[0]), len(K[0])
    G = Hq // Hkv
    d = len(q[0][0])
    scale = scale if scale is not None else 1.0 / math.sqrt(d)
    res = {"Kbar": [], "Vbar": [], "score": [], "sel": [], "out": [], "lse": []}
    for b in range(B):
        for x in res.values():
            x.append([])
        for j in range(Hkv):
            Kb, Vb = summaries(K[b][j], L, dtype), summaries(V[b][j], L, dtype)
            heads = [q[b][j * G + g] for g in range(G)]
            logits = [head_block_logits(qh, K[b][j], Kb, L, scale, mode) for qh in heads]
            sc = group_scores(logits)
            S = best_subset(sc, k)
            res["Kbar"][b].append(Kb)
            res["Vbar"][b].append(Vb)
            res["score"][b].append(sc)
            res["sel"][b].append(S)
            t = tok[b][j] if tok else ()
            for qh in heads:
                o, l = attend_head(qh, K[b][j], V[b][j], Kb, Vb, L, scale, S, proxies, t)
                res["out"][b].append(o)
                res["lse"][b].append(l)
    return res
