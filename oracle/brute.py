"""Exact rational brute force for tiny inputs (fractions.Fraction, pure Python loops).

TEST INFRASTRUCTURE ONLY (see the package docstring).  These follow the
definitions of "bitsandbytes deep dive" section 5.2 (q = argmin_j |u - c_j|,
u = w/a) and section 7.2 (8-bit first-level scales over 0..255) literally, with
no threshold rewriting, and exist to pin the vectorized forms in oracle.nf4.
"""
from fractions import Fraction


def argmin_lower(values, target):
    """Index of the value nearest to target; ties go to the lower index."""
    best, best_d = None, None
    for j, v in enumerate(values):
        d = abs(target - v)
        if best_d is None or d < best_d:
            best, best_d = j, d
    return best


def nf4_codes_block(block, table, zero_code=7):
    """Codes of one block by the literal definition: a = max|w|, u = w/a, nearest level."""
    ws = [Fraction(float(w)) for w in block]
    cs = [Fraction(float(c)) for c in table]
    a = max(abs(w) for w in ws)
    if a == 0:
        return [zero_code] * len(ws)
    return [argmin_lower(cs, w / a) for w in ws]


def fp4_codes_block(block, table):
    """FP4 codes of one block by the literal definition: the code whose level is nearest to u = w/a.

    table: the 16 float32 levels in code order.  Among equally near codes the
    lower level wins, and between the two zeros (+0, code 0 and -0, code 8)
    code 0; an all-zero block is all code 0.
    """
    ws = [Fraction(float(w)) for w in block]
    cs = [Fraction(float(c)) for c in table]
    a = max(abs(w) for w in ws)
    if a == 0:
        return [0] * len(ws)
    out = []
    for w in ws:
        u = w / a
        out.append(min(range(16), key=lambda c: (abs(u - cs[c]), cs[c], c)))
    return out


def scale_code(a, A2):
    """q8 = argmin_k |a/A2 - k/255| over k = 0..255, ties to the lower k; A2 = 0 gives 0."""
    a, A2 = Fraction(float(a)), Fraction(float(A2))
    if A2 == 0:
        return 0
    levels = [Fraction(k, 255) for k in range(256)]
    return argmin_lower(levels, a / A2)


def round_f32(x):
    """Nearest IEEE binary32 to the rational x (ties to even), normal range, as a Fraction."""
    x = Fraction(x)
    if x == 0:
        return Fraction(0)
    s = -1 if x < 0 else 1
    m = abs(x)
    e = m.numerator.bit_length() - m.denominator.bit_length()
    while Fraction(2) ** e > m:
        e -= 1
    while Fraction(2) ** (e + 1) <= m:
        e += 1
    assert -126 <= e <= 127, "normal range only"
    ulp = Fraction(2) ** (e - 23)
    q, r = divmod(m, ulp)                # m = q*ulp + r, 0 <= r < ulp
    if r * 2 > ulp or (r * 2 == ulp and q % 2 == 1):
        q += 1
    return s * q * ulp
