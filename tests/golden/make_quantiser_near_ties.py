"""Write quantiser_near_ties.json: rows whose int8 codes depend on how the
quantiser's division is carried out.

The reading of the int8 KV cache ("Character.AI: inference optimization",
section 05: the attention KV cache is int8; the scheme is not given on the
page) is: per token row x, a = max|x|, s = fl32(a / 127), and each code is
rint(fl32(x / s)) (round half to even), clamped to [-127, 127].  Two other
ways to write the same formula round differently near a tie:
    x * fl32(1 / s)      (a reciprocal, then a product)
    x * fl32(127 / a)    (the inverse scale, then a product)
This script searches rows where the three forms give different codes, so
that a quantiser written either way fails the pin.

Every value is derived here with exact rational arithmetic (Python's
``fractions``) and a round-to-nearest-even onto the fp32 grid written out
below; nothing else is called -- no numpy, no oracle, no GPU.

    python tests/golden/make_quantiser_near_ties.py
"""
import json
import os
import random
from fractions import Fraction

HERE = os.path.dirname(os.path.abspath(__file__))
OUT = os.path.join(HERE, "quantiser_near_ties.json")


# --------------------------------------------------------------------------
# IEEE binary32 round-to-nearest-even of an exact rational
# --------------------------------------------------------------------------
def _rne_int(q: Fraction) -> int:
    """Nearest integer to q, ties to even."""
    f = q.numerator // q.denominator            # floor
    r = q - f
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and f % 2 == 1):
        f += 1
    return f


def fl32(q: Fraction) -> Fraction:
    """q rounded to the nearest binary32 value (ties to even), as a Fraction.
    Subnormals are handled; overflow is not needed here and is refused."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -126)                              # subnormal range: fixed spacing 2^-149
    ulp = Fraction(2) ** (e - 23)
    m = _rne_int(a / ulp)
    out = m * ulp
    if out >= Fraction(2) ** 128:
        raise OverflowError(q)
    return sign * out


def f32_bits(q: Fraction) -> int:
    """Bit pattern of an exactly representable binary32 value."""
    assert fl32(q) == q
    if q == 0:
        return 0
    sign = 0x80000000 if q < 0 else 0
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    if e < -126:                                  # subnormal
        return sign | int(a / Fraction(2) ** -149)
    m = a / Fraction(2) ** e                      # in [1, 2)
    frac = int((m - 1) * 2 ** 23)
    return sign | ((e + 127) << 23) | frac


def f32_from_bits(b: int) -> Fraction:
    sign = -1 if b & 0x80000000 else 1
    e = (b >> 23) & 0xFF
    frac = b & 0x7FFFFF
    assert e != 0xFF
    if e == 0:
        return sign * Fraction(frac) * Fraction(2) ** -149
    return sign * (1 + Fraction(frac, 2 ** 23)) * Fraction(2) ** (e - 127)


def next_up(q: Fraction) -> Fraction:
    return f32_from_bits(f32_bits(q) + 1) if q > 0 else -f32_from_bits(f32_bits(-q) - 1)


def next_down(q: Fraction) -> Fraction:
    return f32_from_bits(f32_bits(q) - 1) if q > 0 else -f32_from_bits(f32_bits(-q) + 1)


# --------------------------------------------------------------------------
# The three ways of forming the code
# --------------------------------------------------------------------------
def clamp127(n: int) -> int:
    return max(-127, min(127, n))


def code_divide(x: Fraction, a: Fraction, s: Fraction) -> int:
    return clamp127(_rne_int(fl32(x / s)))


def code_reciprocal(x: Fraction, a: Fraction, s: Fraction) -> int:
    return clamp127(_rne_int(fl32(x * fl32(1 / s))))


def code_inverse_scale(x: Fraction, a: Fraction, s: Fraction) -> int:
    return clamp127(_rne_int(fl32(x * fl32(Fraction(127) / a))))


def find_row(rng: random.Random, per_row: int):
    """A row: its max |x| first, then per_row near-tie elements for which the
    division form differs from at least one of the other two forms (and each
    of the two other forms differs on at least one element of the row)."""
    while True:
        # a random fp32 max in [0.5, 8): s = a/127 is then never a power of two
        a = fl32(Fraction(rng.randrange(1 << 23, 1 << 26), 1 << 23))
        s = fl32(a / 127)
        elems = []
        seen_rec = seen_inv = False
        for _ in range(4000):
            k = rng.randrange(-126, 126)
            t = (Fraction(2 * k + 1, 2)) * s          # an exact tie of x / s
            x0 = fl32(t)
            for x in (x0, next_up(x0), next_down(x0)):
                if abs(x) >= a or x == 0:
                    continue
                cd = code_divide(x, a, s)
                cr = code_reciprocal(x, a, s)
                ci = code_inverse_scale(x, a, s)
                if cd != cr or cd != ci:
                    if any(e[0] == x for e in elems):
                        continue
                    elems.append((x, cd, cr, ci))
                    seen_rec |= cd != cr
                    seen_inv |= cd != ci
                    break
            if len(elems) >= per_row and seen_rec and seen_inv:
                break
        if len(elems) >= per_row and seen_rec and seen_inv:
            return a, s, elems


def main():
    rng = random.Random(20240620)
    rows = []
    for sign in (1, -1, 1, -1, 1, 1):
        a, s, elems = find_row(rng, 12)
        xs = [sign * a] + [e[0] for e in elems]
        row = {
            "x_bits": ["0x%08x" % f32_bits(x) for x in xs],
            "x": [float(x) for x in xs],
            "scale_bits": "0x%08x" % f32_bits(s),
            "codes": [code_divide(x, a, s) for x in xs],
            "codes_if_reciprocal": [code_reciprocal(x, a, s) for x in xs],
            "codes_if_inverse_scale": [code_inverse_scale(x, a, s) for x in xs],
        }
        rows.append(row)
    doc = {
        "_source": (
            "Reading of the int8 KV quantiser ('Character.AI: inference optimization', section 05: "
            "the attention KV cache is int8; the scheme itself is not on the page): a = max|x|, "
            "s = fl32(a / 127), code = rint(fl32(x / s)) with ties to even, clamped to [-127, 127]. "
            "The rows are near ties of x / s, chosen so that x * fl32(1 / s) or x * fl32(127 / a) "
            "gives another code on some element.  Derived with exact rational arithmetic by "
            "make_quantiser_near_ties.py (no numpy, no oracle, no GPU).  Element 0 of each row "
            "is the row's max |x|; x_bits are the fp32 inputs, x the same values as decimals."),
        "rows": rows,
    }
    with open(OUT, "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")
    n_rec = sum(c != d for r in rows for c, d in zip(r["codes"], r["codes_if_reciprocal"]))
    n_inv = sum(c != d for r in rows for c, d in zip(r["codes"], r["codes_if_inverse_scale"]))
    print(f"wrote {OUT}: {len(rows)} rows; reciprocal form differs on {n_rec} codes, "
          f"inverse-scale form on {n_inv}")


if __name__ == "__main__":
    main()
