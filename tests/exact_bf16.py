"""Round-to-nearest-even of an exact rational to bf16, written from the
definition (8 significant bits, ties to the even neighbour), for the pins
that check the oracle's roundings against exact arithmetic."""
from fractions import Fraction

import numpy as np
import torch


def bf16_rne_of_fraction(fr: Fraction) -> int:
    """bf16 bits of the exact rational fr rounded to 8 significant bits, ties to even."""
    if fr == 0:
        return 0
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    assert Fraction(2) ** e <= a < Fraction(2) ** (e + 1)
    unit = Fraction(2) ** (e - 7)
    n = a / unit                      # in [128, 256)
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    v = float(fl * unit) * (-1 if fr < 0 else 1)
    assert Fraction(v) == fl * unit * (-1 if fr < 0 else 1)
    # v has at most 8 significant bits: the fp32 -> bf16 conversion is exact
    t = torch.tensor([v], dtype=torch.float32).to(torch.bfloat16).view(torch.int16)
    return int(t.numpy().view(np.uint16)[0])
