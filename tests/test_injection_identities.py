"""The pages' bit identities for building matrix-unit operands from packed
codes (rag-lover.com explainer), checked against torch/numpy's own decoding of
those floating-point formats, plus the binary16-subnormal identity the GPU
library relies on."""
import os
from fractions import Fraction

import numpy as np
import torch


def _cases():
    path = os.path.join(os.path.dirname(__file__), "golden", "injection_identities.txt")
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        lhs, rhs = line.split("->")
        name, code = lhs.split()
        yield name, int(code), Fraction(rhs.strip())


def _e2m1(nibble):
    # decode one fp4 E2M1 value with torch's packed fp4 dtype (low nibble = first element)
    t = torch.tensor([nibble & 0xF], dtype=torch.uint8).view(torch.float4_e2m1fn_x2)
    # torch has no direct float conversion for x2; decode the format by definition
    # only as a fallback
    try:
        return float(t.to(torch.float32)[0])
    except Exception:
        e, m = (nibble >> 1) & 3, nibble & 1
        return (m / 2) if e == 0 else (1 + m / 2) * 2.0 ** (e - 1)


def test_page_identities():
    seen = set()
    for name, code, want in _cases():
        seen.add(name)
        if name == "bf16_or_0x4300":
            got = torch.tensor([0x4300 | code], dtype=torch.int16).view(torch.bfloat16).float().item()
        elif name == "e4m3_low_bits":
            got = torch.tensor([code], dtype=torch.uint8).view(torch.float8_e4m3fn).float().item()
        elif name == "e2m1_low_bits":
            got = _e2m1(code)
        else:
            raise AssertionError(name)
        assert Fraction(got) == want, (name, code, got, want)
    assert seen == {"bf16_or_0x4300", "e2m1_low_bits", "e4m3_low_bits"}


def test_e4m3_low_nibble_is_linear_for_all_int4_codes():
    got = torch.arange(16, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    assert np.array_equal(got, np.arange(16) / 512.0)


def test_binary16_subnormal_codes():
    # INT4: nibbles at bit offsets 0 and 4; INT2: pairs at offsets 0, 2, 4, 6, 8
    for bits, offsets in ((4, (0, 4)), (2, (0, 2, 4, 6, 8))):
        for k in offsets:
            for c in range(1 << bits):
                v = np.array([c << k], np.uint16).view(np.float16).astype(np.float64)[0]
                assert v == c * 2.0 ** k * 2.0 ** -24
