"""Pin of the oracle's bfloat16 decoder (oracle.round.widen) against torch's own
bfloat16 -> float64 conversion, on every one of the 65536 encodings that is not a
NaN, and on hand-checked values: a bfloat16 is the upper half of an IEEE binary32."""
import numpy as np
import torch

import oracle


def test_widen_matches_torch_on_every_encoding():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.round.widen(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2 * 127          # exponent all ones, nonzero mantissa, both signs
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_widen_hand_values():
    enc = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x7F80, 0xFF80, 0x0001, 0x3FC0, 0x4049],
                   dtype=np.uint16)
    want = [1.0, -2.0, 0.0, -0.0, np.inf, -np.inf, 2.0 ** -133, 1.5, 3.140625]
    got = oracle.round.widen(enc)
    assert got.dtype == np.float64
    assert got.tolist() == want
    assert np.signbit(got[3])


def test_widen_passes_fp32_through_exactly():
    x = np.array([1.0, -0.1, 3.4e38, 1e-45], dtype=np.float32)
    assert oracle.round.widen(x).tolist() == [float(v) for v in x]
