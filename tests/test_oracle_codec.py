"""Pins of the oracle's FP8 codec (decode, saturating RNE encode) against
things other than itself: the constants the pages print, an independent
library (torch's float8 dtypes), a brute-force nearest-value search over all
2^32 binary32 patterns, and the mathematics of ties and saturation."""
import os

import numpy as np
import pytest
import torch

GOLD = os.path.join(os.path.dirname(__file__), "golden", "fp8_format_constants.txt")


def _golden():
    d = {}
    for line in open(GOLD):
        line = line.split("#", 1)[0].strip()
        if line:
            k, v = line.split()[:2]
            d[k] = v
    return d


TORCH_DT = {0: torch.float8_e4m3fn, 1: torch.float8_e5m2}
MAXCODE = {0: 0x7E, 1: 0x7B}


def torch_decode(fmt):
    return torch.arange(256, dtype=torch.uint8).view(TORCH_DT[fmt]).to(torch.float64).numpy()


def torch_encode_in_range(x_f32, fmt):
    """torch's RNE conversion, valid only for |x| <= max (it does not saturate)."""
    return torch.from_numpy(np.ascontiguousarray(x_f32, np.float32)).to(TORCH_DT[fmt]).view(torch.uint8).numpy()


@pytest.mark.parametrize("fmt", [0, 1])
def test_decode_matches_library_all_codes(O, fmt):
    ours = O.decode(np.arange(256, dtype=np.uint8), fmt)
    ref = torch_decode(fmt)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])


def test_decode_page_constants(O):
    g = _golden()
    for fmt, tag in [(0, "e4m3"), (1, "e5m2")]:
        v = O.decode(np.arange(256, dtype=np.uint8), fmt)
        fin = v[np.isfinite(v)]
        assert fin.max() == float(g[f"{tag}_max"]) == O.fp8_max(fmt)
        assert fin[fin > 0].min() == 2.0 ** int(g[f"{tag}_min_log2"])
        # field widths: number of binades (exponent codes) and steps per binade
        eb, mb = int(g[f"{tag}_exponent_bits"]), int(g[f"{tag}_mantissa_bits"])
        pos = np.sort(fin[fin > 0])
        normals = pos[pos >= 2.0 ** (int(g[f"{tag}_min_log2"]) + mb)]
        binades = np.unique(np.floor(np.log2(normals)))
        # E4M3 uses every exponent code for numbers; E5M2 reserves the top one
        assert len(binades) == (2 ** eb - 1 if fmt == 0 else 2 ** eb - 2)
        per = len(normals) / len(binades)
        assert per == 2 ** mb or (fmt == 0 and len(normals) == len(binades) * 2 ** mb - 1)


@pytest.mark.parametrize("fmt,nfinite", [(0, 254), (1, 248)])
def test_decode_structure(O, fmt, nfinite):
    v = O.decode(np.arange(256, dtype=np.uint8), fmt)
    assert np.isfinite(v).sum() == nfinite
    pos = v[:128]
    fin = pos[np.isfinite(pos)]
    assert np.all(np.diff(fin) > 0), "magnitude codes must be monotone"
    neg = v[128:]
    same = np.isfinite(pos)
    assert np.array_equal(-pos[same], neg[same])
    assert np.signbit(v[128]) and v[128] == 0.0


@pytest.mark.slow
@pytest.mark.parametrize("fmt", [0, 1])
def test_encode_exhaustive_vs_bruteforce(O, fmt):
    n, first = O.encode_exhaustive(fmt)
    assert n == 0, f"first mismatch at binary32 pattern {first:#010x}"


@pytest.mark.parametrize("fmt", [0, 1])
def test_encode_matches_library_in_range(O, fmt):
    rng = np.random.default_rng(7)
    mx = O.fp8_max(fmt)
    # every bf16 pattern in range, plus random binary32 over many binades
    allb = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    allb = allb[np.isfinite(allb) & (np.abs(allb) <= mx)]
    e = rng.uniform(-40, np.log2(mx), size=400_000)
    r = (np.exp2(e) * rng.choice([-1.0, 1.0], size=e.size)).astype(np.float32)
    r = r[np.abs(r) <= mx]
    x = np.concatenate([allb, r])
    assert np.array_equal(O.encode(x, fmt), torch_encode_in_range(x, fmt))


@pytest.mark.parametrize("fmt", [0, 1])
def test_encode_roundtrip_every_code(O, fmt):
    codes = np.arange(256, dtype=np.uint8)
    v = O.decode(codes, fmt)
    fin = np.isfinite(v)
    assert np.array_equal(O.encode(v[fin].astype(np.float32), fmt), codes[fin])


@pytest.mark.parametrize("fmt", [0, 1])
def test_encode_ties_go_to_even(O, fmt):
    v = O.decode(np.arange(0, MAXCODE[fmt] + 1, dtype=np.uint8), fmt)
    for c in range(MAXCODE[fmt]):
        mid = np.float32((v[c] + v[c + 1]) / 2)          # exact in binary32
        assert float(mid) == (v[c] + v[c + 1]) / 2
        want = c if c % 2 == 0 else c + 1
        assert O.encode(np.array([mid]), fmt)[0] == want
        assert O.encode(np.array([-mid]), fmt)[0] == want | 0x80
        below = np.nextafter(mid, np.float32(0))
        above = np.nextafter(mid, np.float32(np.inf))
        assert O.encode(np.array([below]), fmt)[0] == c
        assert O.encode(np.array([above]), fmt)[0] == c + 1


def test_encode_saturation_and_specials(O):
    f32 = lambda *a: np.array(a, dtype=np.float32)
    e4 = O.encode(f32(448, 463.99, 464, 464.01, 1e30, np.inf, -np.inf, -1e30), 0)
    assert list(e4) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
    e5 = O.encode(f32(57344, 61439, 61440, 61441, 1e30, np.inf, -np.inf), 1)
    assert list(e5) == [0x7B, 0x7B, 0x7B, 0x7B, 0x7B, 0x7B, 0xFB]
    nan = np.array([np.nan, -np.nan], dtype=np.float32)
    nan[1] = -np.abs(nan[1])
    assert list(O.encode(nan, 0)) == [0x7F, 0xFF]
    assert list(O.encode(nan, 1)) == [0x7F, 0xFF]
    # signed zero and underflow (Numerical stability deep dive > Underflow)
    t = 2.0 ** -10
    e4 = O.encode(f32(0.0, -0.0, t, np.nextafter(np.float32(t), np.float32(1)), -t, 1e-45), 0)
    assert list(e4) == [0x00, 0x80, 0x00, 0x01, 0x80, 0x00]
    t = 2.0 ** -17
    e5 = O.encode(f32(t, np.nextafter(np.float32(t), np.float32(1)), -t), 1)
    assert list(e5) == [0x00, 0x01, 0x80]
    # the brute-force encoder agrees on the same specials
    for x in [448, 464, 1e30, 2.0 ** -10, -0.0]:
        assert O.encode_brute(x, 0) == O.encode(f32(x), 0)[0]
