"""GPU checks of the two pieces of device arithmetic the parity contract rests on, through the
library's diagnostic entry points (which run them exactly as the production kernels do).

* The quantisation kernels' E4M3 encoder against the oracle's encoder (round to nearest even
  onto the OCP E4M3 grid, saturating) over every FP32 bit pattern with |x| <= 448 (1 + 2^-23):
  the codes of fl32(x * 448 / amax) can be any of them, and codes are compared bit for bit.
* The E4M3 matrix-core product (the QK and PV contraction) against the exact sum of the exact
  E4M3 products: the hardware truncates each group of 8 consecutive products before an FP32
  sum, so |device - exact| <= 2^-11 * sum over the 8 groups of the group's largest |product|.
  The oracle's tolerance model carries this bound; here it is tested on the chip.
"""
import sys
import time

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(*a):
    print("[gpu-diag]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def m():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_attention_video_qkv_amd as m
    m.lib()
    return m


def test_e4m3_encoder_exhaustive(m, orc):
    top = 0x43E00001 + 1          # patterns 0 .. bits(448 (1 + 2^-23)), and the same with the sign
    chunk = 1 << 26
    out = torch.empty(chunk, dtype=torch.uint8, device=DEV)
    total = 0
    t0 = time.time()
    for sign in (0, 0x80000000):
        for start in range(sign, sign + top, chunk):
            n = min(chunk, sign + top - start)
            n4 = (n + 3) // 4 * 4    # (up to 3 more patterns, still below 464)
            m.diag_e4m3_encode(start, n4, out)
            x = np.arange(start, start + n4, dtype=np.uint64).astype(np.uint32).view(np.float32)
            want = orc.e4m3_encode_f32(x)
            got = out[:n4].cpu().numpy()
            bad = np.flatnonzero(got != want)
            assert bad.size == 0, (hex(start + int(bad[0])), int(got[bad[0]]), int(want[bad[0]]), bad.size)
            total += n
        say(f"sign {'-' if sign else '+'}: {total} patterns equal so far ({time.time() - t0:.1f} s)")
    assert total == 2 * top


def test_e4m3_decoder_every_finite_code(m, orc):
    # every finite code (the encoders never write 0x7F / 0xFF), in an order that puts each code
    # at each byte position of a word; both device decoders against the oracle's exact values,
    # sign of zero included
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    codes = np.concatenate([np.roll(finite, k) for k in range(4)])
    codes = np.concatenate([codes, np.zeros((-codes.size) % 4, np.uint8)])
    got = m.diag_e4m3_decode(torch.from_numpy(codes).to(DEV)).cpu().numpy()
    want = orc.e4m3_decode(codes).astype(np.float32)
    for row, how in enumerate(("two codes per conversion", "one code per conversion")):
        bad = np.flatnonzero(got[row].view(np.uint32) != want.view(np.uint32))
        assert bad.size == 0, (how, hex(int(codes[bad[0]])), float(got[row][bad[0]]), float(want[bad[0]]))
    say(f"{codes.size} codes decoded equal to the oracle's values by both decoders")


def _tiles(orc, rng, kind, T):
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    if kind == "all_codes":
        a = rng.choice(finite, (T, 32, 64))
        b = rng.choice(finite, (T, 32, 64))
    elif kind == "normal":
        sa = rng.uniform(0.5, 100.0, (T, 1, 1))
        a = orc.e4m3_encode(rng.standard_normal((T, 32, 64)) * sa)
        b = orc.e4m3_encode(rng.standard_normal((T, 32, 64)) * 3.0)
    elif kind == "cancel":
        # products of equal magnitude and alternating sign, plus one small odd one per group
        a = orc.e4m3_encode(np.tile(rng.uniform(100.0, 448.0, (T, 32, 1)), (1, 1, 64)))
        sgn = np.where(np.arange(64) % 2 == 0, 1.0, -1.0)
        b = orc.e4m3_encode(rng.uniform(100.0, 448.0, (T, 32, 1)) * sgn[None, None, :])
        b[:, :, ::8] = orc.e4m3_encode(rng.uniform(2.0 ** -9, 2.0 ** -3, (T, 32, 8)))
    elif kind == "dominant":
        a = orc.e4m3_encode(rng.uniform(2.0 ** -9, 1.0, (T, 32, 64)) * np.where(rng.random((T, 32, 64)) < 0.5, 1, -1))
        b = orc.e4m3_encode(rng.uniform(2.0 ** -9, 1.0, (T, 32, 64)) * np.where(rng.random((T, 32, 64)) < 0.5, 1, -1))
        a[:, :, rng.integers(0, 64)] = 0x7E   # one product near 448 * 448 per row and column pair
        b[:, :, rng.integers(0, 64)] = 0x7E
    else:
        raise ValueError(kind)
    return np.ascontiguousarray(a, np.uint8), np.ascontiguousarray(b, np.uint8)


@pytest.mark.parametrize("kind", ["all_codes", "normal", "cancel", "dominant"])
def test_mfma_contraction_bound(m, orc, kind):
    rng = np.random.default_rng({"all_codes": 1, "normal": 2, "cancel": 3, "dominant": 4}[kind])
    T = 1024
    a, bt = _tiles(orc, rng, kind, T)
    got = m.diag_mfma_e4m3(torch.from_numpy(a).to(DEV), torch.from_numpy(bt).to(DEV)).cpu().numpy().astype(np.float64)
    av = orc.e4m3_decode(a).astype(np.float64)
    bv = orc.e4m3_decode(bt).astype(np.float64)
    prod = av[:, :, None, :] * bv[:, None, :, :]              # [T, 32, 32, 64], exact in FP64
    exact = prod.sum(axis=3)                                  # 64 exact products: exact in FP64
    bound = 2.0 ** -11 * np.abs(prod).reshape(T, 32, 32, 8, 8).max(axis=4).sum(axis=3)
    err = np.abs(got - exact)
    ratio = err / np.maximum(bound, 1e-300)
    say(f"{kind}: {np.mean(err > 0) * 100:.2f}% of outputs inexact, max error / bound {ratio.max():.3f}, "
        f"max relative error {float((err / np.maximum(np.abs(exact), 1e-300)).max()):.3e}")
    assert np.all(err <= bound)
