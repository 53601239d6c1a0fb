"""The device's fp32 -> bf16 storage rounding, bit for bit, through the C ABI.

Every bf16 output of the step (activations, expert rows, hidden states) is an
fp32 value rounded to bf16 by the kernels' one conversion helper (the gfx950
packed conversion instruction).  moe_combine in bf16 with one routed row per
token and no shared rows stores

    combined = bf16(fmaf(w, y, 0))        out = bf16(h + fmaf(w, y, 0))

so choosing the fp32 weight w and the bf16 bit patterns of y and h drives
arbitrary fp32 values through that rounding: random bit patterns (denormals,
infinities, NaN), exact ties and near-ties at every exponent, products that
land among the fp32 denormals, and overflow past the largest bf16.  The
expected bits are computed on the host: the fp32 product and sum in numpy
float32 (IEEE, round to nearest even), then round-to-nearest-even on the
integer bits of the fp32 value (a NaN stays a NaN; its payload is not
compared, since which operand's payload an fp32 add passes on is not fixed
by IEEE 754).
"""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def m():
    import moe_decoder_step_amd as mod
    mod.load()
    assert torch.cuda.is_available(), "GPU tests need a device"
    return mod


def _bf16_rne(x32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits, round to nearest, ties to even, on the integer bits."""
    u = x32.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(x32)
    r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return r


def _f32(bits16: np.ndarray) -> np.ndarray:
    return (bits16.astype(np.uint32) << 16).view(np.float32)


def _to_dev(bits16: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(bits16.astype(np.uint16).view(np.int16)).to(DEV).view(torch.bfloat16)


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _cases(rng: np.random.Generator, T: int, H: int):
    """Per token a weight w (fp32) and per element y, h (bf16 bits), by regime."""
    y = np.zeros((T, H), np.uint16)
    h = np.zeros((T, H), np.uint16)
    w = np.ones(T, np.float32)
    rand16 = lambda n: rng.integers(0, 1 << 16, size=n, dtype=np.uint32).astype(np.uint16)  # noqa: E731
    for t in range(T):
        kind = t % 8
        if kind == 0:      # every bf16 pattern for y (NaN, inf, denormals), arbitrary fp32 weight
            y[t] = rand16(H)
            w[t] = np.float32(rng.uniform(0.5, 2.0))
        elif kind == 1:    # ... and a random residual on top
            y[t] = rand16(H)
            h[t] = rand16(H)
            w[t] = np.float32(rng.uniform(-2.0, 2.0))
        elif kind == 2:    # exact ties: h + y with y half a bf16 ulp of h, h's mantissa odd or even
            e = rng.integers(1, 254, size=H).astype(np.uint32)           # exponent of h
            mh = rng.integers(0, 128, size=H).astype(np.uint32)          # mantissa of h (7 bits)
            sign = rng.integers(0, 2, size=H).astype(np.uint32) << 15
            h[t] = (sign | (e << 7) | mh).astype(np.uint16)
            ey = e.astype(np.int64) - 8                                   # y = 2^(e-127-8): half an ulp of h
            ok = ey >= 1
            y[t] = np.where(ok, (sign | (np.maximum(ey, 1).astype(np.uint32) << 7)), 0).astype(np.uint16)
            w[t] = np.float32(1.0)
        elif kind == 3:    # y = +-2^e, so the product is w scaled exactly: ties to even (down and
            # up) and values one fp32 ulp either side of a tie, at every exponent
            y[t] = ((rng.integers(0, 2, size=H).astype(np.uint32) << 15)
                    | (rng.integers(20, 230, size=H).astype(np.uint32) << 7)).astype(np.uint16)
            tie_even, tie_odd = 1.0 + 2.0 ** -8, 1.0 + 2.0 ** -7 + 2.0 ** -8
            w[t] = np.float32([tie_even, tie_odd, tie_even + 2.0 ** -23, tie_even - 2.0 ** -23,
                               tie_odd + 2.0 ** -23, tie_odd - 2.0 ** -23][(t // 8) % 6])
        elif kind == 4:    # products among the fp32 denormals (bf16 rounding of a denormal)
            y[t] = ((rng.integers(0, 2, size=H).astype(np.uint32) << 15)
                    | (rng.integers(1, 12, size=H).astype(np.uint32) << 7)
                    | rng.integers(0, 128, size=H).astype(np.uint32)).astype(np.uint16)
            w[t] = np.float32(rng.uniform(1.0, 2.0)) * np.float32(2.0 ** -12)
        elif kind == 5:    # bf16 denormal inputs with an arbitrary weight
            y[t] = ((rng.integers(0, 2, size=H).astype(np.uint32) << 15)
                    | rng.integers(0, 128, size=H).astype(np.uint32)).astype(np.uint16)
            w[t] = np.float32(rng.uniform(0.25, 4.0))
        elif kind == 6:    # overflow past the largest bf16 and into infinity
            y[t] = ((rng.integers(0, 2, size=H).astype(np.uint32) << 15)
                    | (rng.integers(240, 255, size=H).astype(np.uint32) << 7)
                    | rng.integers(0, 128, size=H).astype(np.uint32)).astype(np.uint16)
            w[t] = np.float32(rng.uniform(1.0, 2.0)) * np.float32(2.0 ** 12)
        else:              # ordinary magnitudes, random residual
            y[t] = _bf16_rne(rng.standard_normal(H).astype(np.float32))
            h[t] = _bf16_rne(rng.standard_normal(H).astype(np.float32))
            w[t] = np.float32(rng.uniform(0.0, 1.0))
    return y, h, w


@pytest.mark.parametrize("seed", [0, 1])
def test_storage_rounding_bits(m, seed):
    T, H = 512, 1280
    rng = np.random.default_rng(1000 + seed)
    y, h, w = _cases(rng, T, H)
    yd, hd = _to_dev(y), _to_dev(h)
    wd = torch.from_numpy(w.reshape(T, 1)).to(DEV)
    inv = torch.arange(T, dtype=torch.int32, device=DEV)
    out, comb = m.combine_alloc(yd, inv, wd, None, 0, hd)
    torch.cuda.synchronize()

    with np.errstate(over="ignore", invalid="ignore"):
        # fmaf(w, y, +0): the product rounded once, then + 0 (a -0 product becomes +0)
        prod = (w[:, None] * _f32(y)).astype(np.float32) + np.float32(0.0)
        total = (_f32(h) + prod).astype(np.float32)
    for name, got, val in (("combined", _bits(comb), prod), ("out", _bits(out), total)):
        ref = _bf16_rne(val)
        nan = np.isnan(val)
        got_nan = ((got & 0x7F80) == 0x7F80) & ((got & 0x7F) != 0)
        assert np.array_equal(got_nan, nan), f"{name}: NaN-ness differs at {np.argwhere(got_nan != nan)[:5]}"
        bad = (got != ref) & ~nan
        assert not bad.any(), (f"{name}: {bad.sum()} of {bad.size} values round differently; first "
                               f"{[(hex(int(v.view(np.uint32))), hex(int(g)), hex(int(r))) for v, g, r in zip(val[bad][:4], got[bad][:4], ref[bad][:4])]}")
    # the regimes were reached: ties, denormal results, infinities
    assert (np.abs(total.view(np.uint32).astype(np.int64) & 0xFFFF) == 0x8000).sum() > 100
    assert ((prod != 0) & (np.abs(prod) < np.float32(2.0 ** -126))).sum() > 1000
    assert np.isinf(prod).sum() > 100
