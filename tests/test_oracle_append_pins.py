"""Pins of the append oracle (oracle/append.py) against facts that do not
come from it: the OCP E4M3FN definition (every code round-trips, ties go to
the even code, saturation), torch's own float8 and bfloat16 casts as
independent library routines, the half-step error bound of round-to-nearest,
and the Fathom quantizer's closed form (cell midpoints, the clamped ends, the
oracle's own t-bit quantizer at t = 4).  CPU only.
"""
import numpy as np
import torch

from oracle import append as A
from oracle import oracle as O

RNG = np.random.default_rng(2024)


def test_every_finite_code_round_trips():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = O.decode_e4m3fn(codes)  # 0x80 decodes to -0.0
    assert np.signbit(vals[codes == 0x80]).all()
    assert np.array_equal(A.encode_e4m3fn(vals), codes)


def test_ties_go_to_the_even_code():
    pos = O.decode_e4m3fn(np.arange(0x7F, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2.0
    enc = A.encode_e4m3fn(mids).astype(np.int64)
    lo = np.arange(0x7E)
    exp = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(enc, exp)
    assert np.array_equal(A.encode_e4m3fn(-mids).astype(np.int64), exp | 0x80)


def test_saturation_and_signed_zero():
    enc = A.encode_e4m3fn(np.array([1000.0, -1000.0, 448.0, 0.0, -0.0]))
    assert list(enc) == [0x7E, 0xFE, 0x7E, 0x00, 0x80]


def test_encode_matches_torch_float8_cast():
    x = np.concatenate([RNG.normal(size=4000) * 50, RNG.normal(size=2000) * 0.01,
                        RNG.uniform(-448, 448, size=2000)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(A.encode_e4m3fn(x.astype(np.float64)), ref)


def test_index_key_quantisation_bound():
    for _ in range(20):
        k = (RNG.normal(size=128) * RNG.uniform(0.1, 10)).astype(np.float32)
        codes, sigma = A.quantize_index_key(k)
        assert sigma == np.float32(np.max(np.abs(k)) / np.float32(448))
        vals = O.decode_e4m3fn(codes) * float(sigma)
        # round to nearest: within half a step of the 3-bit mantissa (2^-4
        # relative) or half the subnormal step
        err = np.abs(vals - k.astype(np.float64))
        bound = np.maximum(np.abs(k) * 2.0 ** -4, float(sigma) * 2.0 ** -10) * (1 + 1e-6)
        assert np.all(err <= bound)
        i = int(np.argmax(np.abs(k)))
        assert codes[i] & 0x7F == 0x7E  # the largest element maps to 448
    codes, sigma = A.quantize_index_key(np.zeros(128, np.float32))
    assert sigma == 1.0 and np.all(codes == 0)


def test_fathom_code_closed_form():
    zero = np.float32(-1.25)
    cell = np.float32(0.125)
    mids = zero.astype(np.float64) + (np.arange(16) + 0.5) * float(cell)
    assert np.array_equal(A.fathom_code(mids.astype(np.float32), zero, cell), np.arange(16))
    assert A.fathom_code(np.float32(-5.0), zero, cell) == 0        # below the range
    assert A.fathom_code(np.float32(5.0), zero, cell) == 15        # above the range
    assert A.fathom_code(np.float32(3.0), zero, np.float32(0.0)) == 0  # constant channel
    x = RNG.uniform(-1.25, 0.75, size=500).astype(np.float32)
    assert np.array_equal(A.fathom_code(x, zero, cell),
                          O.fathom_tbit_quantize(x.astype(np.float64), float(zero),
                                                 float(cell), 4))


def test_bf16_rne_matches_torch_cast():
    x = np.concatenate([RNG.normal(size=5000), RNG.normal(size=1000) * 1e-30]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(A.bf16_rne(x), ref)


def test_plane_bits_round_trip():
    D, n = 5, 70
    codes = RNG.integers(0, 16, size=(n, D))
    planes = np.zeros((D, 4, (n + 31) // 32), dtype=np.int32)
    for t in range(n):
        A.set_plane_bits(planes, t, codes[t])
    # read back: bit (3 - j) of token t's code sits in plane j, word t // 32
    u = planes.view(np.uint32).astype(np.int64)
    back = np.zeros_like(codes)
    for t in range(n):
        for j in range(4):
            back[t] |= ((u[:, j, t // 32] >> (t % 32)) & 1) << (3 - j)
    assert np.array_equal(back, codes)
    # overwriting a token replaces its bits only
    A.set_plane_bits(planes, 33, np.zeros(D, np.int64))
    u2 = planes.view(np.uint32).astype(np.int64)
    assert np.all(((u2[:, :, 1] >> 1) & 1) == 0)
    assert np.array_equal(u2[:, :, 0], u[:, :, 0])
