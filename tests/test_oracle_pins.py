"""Pins of the CPU oracle to the mathematics and to hand-worked examples (CPU only).

Each test checks the oracle against something other than itself: textbook closed forms
(Sylvester's Hadamard matrix via scipy), exhaustive enumeration of binary16, brute force on small
inputs, invariants the method guarantees, and worked examples derived by hand (tests/golden).
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    vals = {}
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if "=" in line:
                k, v = line.split("=", 1)
                vals[k.strip()] = v.strip()
            else:
                rows.append([float(t) for t in line.split()])
    return vals, rows


def _bf16_bits(x):
    """RNE of fp32 to bf16 bit patterns (input generation for the tests)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return r


# ------------------------------------------------------------------------------------------------
# rotation
# ------------------------------------------------------------------------------------------------

@pytest.mark.parametrize("b", [1, 2, 4, 8, 16, 32, 64, 128])
def test_fwht_matches_sylvester_closed_form(b):
    """FWHT of each unit vector e_k is column k of H_b times fl32(1/sqrt(b)), exactly
    (butterflies of 0 and +-1 are exact); H_b from scipy.linalg.hadamard (Sylvester)."""
    H = scipy.linalg.hadamard(b).astype(np.float64)
    cb = np.float32(1.0 / np.sqrt(b))
    assert oracle.rotation_scale(b) == cb
    for k in range(b):
        e = np.zeros(b, dtype=np.float32)
        e[k] = 1
        y = oracle.fwht_f32(e, b)
        assert np.array_equal(y, (H[:, k] * cb).astype(np.float32))


def test_sylvester_golden_matrix():
    _, rows = _golden("hadamard_sylvester_8.txt")
    H8 = np.array(rows)
    cb = np.float32(1.0 / np.sqrt(8))
    cols = np.stack([oracle.fwht_f32(np.eye(8, dtype=np.float32)[k], 8) for k in range(8)], axis=1)
    assert np.array_equal(cols, (H8 * cb).astype(np.float32))


def test_fwht_stage_order_worked_example():
    vals, _ = _golden("fwht_stage_order_b4.txt")
    x = np.array([int(h, 16) for h in vals["x_hex"].split()], dtype=np.uint32).view(np.float32)
    want = np.array([int(h, 16) for h in vals["y_hex"].split()], dtype=np.uint32)
    got = oracle.fwht_f32(x, int(vals["b"])).view(np.uint32)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("b", [2, 8, 32, 128])
def test_rotation_orthonormal_and_block_diagonal(b):
    """H_bd H_bd^T = I: rotating the identity (n = 2b, two blocks) gives a matrix whose Gram matrix
    is the identity within fp32 rounding of 1/sqrt(b), and whose off-block entries are zero."""
    n = 2 * b
    M = np.stack([oracle.fwht_f32(np.eye(n, dtype=np.float32)[k], b) for k in range(n)]).astype(np.float64)
    G = M @ M.T
    assert np.abs(G - np.eye(n)).max() <= 4 * 2.0 ** -23
    assert np.all(M[:b, b:] == 0) and np.all(M[b:, :b] == 0)


@pytest.mark.parametrize("b", [4, 32, 128])
def test_rotation_involution_and_dot_product(b):
    rng = np.random.default_rng(b)
    x = rng.standard_normal((16, 128)).astype(np.float32)
    y = oracle.fwht_f32(x, b)
    xx = oracle.fwht_f32(y, b)
    nrm = np.linalg.norm(x.astype(np.float64), axis=1, keepdims=True)
    bound = 2 * np.log2(b) * 2.0 ** -23 * nrm + 1e-12
    assert np.all(np.abs(xx - x) <= bound)
    # rotation preserves dot products: (q H).(k H) = q.k
    q = rng.standard_normal((16, 128)).astype(np.float32)
    qy = oracle.fwht_f32(q, b).astype(np.float64)
    dots_rot = (qy * y.astype(np.float64)).sum(1)
    dots = (q.astype(np.float64) * x.astype(np.float64)).sum(1)
    scale = np.linalg.norm(q, axis=1) * nrm[:, 0]
    assert np.all(np.abs(dots_rot - dots) <= 4 * np.log2(b) * 2.0 ** -23 * scale)


def test_rotate_bf16_widens_exactly():
    rng = np.random.default_rng(0)
    bits = _bf16_bits(rng.standard_normal(64).astype(np.float32))
    y = oracle.rotate_bf16(bits, 1)
    assert np.array_equal(y.view(np.uint32), bits.astype(np.uint32) << 16)


# ------------------------------------------------------------------------------------------------
# fp16 directed rounding: exhaustive enumeration of binary16
# ------------------------------------------------------------------------------------------------

def _all_finite_fp16():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = b.view(np.float16)
    m = np.isfinite(v)
    vals = v[m].astype(np.float64)
    bits = b[m]
    order = np.lexsort((bits, vals))
    return vals[order], bits[order]


def test_fp16_value_matches_ieee_definition():
    vals, bits = _all_finite_fp16()
    for i in range(0, len(bits), 97):
        assert oracle.fp16_value(int(bits[i])) == vals[i]


def test_fp16_directed_rounding_brute_force():
    vals, bits = _all_finite_fp16()
    rng = np.random.default_rng(1)
    xs = np.concatenate([
        rng.standard_normal(3000) * 10.0 ** rng.integers(-8, 5, 3000),
        vals[rng.integers(0, len(vals), 500)],                       # exactly representable
        (vals[:-1] + vals[1:])[rng.integers(0, len(vals) - 1, 500)] / 2,  # midpoints
        [0.0, -0.0, 1e-9, -1e-9, 65504.0, -65504.0, 6.1e-5, -6.1e-5, 2.0 ** -24, -(2.0 ** -24)],
    ]).astype(np.float32)
    xs = xs[np.abs(xs) <= 65504]
    for x in xs:
        x64 = float(x)
        # largest fp16 <= x; smallest fp16 >= x; zeros canonical +0
        i = np.searchsorted(vals, x64, side="right") - 1
        down = vals[i]
        j = np.searchsorted(vals, x64, side="left")
        up = vals[j]
        d = oracle.fp16_round_down(x)
        u = oracle.fp16_round_up(x)
        assert oracle.fp16_value(d) == down, (x, d, down)
        assert oracle.fp16_value(u) == up, (x, u, up)
        if down == 0:
            assert d == 0
        if up == 0:
            assert u == 0


# ------------------------------------------------------------------------------------------------
# quantizer
# ------------------------------------------------------------------------------------------------

def _dequant(codes, s_bits, z_bits):
    return oracle.fp16_value(s_bits) * codes.astype(np.float64) + oracle.fp16_value(z_bits)


def test_quantizer_worked_example():
    vals, _ = _golden("quantizer_worked_example.txt")
    y = np.array([float(t) for t in vals["y"].split()], dtype=np.float32)
    codes, s, z = oracle.quantize(y, int(vals["Q"]))
    assert s == int(vals["s_bits"], 16) and z == int(vals["z_bits"], 16)
    assert codes.tolist() == [int(t) for t in vals["codes"].split()]
    assert _dequant(codes, s, z).tolist() == [float(t) for t in vals["dequant"].split()]


@pytest.mark.parametrize("Q", [15, 255])
def test_quantizer_invariants(Q):
    rng = np.random.default_rng(Q)
    for trial in range(300):
        n = int(rng.choice([4, 32, 64, 128]))
        y = (rng.standard_normal(n) * 10.0 ** rng.uniform(-3, 3)).astype(np.float32)
        if trial % 3 == 0:
            y[rng.integers(0, n, 2)] *= 20  # outliers
        codes, s, z = oracle.quantize(y, Q)
        sf, zf = oracle.fp16_value(s), oracle.fp16_value(z)
        mn, mx = float(y.min()), float(y.max())
        assert zf <= mn
        assert mx <= zf + Q * sf * (1 + 2.0 ** -22)
        assert codes.max() <= Q
        err = np.abs(_dequant(codes, s, z) - y.astype(np.float64))
        assert np.all(err <= sf / 2 * (1 + 2.0 ** -20) + 1e-300), (trial, err.max(), sf)


@pytest.mark.parametrize("Q", [15, 255])
def test_quantizer_brute_force_nearest_code(Q):
    """For small groups the code is the nearest grid point z + c*s (ties to even), except where the
    binary32 evaluation of (y - z)/s lies within 2^-20 of a half-integer."""
    rng = np.random.default_rng(7 + Q)
    for _ in range(400):
        y = (rng.standard_normal(4) * 3).astype(np.float32)
        codes, s, z = oracle.quantize(y, Q)
        sf, zf = Fraction(oracle.fp16_value(s)), Fraction(oracle.fp16_value(z))
        for yi, ci in zip(y, codes):
            yq = Fraction(float(yi))
            dist = [abs(zf + c * sf - yq) for c in range(Q + 1)]
            best = min(dist)
            cands = [c for c in range(Q + 1) if dist[c] == best]
            expect = cands[0] if len(cands) == 1 else [c for c in cands if c % 2 == 0][0]
            if ci != expect:
                u = (yq - zf) / sf
                assert abs(u - (int(u) + Fraction(1, 2))) <= Fraction(1, 2 ** 20) * max(1, u), (yi, ci, expect)


def test_quantizer_special_cases():
    # zero group: s = z = +0, codes 0
    c, s, z = oracle.quantize(np.zeros(8, dtype=np.float32), 15)
    assert s == 0 and z == 0 and not c.any()
    c, s, z = oracle.quantize(-np.zeros(8, dtype=np.float32), 15)
    assert s == 0 and z == 0 and not c.any()
    # constant group on the fp16 grid: s = 0, reproduces exactly through z
    c, s, z = oracle.quantize(np.full(8, 1.5, dtype=np.float32), 15)
    assert s == 0 and oracle.fp16_value(z) == 1.5 and not c.any()
    # values on the grid reproduce exactly: z = -1, s = 0.25, codes 0..15
    y = (-1 + 0.25 * np.arange(16)).astype(np.float32)
    c, s, z = oracle.quantize(y, 15)
    assert oracle.fp16_value(z) == -1 and oracle.fp16_value(s) == 0.25
    assert c.tolist() == list(range(16))
    # ties go to even: z = 0, s = 1 (y spans [0, 15]); 2.5 -> 2, 3.5 -> 4, 12.5 -> 12
    y = np.array([0, 15, 2.5, 3.5, 12.5, 13.5], dtype=np.float32)
    c, s, z = oracle.quantize(y, 15)
    assert oracle.fp16_value(s) == 1 and z == 0
    assert c.tolist() == [0, 15, 2, 4, 12, 14]
    # outside the fp16 range is a precondition violation
    with pytest.raises(ValueError):
        oracle.quantize(np.array([0, 70000], dtype=np.float32), 15)
    with pytest.raises(ValueError):
        oracle.quantize(np.array([0, np.inf], dtype=np.float32), 15)


def test_pack_int4_nibble_order():
    assert oracle.pack_int4(np.array([1, 2, 3, 4, 15, 0], dtype=np.uint8)).tolist() == [0x21, 0x43, 0x0F]


def test_dequant_exact_in_binary64():
    """s*code + z is held exactly in binary64: compare with rational arithmetic."""
    rng = np.random.default_rng(3)
    for _ in range(200):
        s = int(rng.integers(1, 0x7BFF))
        z = int(rng.integers(0, 0xFBFF))
        if (z & 0x7C00) == 0x7C00:
            continue
        c = int(rng.integers(0, 256))
        exact = Fraction(oracle.fp16_value(s)) * c + Fraction(oracle.fp16_value(z))
        assert Fraction(oracle.fp16_value(s) * c + oracle.fp16_value(z)) == exact


# ------------------------------------------------------------------------------------------------
# protected set
# ------------------------------------------------------------------------------------------------

@pytest.mark.parametrize("S,R", [(4, 128), (4, 32), (0, 16), (3, 0), (0, 0)])
def test_protected_set_size_and_slots(S, R):
    for L in list(range(0, 300)) + [1000, 4097]:
        prot = [t for t in range(L) if oracle.is_protected(t, L, S, R)]
        assert len(prot) == min(L, S + R)
        # sinks are the first min(S, L); the rest are the last positions
        assert prot[: min(S, L)] == list(range(min(S, L)))
        rest = prot[min(S, L):]
        assert rest == list(range(L - len(rest), L))
        # slots are distinct within Prot(L) and below S + R
        slots = [oracle.int8_slot(t, S, R) for t in prot]
        assert len(set(slots)) == len(slots) and all(0 <= u < S + R for u in slots)
