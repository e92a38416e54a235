"""Pins of the CPU oracle against things other than itself.

Each test ties one oracle function to a closed form, a textbook or library
routine, brute force on a tiny input, an invariant the VecInfer pages state, or
a fixture under tests/golden/ -- chosen so that a dropped term, a wrong sign or
index, or a transposed operand in the oracle fails at least one of them.
"""
import math
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg
import scipy.special

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
D = 128


def _golden_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


# ----------------------------------------------------------------- Hadamard / FWHT

def test_inv_sqrt_constant_is_correctly_rounded():
    """The scale that normalizes H is the fp64 nearest to 2^-3.5 (closed form)."""
    H = oracle.hadamard()
    c = float(H[0, 0])
    getcontext().prec = 80
    exact = Decimal(1) / Decimal(128).sqrt()
    err = abs(Decimal(Fraction(c).numerator) / Decimal(Fraction(c).denominator) - exact)
    for nb in (np.nextafter(c, 0.0), np.nextafter(c, 1.0)):
        e2 = abs(Decimal(Fraction(float(nb)).numerator) / Decimal(Fraction(float(nb)).denominator) - exact)
        assert err < e2


def test_hadamard_is_normalized_sylvester():
    """Matches scipy's Sylvester construction exactly up to the scale; symmetric; H H = I."""
    H = oracle.hadamard()
    c = float(H[0, 0])
    assert np.array_equal(H, scipy.linalg.hadamard(D).astype(np.float64) * c)
    assert np.array_equal(H, H.T)
    assert np.abs(H @ H - np.eye(D)).max() < 1e-15


def test_hadamard_golden_block_and_recursion():
    """Top-left 8x8 block is the textbook H_8; blocks obey H_2n = [[H, H], [H, -H]]."""
    H = oracle.hadamard()
    c = float(H[0, 0])
    H8 = np.array([[int(x) for x in r] for r in _golden_rows("hadamard8_sylvester.txt")], dtype=np.float64)
    assert np.array_equal(H[:8, :8], H8 * c)
    n = D // 2
    assert np.array_equal(H[:n, :n], H[:n, n:])
    assert np.array_equal(H[:n, :n], H[n:, :n])
    assert np.array_equal(H[:n, :n], -H[n:, n:])


@pytest.mark.parametrize("scale_outliers", [False, True])
def test_fwht_equals_matrix_product(scale_outliers):
    rng = np.random.default_rng(1)
    H = scipy.linalg.hadamard(D).astype(np.float64) / math.sqrt(D)
    for _ in range(50):
        x = rng.standard_normal(D)
        if scale_outliers:
            x[rng.permutation(D)[:4]] *= 15.0
        y = oracle.fwht(x)
        assert np.abs(y - H @ x).max() <= 1e-14 * np.linalg.norm(x)


def test_fwht_closed_forms():
    """FWHT(e_0) is the constant vector 1/sqrt(128) exactly; FWHT(e_i) is column i of H; H^2 = I."""
    H = oracle.hadamard()
    e0 = np.zeros(D)
    e0[0] = 1.0
    assert np.array_equal(oracle.fwht(e0), np.full(D, H[0, 0]))
    for i in (1, 5, 64, 127):
        ei = np.zeros(D)
        ei[i] = 1.0
        assert np.array_equal(oracle.fwht(ei), H[:, i])
    x = np.random.default_rng(2).standard_normal(D)
    assert np.abs(oracle.fwht(oracle.fwht(x)) - x).max() < 1e-14


# ---------------------------------------------------------------------- smoothing

def test_smooth_scales_closed_form():
    """s_c = sqrt(max_t |k[t][c]|), fp32 of the fp64 root, with planted per-channel maxima."""
    rng = np.random.default_rng(3)
    n = 257
    k = rng.uniform(-1.0, 1.0, size=(n, D))
    m = rng.uniform(1.5, 300.0, size=D)
    rows = rng.integers(0, n, size=D)
    signs = rng.choice([-1.0, 1.0], size=D)
    for c in range(D):
        k[rows[c], c] = signs[c] * m[c]
    s = oracle.smooth_scales(k)
    assert s.dtype == np.float32
    assert np.array_equal(s, np.sqrt(m).astype(np.float32))


def test_smooth_scales_flag_outlier_channels():
    case = synth.make_cpu_case(synth.WORKLOADS["tiny_g4_t2048"], 11, seq_len=64)
    s = oracle.smooth_scales(case.k_cal[0])
    out = case.channels[0]
    rest = np.setdiff1d(np.arange(D), out)
    assert s[out].min() > 2.0 * s[rest].max()


# ---------------------------------------------------------------- score invariance

@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_transform_leaves_scores_unchanged(dtype):
    """VecInfer summary card, Summary: the inverse operations on the query keep
    attention scores unchanged, i.e. q'.k' = q.k."""
    wl = synth.WORKLOADS["tiny_g4_t2048"]
    case = synth.make_cpu_case(dataclass_replace(wl, dtype=dtype), 5, seq_len=40)
    s = oracle.smooth_scales(case.k_cal[0])
    for t in range(40):
        k = case.k[0, 0, t].astype(np.float64)
        for g in range(4):
            q = case.q[0, g].astype(np.float64)
            lhs = float(oracle.transform_query(q, s) @ oracle.transform_key(k, s))
            rhs = float(q @ k)
            assert abs(lhs - rhs) <= 1e-12 * np.linalg.norm(q) * np.linalg.norm(k)


def test_transform_key_is_divide_then_rotate():
    """x' = H (k / s): checked with scipy's Hadamard and a numpy division."""
    rng = np.random.default_rng(6)
    k = rng.standard_normal(D)
    s = rng.uniform(0.5, 4.0, D).astype(np.float32)
    H = scipy.linalg.hadamard(D) / math.sqrt(D)
    assert np.abs(oracle.transform_key(k, s) - H @ (k / s.astype(np.float64))).max() < 1e-14
    assert np.abs(oracle.transform_query(k, s) - H @ (k * s.astype(np.float64))).max() < 1e-13


def dataclass_replace(wl, **kw):
    import dataclasses
    return dataclasses.replace(wl, **kw)


# -------------------------------------------------------------------------- fp16

def test_half_to_double_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.half_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_double_to_half_round_to_nearest_even():
    rng = np.random.default_rng(7)
    vals = list(rng.standard_normal(3000) * np.exp(rng.uniform(-20, 12, 3000)))
    finite = np.arange(0, 0x7c00, 7, dtype=np.uint16).view(np.float16).astype(np.float64)
    nxt = (np.arange(0, 0x7c00, 7, dtype=np.uint16) + 1).view(np.float16).astype(np.float64)
    vals += list((finite + nxt) / 2.0)          # exact midpoints: ties to even
    vals += list(np.nextafter((finite + nxt) / 2.0, np.inf))
    vals += [0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e6, -1e6, 2.0 ** -24, 2.0 ** -25, 2.0 ** -26,
             3 * 2.0 ** -26, 6.1e-5]
    for v in vals:
        for x in (v, -v):
            with np.errstate(over="ignore"):
                ref = np.array(x, dtype=np.float64).astype(np.float16).view(np.uint16)
            assert oracle.double_to_half(x) == int(ref), x


# ---------------------------------------------------------------- nearest centroid

@pytest.mark.parametrize("dsub", [2, 4, 8])
@pytest.mark.parametrize("E", [4, 7, 16])
def test_nearest_brute_force(dsub, E):
    rng = np.random.default_rng(E * 10 + dsub)
    for _ in range(200):
        book = rng.standard_normal((E, dsub))
        x = rng.standard_normal(dsub) * 1.5
        ref = int(np.argmin(((x[None, :] - book) ** 2).sum(axis=1)))
        assert oracle.nearest(x, book) == ref


@pytest.mark.parametrize("dsub", [2, 4, 8])
def test_nearest_exact_ties_take_lowest_index(dsub):
    """Small integers make every distance exact, so ties are frequent and
    numpy's argmin (first occurrence) is the lowest-index rule."""
    rng = np.random.default_rng(dsub)
    hits = 0
    for _ in range(2000):
        book = rng.integers(-2, 3, size=(12, dsub)).astype(np.float64)
        x = rng.integers(-2, 3, size=dsub).astype(np.float64)
        d = ((x[None, :] - book) ** 2).sum(axis=1)
        ref = int(np.argmin(d))
        hits += int((d == d[ref]).sum() > 1)
        assert oracle.nearest(x, book) == ref
    assert hits > 100


def test_nearest_duplicate_centroid_goes_to_first():
    rng = np.random.default_rng(9)
    book = rng.standard_normal((16, 4))
    book[11] = book[3]
    assert oracle.nearest(book[3] + 1e-3, book) == 3


@pytest.mark.parametrize("fmt", [0, 1, 3, 4])
def test_quantize_recovers_codes_of_keys_built_from_centroids(fmt):
    """Keys built as k = s * H(concat C_K[codes]) (scipy's H, numpy arithmetic)
    quantize back to the generating codes; values built from C_V likewise."""
    E, dsub = oracle.FORMATS[fmt]
    J = D // dsub
    rng = np.random.default_rng(20 + fmt)
    kbook = synth.random_fp16_book(1 + fmt, (E, dsub))
    vbook = synth.random_fp16_book(2 + fmt, (E, dsub))
    kc = synth.random_codes(3, (50, J), E)
    vc = synth.random_codes(4, (50, J), E)
    s = rng.uniform(0.7, 6.0, D).astype(np.float32)
    H = scipy.linalg.hadamard(D) / math.sqrt(D)
    kf = kbook.view(np.float16).astype(np.float64)
    vf = vbook.view(np.float16).astype(np.float64)
    xk = kf[kc].reshape(50, D)
    k = (xk @ H) * s.astype(np.float64)        # H symmetric: H^-1 = H
    v = vf[vc].reshape(50, D)
    gk, gv = oracle.quantize(fmt, k, v, s, kbook, vbook)
    # Duplicate fp16 entries would legitimately map to the lower index.
    kmap = np.array([np.flatnonzero((kf == kf[e]).all(axis=1))[0] for e in range(E)])
    vmap = np.array([np.flatnonzero((vf == vf[e]).all(axis=1))[0] for e in range(E)])
    assert np.array_equal(gk, kmap[kc])
    assert np.array_equal(gv, vmap[vc])


def test_quantize_matches_numpy_brute_force_on_real_keys():
    wl = synth.WORKLOADS["tiny_g4_t2048"]
    case = synth.make_cpu_case(wl, 12, seq_len=64, n_cal=256)
    s = oracle.smooth_scales(case.k_cal[0])
    kbook = synth.random_fp16_book(5, (256, 4))
    vbook = synth.random_fp16_book(6, (256, 4))
    kc, vc = oracle.quantize(0, case.k[0, 0], case.v[0, 0], s, kbook, vbook)
    H = scipy.linalg.hadamard(D) / math.sqrt(D)
    xk = (case.k[0, 0].astype(np.float64) / s.astype(np.float64)) @ H
    kf = kbook.view(np.float16).astype(np.float64)
    vf = vbook.view(np.float16).astype(np.float64)
    dk = ((xk.reshape(-1, 1, 4) - kf[None]) ** 2).sum(-1)
    dv = ((case.v[0, 0].astype(np.float64).reshape(-1, 1, 4) - vf[None]) ** 2).sum(-1)
    assert np.array_equal(kc.ravel(), dk.argmin(1))
    assert np.array_equal(vc.ravel(), dv.argmin(1))


# ---------------------------------------------------------------------- attention

def _numpy_attention(fmt, q, s, kbook, vbook, kc, vc, sm_scale):
    """Dequantize with numpy, rotate q with scipy's H, softmax with scipy."""
    E, dsub = oracle.FORMATS[fmt]
    B, Hq, _ = q.shape
    _, Hkv, T, J = kc.shape
    G = Hq // Hkv
    H = scipy.linalg.hadamard(D) / math.sqrt(D)
    out = np.zeros((B, Hq, D))
    for b in range(B):
        for g in range(Hq):
            h = g // G
            kf = kbook[h].view(np.float16).astype(np.float64)
            vf = vbook[h].view(np.float16).astype(np.float64)
            K = kf[kc[b, h]].reshape(T, D)
            V = vf[vc[b, h]].reshape(T, D)
            qp = H @ (q[b, g].astype(np.float64) * s[h].astype(np.float64))
            p = scipy.special.softmax(sm_scale * (K @ qp))
            out[b, g] = p @ V
    return out


@pytest.mark.parametrize("fmt,Hq,Hkv,T", [(0, 4, 1, 300), (0, 8, 2, 129), (1, 5, 1, 77), (1, 4, 2, 1),
                                          (3, 5, 1, 131), (3, 8, 2, 64), (4, 4, 1, 100), (4, 8, 2, 65)])
def test_attention_matches_numpy_scipy(fmt, Hq, Hkv, T):
    E, dsub = oracle.FORMATS[fmt]
    J = D // dsub
    rng = np.random.default_rng(T)
    B = 2
    q = rng.standard_normal((B, Hq, D))
    s = rng.uniform(0.5, 5.0, (Hkv, D)).astype(np.float32)
    kbook = synth.random_fp16_book(7, (Hkv, E, dsub))
    vbook = synth.random_fp16_book(8, (Hkv, E, dsub))
    kc = synth.random_codes(9, (B, Hkv, T, J), E)
    vc = synth.random_codes(10, (B, Hkv, T, J), E)
    sm = 1.0 / math.sqrt(D)
    got = oracle.attention(fmt, q, s, kbook, vbook, kc, vc, sm)
    ref = _numpy_attention(fmt, q, s, kbook, vbook, kc, vc, sm)
    assert np.abs(got - ref).max() <= 1e-12 * np.abs(ref).max()


def test_attention_single_token_returns_its_value():
    """T = 1: softmax weight 1, so o = the dequantized value of token 0."""
    rng = np.random.default_rng(13)
    q = rng.standard_normal((1, 4, D)) * 10
    s = rng.uniform(0.5, 5.0, (1, D)).astype(np.float32)
    kbook = synth.random_fp16_book(1, (1, 256, 4))
    vbook = synth.random_fp16_book(2, (1, 256, 4))
    kc = synth.random_codes(3, (1, 1, 1, 32), 256)
    vc = synth.random_codes(4, (1, 1, 1, 32), 256)
    out = oracle.attention(0, q, s, kbook, vbook, kc, vc)
    v0 = vbook[0].view(np.float16).astype(np.float64)[vc[0, 0, 0]].reshape(D)
    for g in range(4):
        assert np.array_equal(out[0, g], v0)


def test_attention_equal_scores_give_mean_value():
    """All keys share one code: uniform softmax, o = mean of the dequantized values."""
    rng = np.random.default_rng(14)
    T = 97
    q = rng.standard_normal((1, 2, D))
    s = np.ones((1, D), dtype=np.float32)
    kbook = synth.random_fp16_book(1, (1, 256, 4))
    vbook = synth.random_fp16_book(2, (1, 256, 4))
    kc = np.broadcast_to(synth.random_codes(3, (1, 1, 1, 32), 256), (1, 1, T, 32)).copy()
    vc = synth.random_codes(4, (1, 1, T, 32), 256)
    out = oracle.attention(0, q, s, kbook, vbook, kc, vc)
    V = vbook[0].view(np.float16).astype(np.float64)[vc[0, 0]].reshape(T, D)
    for g in range(2):
        assert np.abs(out[0, g] - V.mean(axis=0)).max() < 1e-14


def test_fp_attention_matches_scipy():
    rng = np.random.default_rng(15)
    B, Hq, Hkv, T = 2, 6, 2, 33
    q = rng.standard_normal((B, Hq, D))
    k = rng.standard_normal((B, Hkv, T, D))
    v = rng.standard_normal((B, Hkv, T, D))
    got = oracle.attention_fp(q, k, v)
    for b in range(B):
        for g in range(Hq):
            h = g // (Hq // Hkv)
            p = scipy.special.softmax(k[b, h] @ q[b, g] / math.sqrt(D))
            assert np.abs(got[b, g] - p @ v[b, h]).max() < 1e-13


@pytest.mark.parametrize("fmt", [0, 1, 3, 4])
def test_vq_attention_equals_full_precision_on_exact_cache(fmt):
    """Keys and values built exactly from centroids: VQ attention over the codes
    equals full-precision attention over the raw cache (the transform changes
    no score), to fp64 rounding."""
    E, dsub = oracle.FORMATS[fmt]
    J = D // dsub
    rng = np.random.default_rng(16 + fmt)
    B, Hq, Hkv, T = 1, 8, 2, 65
    s = rng.uniform(0.7, 6.0, (Hkv, D)).astype(np.float32)
    kbook = synth.random_fp16_book(11, (Hkv, E, dsub))
    vbook = synth.random_fp16_book(12, (Hkv, E, dsub))
    kc = synth.random_codes(13, (B, Hkv, T, J), E)
    vc = synth.random_codes(14, (B, Hkv, T, J), E)
    H = scipy.linalg.hadamard(D) / math.sqrt(D)
    k = np.zeros((B, Hkv, T, D))
    v = np.zeros((B, Hkv, T, D))
    for h in range(Hkv):
        kf = kbook[h].view(np.float16).astype(np.float64)
        vf = vbook[h].view(np.float16).astype(np.float64)
        k[0, h] = (kf[kc[0, h]].reshape(T, D) @ H) * s[h].astype(np.float64)
        v[0, h] = vf[vc[0, h]].reshape(T, D)
    q = rng.standard_normal((B, Hq, D))
    vq = oracle.attention(fmt, q, s, kbook, vbook, kc, vc)
    fp = oracle.attention_fp(q, k, v)
    assert np.abs(vq - fp).max() < 1e-12


@pytest.mark.parametrize("fmt", [0, 1, 3, 4])
def test_value_transform_quantize_recovers_codes(fmt):
    """Value-transform variant: values built as v = sv * H(concat C_V[codes])
    (scipy's H) quantize back to the generating codes when the quantizer is
    given sv; without sv they do not (the values are no longer the centroids)."""
    E, dsub = oracle.FORMATS[fmt]
    J = D // dsub
    rng = np.random.default_rng(40 + fmt)
    kbook = synth.random_fp16_book(41 + fmt, (E, dsub))
    vbook = synth.random_fp16_book(43 + fmt, (E, dsub))
    vc = synth.random_codes(45, (40, J), E)
    s = rng.uniform(0.7, 6.0, D).astype(np.float32)
    sv = rng.uniform(0.5, 3.0, D).astype(np.float32)
    H = scipy.linalg.hadamard(D) / math.sqrt(D)
    vf = vbook.view(np.float16).astype(np.float64)
    v = (vf[vc].reshape(40, D) @ H) * sv.astype(np.float64)
    k = rng.standard_normal((40, D))
    _, gv = oracle.quantize(fmt, k, v, s, kbook, vbook, sv=sv)
    vmap = np.array([np.flatnonzero((vf == vf[e]).all(axis=1))[0] for e in range(E)])
    assert np.array_equal(gv, vmap[vc])
    _, raw = oracle.quantize(fmt, k, v, s, kbook, vbook)
    assert not np.array_equal(raw, gv)


def test_value_output_transform_undoes_the_value_transform():
    """sv * H(H(v / sv)) = v: the output map inverts the value transform."""
    rng = np.random.default_rng(47)
    sv = rng.uniform(0.5, 3.0, D).astype(np.float32)
    for _ in range(20):
        v = rng.standard_normal(D) * rng.uniform(0.1, 30.0)
        back = oracle.value_output_transform(oracle.transform_key(v, sv), sv)
        assert np.abs(back - v).max() <= 1e-13 * np.abs(v).max()


@pytest.mark.parametrize("fmt", [0, 1, 3, 4])
def test_vq_attention_with_value_transform_equals_full_precision(fmt):
    """Keys and values built exactly from centroids in the transformed spaces
    (k = s * H k', v = sv * H v'): VQ attention with the value transform equals
    full-precision attention over the raw cache, to fp64 rounding."""
    E, dsub = oracle.FORMATS[fmt]
    J = D // dsub
    rng = np.random.default_rng(48 + fmt)
    B, Hq, Hkv, T = 2, 6, 2, 40
    s = rng.uniform(0.7, 6.0, (Hkv, D)).astype(np.float32)
    sv = rng.uniform(0.5, 3.0, (Hkv, D)).astype(np.float32)
    kbook = synth.random_fp16_book(50, (Hkv, E, dsub))
    vbook = synth.random_fp16_book(51, (Hkv, E, dsub))
    kc = synth.random_codes(52, (B, Hkv, T, J), E)
    vc = synth.random_codes(53, (B, Hkv, T, J), E)
    H = scipy.linalg.hadamard(D) / math.sqrt(D)
    k = np.zeros((B, Hkv, T, D))
    v = np.zeros((B, Hkv, T, D))
    for b in range(B):
        for h in range(Hkv):
            kf = kbook[h].view(np.float16).astype(np.float64)
            vf = vbook[h].view(np.float16).astype(np.float64)
            k[b, h] = (kf[kc[b, h]].reshape(T, D) @ H) * s[h].astype(np.float64)
            v[b, h] = (vf[vc[b, h]].reshape(T, D) @ H) * sv[h].astype(np.float64)
    q = rng.standard_normal((B, Hq, D))
    got = oracle.attention(fmt, q, s, kbook, vbook, kc, vc, sv=sv)
    fp = oracle.attention_fp(q, k, v)
    assert np.abs(got - fp).max() < 1e-12
    plain = oracle.attention(fmt, q, s, kbook, vbook, kc, vc)
    assert np.abs(plain - fp).max() > 1e-3          # without the output map it is wrong


# ------------------------------------------------------------------------ packing

def test_codebook_formats_golden():
    for fmt, E, dsub, bits in _golden_rows("codebook_formats.txt"):
        e, d = oracle.FORMATS[int(fmt)]
        assert (e, d) == (int(E), int(dsub))
        assert math.log2(e) / d == float(bits)
        assert oracle.code_bytes_per_token(int(fmt)) * 8 == int(math.log2(e)) * (D // d)


def test_pack12_golden_examples():
    for c0, c1, b0, b1, b2 in _golden_rows("pack12_examples.txt"):
        codes = np.zeros((1, 16), dtype=np.uint16)
        codes[0, 0], codes[0, 1] = int(c0, 16), int(c1, 16)
        kb = oracle.pack_k(1, codes, 64)
        assert list(kb[:3]) == [int(b0, 16), int(b1, 16), int(b2, 16)]
        # Values pair sub-vectors j and j + 8 of one token: (5, 13) of token 0
        # is stream 8 * 2 + 0 + 1 = 17, bytes 17 * 48 ..
        vcodes = np.zeros((1, 16), dtype=np.uint16)
        vcodes[0, 5], vcodes[0, 13] = int(c0, 16), int(c1, 16)
        vb = oracle.pack_v(1, vcodes, 64)
        assert list(vb[17 * 48:17 * 48 + 3]) == [int(b0, 16), int(b1, 16), int(b2, 16)]


def test_pack12_round_trip_exhaustive():
    """All 2^24 (c0, c1) pairs survive pack/unpack in both layouts."""
    pairs = np.arange(1 << 24, dtype=np.uint32)
    c = np.stack([(pairs & 0xFFF), (pairs >> 12)], axis=1).astype(np.uint16).reshape(-1, 16)
    T = c.shape[0]
    kb = oracle.pack_k(1, c, T)
    assert kb.size == T * 24
    assert np.array_equal(oracle.unpack_k(1, kb, T), c)
    vb = oracle.pack_v(1, c, T)
    assert np.array_equal(oracle.unpack_v(1, vb, T), c)


def test_pack_1p5bit_value_positions():
    """Hand-computed positions of the 1.5-bit value layout: token t (u = t % 64),
    sub-vector j -> block t // 64 of 1536 bytes, stream 8*((j%8)//2) + 2*(u%4) + j%2,
    bytes 3*(u//4)..+2, element j // 8 of the pair."""
    T = 130
    c = synth.random_codes(2, (T, 16), 4096)
    vb = oracle.pack_v(1, c, 192)

    def pair(off):
        b0, b1, b2 = (int(x) for x in vb[off:off + 3])
        return b0 | ((b1 & 0xF) << 8), (b1 >> 4) | (b2 << 4)
    assert pair(0) == (c[0, 0], c[0, 8])                        # stream 0
    assert pair(48 * 1 + 0) == (c[0, 1], c[0, 9])               # j = 1 -> stream 1
    assert pair(48 * 3 + 0) == (c[1, 1], c[1, 9])               # t = 1, j = 1 -> 2 + 1
    assert pair(48 * 28 + 3 * 15) == (c[62, 6], c[62, 14])      # u = 62: 8*3 + 2*2 + 0, byte 45
    assert pair(1536 + 48 * 31 + 3 * 0) == (c[67, 7], c[67, 15])  # block 1, u = 3: 24 + 6 + 1
    assert pair(2 * 1536 + 48 * 8 + 0) == (c[128, 2], c[128, 10])  # block 2, u = 0: 8*1 + 0 + 0
    assert np.array_equal(oracle.unpack_v(1, vb, T), c)


def test_pack_2bit_positions():
    """Hand-computed byte positions of the 2-bit layouts."""
    T = 96
    c = synth.random_codes(1, (T, 32), 256)
    kb = oracle.pack_k(0, c, 128)
    vb = oracle.pack_v(0, c, 128)
    for t, j in [(0, 0), (0, 31), (1, 0), (33, 7), (95, 31)]:
        assert kb[t * 32 + j] == c[t, j]
    # Values: 64-token blocks; (t, j) -> chunk 16*((j%16)//4) + 4*(t%4) + j%4,
    # byte 2*((t%64)//4) + j//16 of that 32-byte chunk.
    assert vb[0] == c[0, 0]
    assert vb[32 * 23 + 0] == c[1, 7]            # chunk 16 + 4 + 3
    assert vb[32 * 23 + 16] == c[33, 7]          # same chunk, byte 2 * 8
    assert vb[2048 + 32 * 63 + 15] == c[95, 31]  # block 1, u = 31: chunk 48 + 12 + 3, byte 14 + 1
    assert vb[2048 + 32 * 24 + 1] == c[66, 20]   # block 1, u = 2: chunk 16 + 8 + 0, byte 0 + 1
    assert vb[32 * 3 + 1] == c[0, 19]            # chunk 3, byte 1
    assert np.array_equal(oracle.unpack_v(0, vb, T), c)
    assert np.array_equal(oracle.unpack_k(0, kb, T), c)


def test_pack_3bit_positions():
    """Hand-computed positions of the 3-bit layouts (2^12 x 4, 12-bit codes):
    keys token-major, 48 bytes per token, pairs (2i, 2i+1) in bytes 3i..3i+2;
    values in 64-token blocks of 3072 bytes, (t, j) -> chunk
    16*((j%16)//4) + 4*(u%4) + j%4 (u = t % 64), bytes 3*(u//4)..+2 of that
    48-byte chunk, element j // 16 of the pair (j%16, j%16 + 16)."""
    T = 130
    c = synth.random_codes(5, (T, 32), 4096)
    kb = oracle.pack_k(2, c, 192)
    vb = oracle.pack_v(2, c, 192)
    assert kb.size == vb.size == 192 * 48

    def pair(buf, off):
        b0, b1, b2 = (int(x) for x in buf[off:off + 3])
        return b0 | ((b1 & 0xF) << 8), (b1 >> 4) | (b2 << 4)
    assert pair(kb, 0) == (c[0, 0], c[0, 1])
    assert pair(kb, 48 * 7 + 3 * 15) == (c[7, 30], c[7, 31])
    assert pair(vb, 0) == (c[0, 0], c[0, 16])                       # chunk 0
    assert pair(vb, 48 * 23) == (c[1, 7], c[1, 23])                 # chunk 16 + 4 + 3
    assert pair(vb, 48 * 23 + 24) == (c[33, 7], c[33, 23])          # same chunk, u // 4 = 8
    assert pair(vb, 3072 + 48 * 63 + 21) == (c[95, 15], c[95, 31])  # block 1, u = 31: 48 + 12 + 3
    assert pair(vb, 2 * 3072 + 48 * 1 + 0) == (c[128, 1], c[128, 17])  # block 2, u = 0, j = 1: chunk 1
    assert np.array_equal(oracle.unpack_k(2, kb, T), c)
    assert np.array_equal(oracle.unpack_v(2, vb, T), c)


def test_3bit_format_is_twelve_bits_per_four_dims():
    """The third width: 4096 entries of 4 dims, so 12 bits per 4 elements
    (3 bits each, inside the pages' 1.25-4 bit range) and 32 codes, 48 bytes,
    per token; quantizing keys built from its centroids recovers their codes."""
    E, dsub = oracle.FORMATS[2]
    assert (E, dsub) == (4096, 4)
    assert math.log2(E) / dsub == 3.0 and oracle.code_bytes_per_token(2) * 8 == 12 * 32
    rng = np.random.default_rng(77)
    kbook = synth.random_fp16_book(78, (E, dsub))
    vbook = synth.random_fp16_book(79, (E, dsub))
    kc = synth.random_codes(80, (30, 32), E)
    s = rng.uniform(0.7, 6.0, D).astype(np.float32)
    H = scipy.linalg.hadamard(D) / math.sqrt(D)
    kf = kbook.view(np.float16).astype(np.float64)
    k = (kf[kc].reshape(30, D) @ H) * s.astype(np.float64)
    gk, _ = oracle.quantize(2, k, rng.standard_normal((30, D)), s, kbook, vbook)
    kmap = np.array([np.flatnonzero((kf == kf[e]).all(axis=1))[0] for e in range(E)])
    assert np.array_equal(gk, kmap[kc])


def _bits(buf, pos, width):
    """Little-endian bit field [pos, pos + width) of a byte array (Python ints)."""
    return (int.from_bytes(bytes(buf), "little") >> pos) & ((1 << width) - 1)


def test_pack10_golden_examples():
    """Hand-derived bytes of four 10-bit codes, in the key layout (sub-vectors
    4..7 of token 0: bytes 5..9) and in the value layout (sub-vectors 5 and
    13 of tokens 0 and 4, pairs 0 and 1 of stream 8*2 + 0 + 1 = 17: bytes
    17*40 .. 17*40 + 4)."""
    for row in _golden_rows("pack10_examples.txt"):
        c = [int(x, 16) for x in row[:4]]
        want = [int(x, 16) for x in row[4:]]
        codes = np.zeros((1, 16), dtype=np.uint16)
        codes[0, 4:8] = c
        kb = oracle.pack_k(3, codes, 64)
        assert list(kb[5:10]) == want and not kb[:5].any() and not kb[10:20].any()
        vcodes = np.zeros((5, 16), dtype=np.uint16)
        vcodes[0, 5], vcodes[0, 13], vcodes[4, 5], vcodes[4, 13] = c
        vb = oracle.pack_v(3, vcodes, 64)
        assert list(vb[17 * 40:17 * 40 + 5]) == want
        assert np.count_nonzero(vb) == np.count_nonzero(want)


def test_pack10_round_trip_exhaustive():
    """All 2^20 pairs of 10-bit codes survive pack/unpack in both layouts, at
    every position of a token (keys) and of a stream (values)."""
    pairs = np.arange(1 << 20, dtype=np.uint32)
    c = np.stack([(pairs & 0x3FF), (pairs >> 10)], axis=1).astype(np.uint16).reshape(-1, 16)
    T = c.shape[0]
    kb = oracle.pack_k(3, c, T)
    assert kb.size == T * 20
    assert np.array_equal(oracle.unpack_k(3, kb, T), c)
    vb = oracle.pack_v(3, c, T)
    assert np.array_equal(oracle.unpack_v(3, vb, T), c)


def test_pack_1p25bit_positions():
    """Hand-computed positions of the 1.25-bit layouts (read with Python's own
    little-endian integers): key code j of token t in bits [160 t + 10 j, +10);
    value code (t, j), u = t % 64, in block t // 64 of 1280 bytes, stream
    8*((j%8)//2) + 2*(u%4) + j%2 of 40 bytes, bits 20*(u//4) + 10*(j//8).."""
    T = 130
    c = synth.random_codes(6, (T, 16), 1024)
    kb = oracle.pack_k(3, c, 192)
    vb = oracle.pack_v(3, c, 192)
    assert kb.size == vb.size == 192 * 20
    for t, j in [(0, 0), (0, 15), (1, 3), (77, 9), (129, 15)]:
        assert _bits(kb[20 * t:20 * t + 20], 10 * j, 10) == c[t, j]
    assert _bits(vb[0:40], 0, 10) == c[0, 0]                       # stream 0, pair 0, half 0
    assert _bits(vb[0:40], 10, 10) == c[0, 8]                      # half 1: sub-vector 8
    assert _bits(vb[40 * 1:40 * 2], 0, 10) == c[0, 1]              # j = 1 -> stream 1
    assert _bits(vb[40 * 3:40 * 4], 0, 10) == c[1, 1]              # t = 1, j = 1 -> 2 + 1
    assert _bits(vb[40 * 28:40 * 29], 20 * 15, 10) == c[62, 6]     # u = 62: 8*3 + 2*2 + 0, pair 15
    assert _bits(vb[40 * 28:40 * 29], 20 * 15 + 10, 10) == c[62, 14]
    assert _bits(vb[1280 + 40 * 31:1280 + 40 * 32], 0, 10) == c[67, 7]   # block 1, u = 3: 24 + 6 + 1
    assert _bits(vb[2 * 1280 + 40 * 8:2 * 1280 + 40 * 9], 10, 10) == c[128, 10]  # block 2, u = 0, j = 10
    assert np.array_equal(oracle.unpack_k(3, kb, T), c)
    assert np.array_equal(oracle.unpack_v(3, vb, T), c)


def test_pack10_leaves_other_tokens_bits_alone():
    """Tokens share bytes in the value layout (two 20-bit pairs per 5 bytes):
    packing one token over a filled stream changes only that token's codes."""
    T = 64
    c = synth.random_codes(7, (T, 16), 1024)
    vb = oracle.pack_v(3, c, T)
    for t in (0, 4, 5, 63):
        one = c.copy()
        one[t] = synth.random_codes(8 + t, (1, 16), 1024)[0]
        vb2 = vb.copy()
        oracle.pack_v(3, one[:t + 1], T, vb2)      # re-pack tokens 0..t (t's codes new)
        got = oracle.unpack_v(3, vb2, T)
        assert np.array_equal(got[t], one[t])
        assert np.array_equal(np.delete(got, t, axis=0), np.delete(c, t, axis=0))


def test_1p25bit_format_is_ten_bits_per_eight_dims():
    """The 1.25-bit width: 1024 entries of 8 dims, 10 bits per 8 elements, 16
    codes and 20 bytes per token."""
    E, dsub = oracle.FORMATS[3]
    assert (E, dsub) == (1024, 8)
    assert math.log2(E) / dsub == 1.25 and oracle.code_bytes_per_token(3) * 8 == 10 * 16


def test_4bit_format_is_eight_bits_per_two_dims():
    """The 4-bit width: 256 entries of 2 dims, 8 bits per 2 elements, 64 codes
    and 64 bytes per token."""
    E, dsub = oracle.FORMATS[4]
    assert (E, dsub) == (256, 2)
    assert math.log2(E) / dsub == 4.0 and oracle.code_bytes_per_token(4) * 8 == 8 * 64


def test_pack_4bit_positions():
    """Hand-computed byte positions of the 4-bit layouts (2^8 x 2, byte codes):
    keys token-major, 64 bytes per token, byte j = sub-vector j; values in
    64-token blocks of 4096 bytes, (t, j) with w = j // 2, u = t % 64 -> chunk
    16*((w%16)//4) + 4*(u%4) + w%4, byte 4*(u//4) + 2*(w//16) + j%2 of that
    64-byte chunk."""
    T = 130
    c = synth.random_codes(6, (T, 64), 256)
    kb = oracle.pack_k(4, c, 192)
    vb = oracle.pack_v(4, c, 192)
    assert kb.size == vb.size == 192 * 64
    for t, j in [(0, 0), (0, 63), (1, 0), (33, 7), (129, 63)]:
        assert kb[t * 64 + j] == c[t, j]
    assert vb[0] == c[0, 0] and vb[1] == c[0, 1]     # chunk 0, bytes 0 and 1
    assert vb[64 * 23] == c[1, 14]                   # w = 7: chunk 16 + 4 + 3, byte 0
    assert vb[64 * 23 + 33] == c[33, 15]             # same chunk, byte 4 * 8 + 0 + 1
    assert vb[64 * 3 + 2] == c[0, 38]                # w = 19: chunk 3, byte 2 * 1
    assert vb[4096 + 64 * 63 + 31] == c[95, 63]      # block 1, u = 31, w = 31: chunk 48 + 12 + 3, byte 28 + 2 + 1
    assert vb[4096 + 64 * 24 + 2] == c[66, 40]       # block 1, u = 2, w = 20: chunk 16 + 8 + 0, byte 2
    assert vb[2 * 4096 + 64 * 4 + 1] == c[129, 1]    # block 2, u = 1: chunk 4, byte 1
    assert np.array_equal(oracle.unpack_k(4, kb, T), c)
    assert np.array_equal(oracle.unpack_v(4, vb, T), c)


def test_pack_4bit_round_trip_and_every_byte_once():
    """Every (token, sub-vector) of a block lands on its own byte: packing the
    code value 1 at one position at a time sets exactly one byte each time,
    all 4096 of them distinct; random codes survive pack/unpack."""
    seen = set()
    for t in range(64):
        for j in range(64):
            c = np.zeros((64, 64), dtype=np.uint16)
            c[t, j] = 1
            nz = np.flatnonzero(oracle.pack_v(4, c, 64))
            assert nz.size == 1
            seen.add(int(nz[0]))
    assert len(seen) == 4096
    c = synth.random_codes(7, (300, 64), 256)
    assert np.array_equal(oracle.unpack_v(4, oracle.pack_v(4, c, 320), 300), c)
    assert np.array_equal(oracle.unpack_k(4, oracle.pack_k(4, c, 320), 300), c)


# ------------------------------------------------------------------------ K-Means

def _blobs(seed, E, dsub, per):
    rng = np.random.default_rng(seed)
    centers = rng.standard_normal((E, dsub)) * 10
    pts = (centers[:, None, :] + rng.standard_normal((E, per, dsub)) * 0.5).reshape(-1, dsub)
    perm = rng.permutation(len(pts))
    pts = pts[perm]
    # One initial point from each blob keeps every cluster non-empty.
    owner = np.repeat(np.arange(E), per)[perm]
    init = np.array([np.flatnonzero(owner == e)[0] for e in range(E)])
    return pts, init


@pytest.mark.parametrize("dsub,E", [(2, 20), (4, 16), (8, 12)])
def test_kmeans_matches_sklearn_lloyd(dsub, E):
    from sklearn.cluster import KMeans
    pts, init = _blobs(dsub, E, dsub, 40)
    # Start both from the same points, not necessarily the nearest blob order.
    init = init[::-1].copy()
    cent, assign = oracle.kmeans(pts, init, iters=20)
    km = KMeans(n_clusters=E, init=pts[init], n_init=1, max_iter=20, tol=0.0, algorithm="lloyd")
    km.fit(pts)
    assert np.abs(cent - km.cluster_centers_).max() < 1e-9
    assert np.array_equal(assign, km.labels_)


@pytest.mark.parametrize("fmt,n_cal", [(0, 64), (1, 512), (4, 32)])
def test_train_codebooks_recovers_planted_books(fmt, n_cal):
    """The composition train_codebooks = transform the keys, cut rows into
    sub-vectors, K-Means, round to fp16: calibration rows built exactly from
    planted fp16 centroids (keys as s * H(concat C_K[codes]) with scipy's H,
    values as concat C_V[codes]), every entry used, and Forgy indices pointing
    at one point of each entry, give back the planted books bit for bit (a
    transposed reshape, a missing transform or a wrong index would mix the
    clusters)."""
    E, dsub = oracle.FORMATS[fmt]
    J = D // dsub
    rng = np.random.default_rng(300 + fmt)

    def planted(seed):
        book = synth.random_fp16_book(seed, (E, dsub))
        while len({r.tobytes() for r in book}) < E:           # distinct rows
            book = synth.random_fp16_book(seed := seed + 1, (E, dsub))
        return book

    kb, vb = planted(310 + fmt), planted(320 + fmt)
    codes = []
    for _ in range(2):
        c = rng.integers(0, E, size=n_cal * J)
        c[:E] = rng.permutation(E)                            # every entry used
        codes.append(c.reshape(n_cal, J))
    kc, vc = codes
    s = rng.uniform(0.7, 6.0, D).astype(np.float32)
    H = scipy.linalg.hadamard(D) / math.sqrt(D)
    kf = kb.view(np.float16).astype(np.float64)
    vf = vb.view(np.float16).astype(np.float64)
    k = (kf[kc].reshape(n_cal, D) @ H) * s.astype(np.float64)
    v = vf[vc].reshape(n_cal, D)
    # Point p = t * J + j of the sub-vector array; entry e starts from a point of entry e.
    init_k = np.array([np.flatnonzero(kc.ravel() == e)[0] for e in range(E)])
    init_v = np.array([np.flatnonzero(vc.ravel() == e)[0] for e in range(E)])
    gk, gv = oracle.train_codebooks(fmt, k, v, s, init_k, init_v, iters=3)
    assert np.array_equal(gk, kb)
    assert np.array_equal(gv, vb)


def test_kmeans_objective_never_increases():
    rng = np.random.default_rng(3)
    pts = rng.standard_normal((3000, 4))
    init = synth.kmeans_init_indices(3, len(pts), 32)
    prev = np.inf
    for it in range(1, 8):
        cent, assign = oracle.kmeans(pts, init, iters=it)
        obj = ((pts - cent[assign]) ** 2).sum()
        assert obj <= prev + 1e-9
        prev = obj


def test_kmeans_empty_cluster_keeps_its_centroid():
    rng = np.random.default_rng(4)
    pts = rng.standard_normal((200, 4))
    init = np.array([0, 1, 2, 2])       # entry 3 duplicates entry 2: ties go to 2, 3 stays empty
    cent, assign = oracle.kmeans(pts, init, iters=1)
    assert not np.any(assign == 3)
    assert np.array_equal(cent[3], pts[2])


def test_kmeans_each_point_its_own_centroid():
    rng = np.random.default_rng(5)
    pts = rng.standard_normal((64, 8))
    cent, assign = oracle.kmeans(pts, np.arange(64), iters=3)
    assert np.array_equal(cent, pts)
    assert np.array_equal(assign, np.arange(64))
