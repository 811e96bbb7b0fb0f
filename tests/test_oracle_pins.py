"""Pins of the CPU oracle to things other than itself.

Each test checks the oracle against what the K-quant kernel arc page and
plain arithmetic fix: records built from known fields by an independent
encoder (tests/kq_encode.py), closed forms, exact special cases,
invariants of the Q8_K quantiser, brute force on tiny inputs, and a
reduction to an ordinary integer matmul.  A plausible mistake in the oracle
(a swapped nibble, a wrong bit of the 6-bit packing, a dropped min term, a
sign slip in the Q6_K fold, a wrong bsum index) fails at least one of them;
test_planted_mistakes_are_caught shows that for a few such mistakes.
"""
import os
import subprocess

import numpy as np
import pytest

import oracle
import synth
from kq_encode import dequant_fields, encode, random_fields, pack_scale_min
from q8k_cases import exact_q8k_chunk, quotient_chunks, reciprocal_codes

FMTS = ["q4_k", "q5_k", "q6_k"]


# --------------------------------------------------------------- f16 -----
def test_f16_decode_matches_numpy_for_every_pattern():
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # subnormals are kept, not flushed
    assert oracle.f16_to_double(0x0001) == 2.0 ** -24


# ------------------------------------------------------------ decode -----
@pytest.mark.parametrize("fmt", FMTS)
def test_decode_recovers_encoded_fields(fmt):
    rng = np.random.default_rng(11)
    for _ in range(50):
        f = random_fields(fmt, rng)
        b = oracle.decode(fmt, encode(fmt, f))
        assert np.array_equal(b["q"], f["q"])
        assert np.array_equal(b["sc"], f["sc"])
        assert b["d"] == float(f["d"])
        if fmt != "q6_k":
            assert np.array_equal(b["m"], f["m"])
            assert b["dmin"] == float(f["dmin"])


def test_scale_min_packing_hand_cases():
    # ggml 6-bit packing worked by hand: scale bytes 0..11 =
    #  [0xC1, 0x02, 0x03, 0x44, 0x85, 0x06, 0x07, 0xC8, 0x9A, 0x0B, 0x0C, 0x3D]
    # sc0..3 = low 6 bits of bytes 0..3         = 1, 2, 3, 4
    # m0..3  = low 6 bits of bytes 4..7         = 5, 6, 7, 8
    # sc4    = (byte8 & 15) | (byte0 >> 6) << 4 = 0xA | 3<<4  = 58
    # sc5    = (byte9 & 15) | (byte1 >> 6) << 4 = 0xB | 0     = 11
    # sc6    = 0xC | 0 = 12;  sc7 = 0xD | (0x44 >> 6 = 1) << 4 = 29
    # m4     = (byte8 >> 4) | (byte4 >> 6) << 4 = 9 | 2<<4    = 41
    # m5     = 0 | 0 = 0; m6 = 0 | 0 = 0; m7 = 3 | (0xC8 >> 6 = 3) << 4 = 51
    s = np.array([0xC1, 0x02, 0x03, 0x44, 0x85, 0x06, 0x07, 0xC8, 0x9A, 0x0B, 0x0C, 0x3D], np.uint8)
    rec = np.zeros(144, np.uint8)
    rec[4:16] = s
    b = oracle.decode("q4_k", rec)
    assert list(b["sc"]) == [1, 2, 3, 4, 58, 11, 12, 29]
    assert list(b["m"]) == [5, 6, 7, 8, 41, 0, 0, 51]
    assert np.array_equal(pack_scale_min(b["sc"], b["m"]), s)


def test_quant_positions_hand_cases():
    # Q4_K: byte 16 + 32p + l holds weight 64p + l (low nibble) and
    # 64p + 32 + l (high nibble)
    rec = np.zeros(144, np.uint8)
    rec[16 + 32 * 2 + 5] = 0x9E
    q = oracle.decode("q4_k", rec)["q"]
    assert q[128 + 5] == 0xE and q[160 + 5] == 0x9 and q.sum() == 0xE + 0x9
    # Q5_K: fifth bit of weight 32j + l is bit j of high-bit byte l
    rec = np.zeros(176, np.uint8)
    rec[16 + 7] = 0b1000_0010
    q = oracle.decode("q5_k", rec)["q"]
    assert q[32 * 1 + 7] == 16 and q[32 * 7 + 7] == 16 and q.sum() == 32
    # Q6_K: weight 128h + 32t + l; t=3 takes the high nibble of low byte
    # 64h + l + 32 and bits 6..7 of high byte 32h + l
    rec = np.zeros(210, np.uint8)
    rec[64 * 1 + 4 + 32] = 0x70           # high nibble 7 -> t = 3, low 0 -> t = 1
    rec[128 + 32 * 1 + 4] = 0b1100_0000   # bits 6..7 = 3 -> t = 3
    q = oracle.decode("q6_k", rec)["q"]
    assert q[128 + 96 + 4] == 7 + 16 * 3 and q[128 + 32 + 4] == 0
    assert q.sum() == 55


# ---------------------------------------------------------- dequant -----
@pytest.mark.parametrize("fmt", FMTS)
def test_dequantize_matches_format_definition(fmt):
    rng = np.random.default_rng(12)
    fields = [random_fields(fmt, rng) for _ in range(6)]
    recs = np.stack([encode(fmt, f) for f in fields]).reshape(2, 3, -1)
    w = oracle.dequantize(fmt, recs)
    ref = np.concatenate([dequant_fields(fmt, f) for f in fields]).reshape(2, 768)
    assert np.array_equal(w, ref)


# ------------------------------------------------------------ Q8_K -------
def test_q8k_integer_inputs_are_exact():
    # x integer in [-127, 127] with a +-127 in every chunk: amax = 127,
    # d8 = 127/127 = 1 exactly, x/d8 = x exactly, so a == x
    rng = np.random.default_rng(13)
    x = rng.integers(-127, 128, size=(3, 1024)).astype(np.float32)
    x[:, ::256] = 127.0
    x[1, 256] = -127.0
    xq, xs, xbs = oracle.quantize_q8k(x)
    assert np.all(xs == 1.0)
    assert np.array_equal(xq, x.astype(np.int8))
    assert np.array_equal(xbs, x.reshape(3, -1, 16).sum(-1).astype(np.int16))


def test_q8k_rounds_half_to_even():
    # amax 127 -> d8 = 1; quotients land exactly on .5
    x = np.zeros((1, 256), np.float32)
    x[0, 0] = 127.0
    x[0, 1:7] = [2.5, 3.5, -2.5, -3.5, 0.5, 126.5]
    xq, _, _ = oracle.quantize_q8k(x)
    assert list(xq[0, :7]) == [127, 2, 4, -2, -4, 0, 126]


def test_q8k_zero_chunk_and_single_value():
    x = np.zeros((1, 512), np.float32)
    x[0, 256 + 9] = -0.3
    xq, xs, xbs = oracle.quantize_q8k(x)
    assert xs[0, 0] == 0.0 and not xq[0, :256].any() and not xbs[0, :16].any()
    assert xs[0, 1] == np.float32(np.float32(0.3) / np.float32(127.0))
    assert xq[0, 256 + 9] == -127 and np.count_nonzero(xq[0, 256:]) == 1
    assert xbs[0, 16] == -127


def test_q8k_invariants_on_random_rows():
    x = synth.activations(4, 2560, 5)
    xq, xs, xbs = oracle.quantize_q8k(x)
    c = x.reshape(4, 10, 256).astype(np.float64)
    a = xq.reshape(4, 10, 256).astype(np.float64)
    d = xs.astype(np.float64)[..., None]
    # scale is amax/127 (to within binary32 rounding), |a| reaches 127
    amax = np.abs(c).max(-1)
    assert np.allclose(xs, amax / 127.0, rtol=2 ** -23, atol=0)
    assert np.all(np.abs(a).max(-1) == 127)
    # every code is the nearest: |x - d8 a| <= d8/2 (+ binary32 slack)
    assert np.all(np.abs(c - d * a) <= d * (0.5 + 1e-5))
    # bsums are exact sums of 16 codes
    assert np.array_equal(xbs, xq.reshape(4, -1, 16).astype(np.int64).sum(-1))


def test_q8k_power_of_two_scaling_is_equivariant():
    # scaling x by 2^e scales d8 by 2^e and leaves every code unchanged
    x = synth.activations(2, 768, 6)
    xq0, xs0, _ = oracle.quantize_q8k(x)
    for e in (-20, -3, 7):
        xq1, xs1, _ = oracle.quantize_q8k(np.ldexp(x, e).astype(np.float32))
        assert np.array_equal(xq1, xq0)
        assert np.array_equal(xs1, np.ldexp(xs0, e))


def test_q8k_code_is_the_rounded_binary32_quotient():
    # the code of x is rint(binary32(x / d8)) with d8 = binary32(amax / 127),
    # both correctly rounded, ties to even ("The pieces", kq v2 item: q =
    # round(x/d) per 256-value chunk), worked out here in exact rationals.
    # These chunks sit where a reciprocal multiply x * (1/d8) lands on the
    # other side of a .5 boundary, so that reading fails this pin.
    x = quotient_chunks(6, seed=31)
    xq, xs, xbs = oracle.quantize_q8k(x.reshape(2, 768))
    xq, xs = xq.reshape(6, 256), xs.reshape(6)
    for c in range(6):
        codes, d8 = exact_q8k_chunk(x[c])
        assert float(d8) == float(xs[c])
        assert np.array_equal(xq[c].astype(np.int64), codes), f"chunk {c}"
        # the chunk separates the two readings in at least 20 places
        assert (reciprocal_codes(x[c]) != codes).sum() >= 20
    assert np.array_equal(xbs.reshape(6, 16), xq.reshape(6, 16, 16).astype(np.int64).sum(-1))


def test_q8k_code_definition_on_random_and_tie_chunks():
    # the same exact definition on ordinary N(0,1) chunks, exact .5 ties at
    # d8 = 1, tiny magnitudes and a chunk whose amax is negative
    x = synth.activations(1, 1024, 32).reshape(4, 256)
    x[1] = 0.0
    x[1, 0] = -127.0
    x[1, 1:9] = [2.5, 3.5, -2.5, -3.5, 0.5, 126.5, -0.5, 1.5]
    x[2] *= np.float32(2.0 ** -60)
    x[3, 7] = -np.abs(x[3]).max() * np.float32(1.5)
    xq, xs, _ = oracle.quantize_q8k(x.reshape(1, 1024))
    for c in range(4):
        codes, d8 = exact_q8k_chunk(x[c])
        assert float(d8) == float(xs[0, c])
        assert np.array_equal(xq[0, 256 * c:256 * (c + 1)].astype(np.int64), codes), f"chunk {c}"


# ------------------------------------------------------------ folds ------
def _brute_partials(fmt, fields, a):
    """int64 brute force of P and M for one superblock: elementwise."""
    q = np.asarray(fields["q"], np.int64)
    a = np.asarray(a, np.int64)
    if fmt == "q6_k":
        sc = np.repeat(np.asarray(fields["sc"], np.int64), 16)
        return int((sc * (q - 32) * a).sum()), 0
    sc = np.repeat(np.asarray(fields["sc"], np.int64), 32)
    m = np.repeat(np.asarray(fields["m"], np.int64), 32)
    # the bsums identity: the min term is sum_i m_j(i) a_i
    return int((sc * q * a).sum()), int((m * a).sum())


@pytest.mark.parametrize("fmt", FMTS)
def test_partials_match_elementwise_brute_force(fmt):
    rng = np.random.default_rng(14)
    n, nsb, t = 3, 4, 3
    fields = [[random_fields(fmt, rng) for _ in range(nsb)] for _ in range(n)]
    recs = np.stack([np.stack([encode(fmt, f) for f in row]) for row in fields])
    x = synth.activations(t, nsb * 256, 7)
    xq, xs, xbs = oracle.quantize_q8k(x)
    P, M = oracle.partials(fmt, recs, xq, xbs)
    for tt in range(t):
        for r in range(n):
            for s in range(nsb):
                p, m = _brute_partials(fmt, fields[r][s], xq[tt, 256 * s: 256 * s + 256])
                assert P[tt, r, s] == p and M[tt, r, s] == m


def _const_q8k(sign):
    # every code +-127: x all equal gives d8 = x/127, a = x/d8 = 127
    x = np.full((1, 256), 0.75 * sign, np.float32)
    xq, xs, xbs = oracle.quantize_q8k(x)
    assert np.all(xq == 127 * sign)
    return xq, xs, xbs


@pytest.mark.parametrize("qv,sign,expect", [
    # sc = -128 everywhere; closed forms of iacc - 32*bacc = sum sc (q-32) a
    (63, -1, 256 * -128 * 31 * -127),
    (0, +1, 256 * -128 * -32 * 127),
    (63, +1, 256 * -128 * 31 * 127),
    (0, -1, 256 * -128 * -32 * -127),
])
def test_q6k_signed_fold_exact_at_extremes(qv, sign, expect):
    # |iacc| reaches 256*128*63*127 = 262,193,152 < 2^28 and
    # |32*bacc| reaches 32*16*128*2032 = 133,169,152 < 2^28
    rec = np.stack([encode("q6_k", {"d": np.float16(1.0), "sc": np.full(16, -128),
                                    "q": np.full(256, qv)})])[None]
    xq, xs, xbs = _const_q8k(sign)
    P, M = oracle.partials("q6_k", rec, xq, xbs)
    assert P[0, 0, 0] == expect and M[0, 0, 0] == 0
    assert abs(expect) < 2 ** 28


@pytest.mark.parametrize("fmt", ["q4_k", "q5_k"])
def test_q4q5_partials_closed_form_at_extremes(fmt):
    qmax = 15 if fmt == "q4_k" else 31
    rec = encode(fmt, {"d": np.float16(1.0), "dmin": np.float16(1.0), "sc": np.full(8, 63),
                       "m": np.full(8, 63), "q": np.full(256, qmax)})[None, None]
    xq, xs, xbs = _const_q8k(-1)
    P, M = oracle.partials(fmt, rec, xq, xbs)
    assert P[0, 0, 0] == 256 * 63 * qmax * -127
    assert M[0, 0, 0] == 8 * 63 * 32 * -127


# ------------------------------------------------------------- float -----
@pytest.mark.parametrize("fmt", FMTS)
def test_float_output_matches_brute_force_dequant_then_dot(fmt):
    rng = np.random.default_rng(15)
    n, nsb, t = 5, 3, 2
    fields = [[random_fields(fmt, rng) for _ in range(nsb)] for _ in range(n)]
    recs = np.stack([np.stack([encode(fmt, f) for f in row]) for row in fields])
    x = synth.activations(t, nsb * 256, 8)
    xq, xs, xbs = oracle.quantize_q8k(x)
    y = oracle.matmul(fmt, recs, xq, xs, xbs)
    R = oracle.rowmag(fmt, recs, xq, xs)
    w = np.stack([np.concatenate([dequant_fields(fmt, f) for f in row]) for row in fields])
    xhat = xq.astype(np.float64) * np.repeat(xs.astype(np.float64), 256, axis=1)
    y_ref = xhat @ w.T
    assert np.all(np.abs(y - y_ref) <= 1e-12 * R)
    assert np.allclose(R, (np.abs(xhat)[:, None, :] * np.abs(w)[None]).sum(-1), rtol=1e-12)
    # the binary32 "file dequant" (w rounded to float32) agrees within 1e-6 R
    y32 = xhat @ w.astype(np.float32).astype(np.float64).T
    assert np.all(np.abs(y - y32) <= 1e-6 * R)


@pytest.mark.parametrize("fmt", FMTS)
def test_reduces_to_integer_matmul(fmt):
    # sc = 1, m = 0, d = 1, dmin = 0 and integer activations with a +-127
    # in every chunk: y == q @ x (or (q - 32) @ x) exactly
    rng = np.random.default_rng(16)
    n, nsb, t = 4, 2, 3
    qmax = {"q4_k": 16, "q5_k": 32, "q6_k": 64}[fmt]
    qs = rng.integers(0, qmax, size=(n, nsb, 256))
    recs = np.empty((n, nsb, synth.BLOCK_BYTES[fmt]), np.uint8)
    for r in range(n):
        for s in range(nsb):
            if fmt == "q6_k":
                f = {"d": np.float16(1.0), "sc": np.ones(16, int), "q": qs[r, s]}
            else:
                f = {"d": np.float16(1.0), "dmin": np.float16(0.0), "sc": np.ones(8, int),
                     "m": np.zeros(8, int), "q": qs[r, s]}
            recs[r, s] = encode(fmt, f)
    x = rng.integers(-127, 128, size=(t, nsb * 256))
    x[:, ::256] = -127
    xq, xs, xbs = oracle.quantize_q8k(x.astype(np.float32))
    y = oracle.matmul(fmt, recs, xq, xs, xbs)
    wq = qs.reshape(n, -1) - (32 if fmt == "q6_k" else 0)
    assert np.array_equal(y, (x.astype(np.int64) @ wq.T).astype(np.float64))


def test_synthetic_workload_never_overflows_int32():
    for fmt in FMTS:
        w = synth.weights(fmt, 64, 2560, synth.seed_for(0, 1))
        x = synth.activations(4, 2560, synth.seed_for(0, 2))
        xq, xs, xbs = oracle.quantize_q8k(x)
        oracle.partials(fmt, w, xq, xbs)  # raises OverflowError on overflow


# --------------------------------------------------- planted mistakes ---
_MUTATIONS = {
    # a dropped min term
    "no_min": ("p += b.sc[j] * dot;\n                        m += b.m[j]",
               "p += b.sc[j] * dot;\n                        m += 0 * b.m[j]"),
    # Q4_K nibble halves swapped
    "nibble": ("int q = (j % 2 == 0) ? (byte & 15) : (byte >> 4);",
               "int q = (j % 2 == 0) ? (byte >> 4) : (byte & 15);"),
    # sign slip in the Q6_K fold
    "q6sign": ("p = iacc - 32 * bacc;", "p = iacc + 32 * bacc;"),
    # wrong bsum pairing
    "bsum": ("((int64_t)bs[2 * j] + bs[2 * j + 1])", "((int64_t)bs[j] + bs[j + 1])"),
    # 6-bit packing: wrong high bits for j >= 4
    "pack": ("sc[j] = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);",
             "sc[j] = (s[j + 4] & 15) | ((s[j] >> 6) << 4);"),
    # the Q8_K quotient taken as a reciprocal multiply
    "recip": ("float v = c[i] / d8;", "float v = c[i] * (1.0f / d8);"),
}


@pytest.mark.parametrize("name", sorted(_MUTATIONS))
def test_planted_mistakes_are_caught(name, tmp_path):
    """Build a copy of the oracle with one planted mistake and check that
    the pins above (brute-force partials, definition dequant) reject it."""
    import ctypes
    src = open(os.path.join(os.path.dirname(oracle.__file__), "kq_oracle.c")).read()
    old, new = _MUTATIONS[name]
    assert src.count(old) == 1
    lib = tmp_path / "libmut.so"
    (tmp_path / "mut.c").write_text(src.replace(old, new))
    subprocess.run(["gcc", "-O1", "-fPIC", "-shared", "-o", str(lib), str(tmp_path / "mut.c"), "-lm"],
                   check=True)
    mut = ctypes.CDLL(str(lib))
    saved = oracle._lib
    try:
        oracle._lib = None
        real = oracle._load()
        for f in ("orc_dequantize", "orc_quantize_q8k", "orc_partials", "orc_matmul",
                  "orc_rowmag", "orc_decode"):
            getattr(mut, f).argtypes = getattr(real, f).argtypes
            getattr(mut, f).restype = ctypes.c_int
        mut.orc_f16_to_double.argtypes = real.orc_f16_to_double.argtypes
        mut.orc_f16_to_double.restype = ctypes.c_double
        oracle._lib = mut
        failed = False
        checks = [lambda f=f, t=t: t(f) for f in FMTS
                  for t in (test_partials_match_elementwise_brute_force, test_dequantize_matches_format_definition)]
        checks += [test_q8k_code_is_the_rounded_binary32_quotient, test_q8k_code_definition_on_random_and_tie_chunks]
        for check in checks:
            try:
                check()
            except AssertionError:
                failed = True
        assert failed, f"planted mistake {name!r} went unnoticed"
    finally:
        oracle._lib = saved
