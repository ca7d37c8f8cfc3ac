"""Pins of the fp8 (E4M3) KV-cache oracle against things other than itself:
values the format fixes (the pages print its largest magnitude), torch's own
float8_e4m3fn type (an independent encoder and decoder), invariants of
rounding, and dense SDPA on keys and values dequantized through torch."""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8 as of
from _pins import build_paged, sdpa_reference

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "e4m3.json")))


def torch_decode_all():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_largest_magnitude_is_the_pages_448():
    t = of.e4m3_table()
    assert np.nanmax(t) == GOLDEN["max_finite"] and np.nanmin(t) == -GOLDEN["max_finite"]
    assert of.e4m3_decode(0x7E) == 448.0 and of.e4m3_decode(0xFE) == -448.0


def test_special_codes():
    assert of.e4m3_decode(0x38) == 1.0
    assert of.e4m3_decode(0x08) == 2.0 ** -6  # smallest normal
    assert of.e4m3_decode(0x01) == 2.0 ** -9  # smallest subnormal
    assert of.e4m3_decode(0x07) == 7 * 2.0 ** -9
    assert of.e4m3_decode(0x00) == 0.0 and math.copysign(1.0, of.e4m3_decode(0x80)) == -1.0
    assert math.isnan(of.e4m3_decode(0x7F)) and math.isnan(of.e4m3_decode(0xFF))
    assert int(np.isfinite(of.e4m3_table()).sum()) == 254


def test_decode_table_matches_torch():
    ours, theirs = of.e4m3_table(), torch_decode_all()
    same = (ours == theirs) | (np.isnan(ours) & np.isnan(theirs))
    assert same.all()


def test_encode_round_trips_every_finite_code():
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        assert of.e4m3_encode(of.e4m3_decode(c)) == c, hex(c)


def _sweep():
    t = of.e4m3_table()
    pos = np.unique(t[np.isfinite(t) & (t >= 0)])
    mids = (pos[1:] + pos[:-1]) / 2  # exact ties
    quarter = pos[:-1] + (pos[1:] - pos[:-1]) / 4
    rng = np.random.default_rng(7)
    rand = rng.uniform(-448, 448, 2000)
    return np.concatenate([pos, -pos, mids, -mids, quarter, -quarter, rand, [2.0 ** -10, 3 * 2.0 ** -11, 1e-30]])


def test_encode_matches_torch_within_range():
    x = _sweep()
    x = x[np.abs(x) <= 448.0]
    theirs = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = np.array([of.e4m3_encode(float(v)) for v in x], dtype=np.uint8)
    assert np.array_equal(ours, theirs)


def test_ties_go_to_the_even_mantissa():
    assert of.e4m3_encode(1.0625) == 0x38  # between 1.0 (m=0) and 1.125 (m=1)
    assert of.e4m3_encode(1.1875) == 0x3A  # between 1.125 (m=1) and 1.25 (m=2)
    assert of.e4m3_encode(2.0 ** -10) == 0x00  # half the smallest subnormal: ties to 0
    assert of.e4m3_encode(3 * 2.0 ** -10) == 0x02  # 1.5 subnormal steps: to 2


def test_saturation_and_nan():
    for v in (448.0, 449.0, 464.0, 1000.0, math.inf):
        assert of.e4m3_encode(v) == 0x7E
        assert of.e4m3_encode(-v) == 0xFE
    assert of.e4m3_encode(math.nan) == 0x7F


def test_encode_is_monotone_and_nearest():
    x = np.sort(_sweep())
    codes = [of.e4m3_encode(float(v)) for v in x]
    vals = np.array([of.e4m3_decode(c) for c in codes])
    assert np.all(np.diff(vals) >= 0)
    t = of.e4m3_table()
    fin = t[np.isfinite(t)]
    for v, q in zip(x, vals):
        assert abs(q - v) <= np.min(np.abs(fin - v)) + 0.0  # no finite code is strictly nearer


def test_quantize_divides_in_fp32():
    """The code is decided from the fp32 quotient, as the kernel computes it: a
    case where the float64 quotient lands on the other side of a tie."""
    rng = np.random.default_rng(3)
    found = None
    for _ in range(200000):
        x = np.float32(rng.uniform(-4, 4))
        s = np.float32(rng.uniform(0.005, 0.05))
        q32 = float(np.float32(x / s))
        q64 = float(x) / float(s)
        if of.e4m3_encode(q32) != of.e4m3_encode(q64):
            found = (x, s)
            break
    assert found is not None
    x, s = found
    assert of.quantize(np.array([x], np.float32), float(s))[0] == of.e4m3_encode(float(np.float32(x / s)))


def _fp8_problem(seed, lens, n_h, n_kv, d, q_len):
    """A small paged fp8 problem, built token by token, plus its dequantized
    contiguous K/V through torch's float8 type (an independent decoder)."""
    P = build_paged(seed, list(lens), n_h, n_kv, d, q_len, "bf16")
    rng = np.random.default_rng(seed + 1)
    k_scale = (0.01 + 0.02 * rng.random(n_kv)).astype(np.float32)
    v_scale = (0.01 + 0.02 * rng.random(n_kv)).astype(np.float32)
    NB = P["k_cache"].shape[0]
    kc = rng.integers(0, 0x7F, size=(NB, 16, n_kv, d)).astype(np.uint8) | (rng.integers(0, 2, size=(NB, 16, n_kv, d)) << 7).astype(np.uint8)
    vc = rng.integers(0, 0x7F, size=(NB, 16, n_kv, d)).astype(np.uint8) | (rng.integers(0, 2, size=(NB, 16, n_kv, d)) << 7).astype(np.uint8)
    # keep magnitudes moderate: codes below 0x58 (values < 2^4) so the scores stay O(1)
    kc = np.where((kc & 0x7F) > 0x57, kc & 0xD7, kc).astype(np.uint8)
    vc = np.where((vc & 0x7F) > 0x57, vc & 0xD7, vc).astype(np.uint8)
    Ks, Vs = [], []
    for b, L in enumerate(lens):
        rows_k = np.stack([kc[P["block_tables"][b, t // 16], t % 16] for t in range(L)])
        rows_v = np.stack([vc[P["block_tables"][b, t // 16], t % 16] for t in range(L)])
        dk = torch.from_numpy(rows_k).view(torch.float8_e4m3fn).to(torch.float64).numpy() * k_scale[None, :, None].astype(np.float64)
        dv = torch.from_numpy(rows_v).view(torch.float8_e4m3fn).to(torch.float64).numpy() * v_scale[None, :, None].astype(np.float64)
        Ks.append(dk)
        Vs.append(dv)
    P.update(k_codes=kc, v_codes=vc, k_scale=k_scale, v_scale=v_scale, Ks=Ks, Vs=Vs)
    return P


@pytest.mark.parametrize("q_len", [1, 5])
def test_fp8_decode_matches_dense_sdpa(q_len):
    P = _fp8_problem(11, (max(1, q_len), 16, 17, 40), 8, 2, 16, q_len)
    scale = 0.29
    ref = sdpa_reference(P, scale)
    got = of.paged_decode_fp8(P["q"], P["k_codes"], P["v_codes"], P["k_scale"], P["v_scale"], P["block_tables"],
                              P["context_lens"], scale, q_len, "bf16")
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_fp8_cache_write_places_codes_and_keeps_the_rest():
    rng = np.random.default_rng(5)
    NB, n_kv, d, T = 6, 2, 16, 9
    kc = rng.integers(0, 256, size=(NB, 16, n_kv, d)).astype(np.uint8)
    vc = rng.integers(0, 256, size=(NB, 16, n_kv, d)).astype(np.uint8)
    k = rng.standard_normal((T, n_kv, d)).astype(np.float32)
    v = rng.standard_normal((T, n_kv, d)).astype(np.float32)
    slots = rng.permutation(NB * 16)[:T].astype(np.int64)
    slots[3] = -1
    ks = np.array([0.011, 0.03], np.float32)
    vs = np.array([0.02, 0.0125], np.float32)
    assert np.abs(k / ks[None, :, None]).max() < 448 and np.abs(v / vs[None, :, None]).max() < 448
    k2, v2 = of.cache_write_fp8(kc, vc, k, v, slots, ks, vs, "f32")
    flatk, flatv = k2.reshape(-1, n_kv, d), v2.reshape(-1, n_kv, d)
    touched = set(int(s) for s in slots if s >= 0)
    for s in range(NB * 16):
        if s not in touched:
            assert np.array_equal(flatk[s], kc.reshape(-1, n_kv, d)[s])
    for t, s in enumerate(slots):
        if s < 0:
            continue
        for g in range(n_kv):
            # independent route: torch's cast of the fp32 quotient (in range here)
            want = torch.from_numpy((k[t, g] / ks[g]).astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert np.array_equal(flatk[s, g], want)
            wantv = torch.from_numpy((v[t, g] / vs[g]).astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert np.array_equal(flatv[s, g], wantv)


def test_fp8_cache_write_saturates_out_of_range():
    k = np.array([[[1000.0, -1000.0, 4.47, -4.49]]], np.float32)  # one token, one head, d = 4
    kc = np.zeros((1, 16, 1, 4), np.uint8)
    k2, _ = of.cache_write_fp8(kc, kc, k, k, np.array([3]), np.array([0.01], np.float32),
                               np.array([0.01], np.float32), "f32")
    assert k2[0, 3, 0].tolist() == [0x7E, 0xFE, of.e4m3_encode(float(np.float32(np.float32(4.47) / np.float32(0.01)))), 0xFE]


FP8_MUTATIONS = {
    "exponent_bias_8": ("e4m3_decode", None),  # every value halved (bias 8 instead of 7); built below
    "no_saturation": ("e4m3_encode", lambda x: 0x7F if (not math.isnan(x) and abs(x) >= 448) else of._orig_encode(x)),
    "ties_away": ("e4m3_encode", lambda x: of._orig_encode(math.nextafter(x, math.copysign(math.inf, x)))),
    "scale_multiplies": ("quantize", lambda x32, s: of._orig_quantize(np.asarray(x32, np.float32) * np.float32(s) * np.float32(s), s)),
}


def _fp8_pins_pass():
    try:
        test_largest_magnitude_is_the_pages_448()
        test_special_codes()
        test_decode_table_matches_torch()
        test_encode_round_trips_every_finite_code()
        test_encode_matches_torch_within_range()
        test_ties_go_to_the_even_mantissa()
        test_saturation_and_nan()
        test_fp8_cache_write_places_codes_and_keeps_the_rest()
        test_fp8_decode_matches_dense_sdpa(1)
    except AssertionError:
        return False
    return True


@pytest.mark.parametrize("name", sorted(FP8_MUTATIONS))
def test_planted_fp8_mistake_is_caught(name, monkeypatch):
    fn, repl = FP8_MUTATIONS[name]
    monkeypatch.setattr(of, "_orig_encode", of.e4m3_encode, raising=False)
    monkeypatch.setattr(of, "_orig_quantize", of.quantize, raising=False)
    orig_decode = of.e4m3_decode
    if fn == "e4m3_decode":
        repl = (lambda c: orig_decode(c) / 2.0)
    monkeypatch.setattr(of, fn, repl)
    assert not _fp8_pins_pass(), name
