"""Pins for oracle/w8a8.py: per-token E4M3 activation quantisation and the
W8A8 product, against the format's definition, torch's E4M3 cast, the W8A16
oracle on exactly representable rows, and the rounding bound."""
import numpy as np
import torch

from oracle import codecs, model, w8a8


def _rows(m, k, seed):
    r = np.random.default_rng(seed)
    x = r.standard_normal((m, k)).astype(np.float32)
    x[1] *= 1e-3          # small row: scale far below 1
    x[2] *= 300.0         # large row
    x[3, ::7] = 0.0       # scattered zeros
    return codecs.bf16_round(x).astype(np.float32)


def test_worked_example():
    # row 0: amax 3.5, so inv = 128 and the codes are those of 128, -64, 448, 0:
    #   128 = 2^7 -> E = 14, m = 0 -> 0x70; -64 = -2^6 -> 0x80 | (13 << 3) = 0xE8;
    #   448 = 1.75 * 2^8 -> E = 15, m = 6 -> 0x7E; scale = 3.5 / 448 = 2^-7.
    # row 1: amax 1, q = [448, 0.3 * 448 = 134.4]; 134.4 lies between 128 and
    #   144 (step 16 in [128, 256)) and is nearer 128 -> 0x70; scale = 1/448.
    x = np.float32([[1.0, -0.5, 3.5, 0.0], [1.0, 0.3, 0.0, 0.0]])
    codes, scale = w8a8.act_quant_e4m3(x)
    assert codes.tolist() == [[0x70, 0xE8, 0x7E, 0x00], [0x7E, 0x70, 0x00, 0x00]]
    assert scale[0] == np.float32(2.0 ** -7)
    assert scale[1] == np.float32(1.0) / np.float32(448.0)


def test_row_max_maps_to_largest_code_and_zero_row():
    x = _rows(6, 96, 0)
    x[5] = 0.0
    codes, scale = w8a8.act_quant_e4m3(x)
    for m in range(5):
        j = int(np.argmax(np.abs(x[m])))
        assert codes[m, j] == (0xFE if x[m, j] < 0 else 0x7E)
        assert scale[m] == np.float32(np.float32(np.abs(x[m]).max()) / np.float32(448.0))
    assert scale[5] == 0.0 and not codes[5].any()
    assert not np.any((codes & 0x7F) == 0x7F)          # never NaN


def test_codes_match_torch_cast_of_the_scaled_row():
    x = _rows(8, 256, 1)
    codes, _ = w8a8.act_quant_e4m3(x)
    amax = np.abs(x).max(axis=1).astype(np.float32)
    q = x * (np.float32(448.0) / amax)[:, None]
    ref = torch.from_numpy(np.clip(q, -448.0, 448.0)).to(torch.float8_e4m3fn)
    assert np.array_equal(codes, ref.view(torch.uint8).numpy())


def test_sign_and_power_of_two_symmetry():
    x = _rows(5, 64, 2)
    c0, s0 = w8a8.act_quant_e4m3(x)
    c1, s1 = w8a8.act_quant_e4m3(-x)
    nz = x != 0
    assert np.array_equal(c1[nz], c0[nz] ^ 0x80)
    assert np.array_equal(s0, s1)
    c2, s2 = w8a8.act_quant_e4m3(x * np.float32(8.0))
    assert np.array_equal(c2, c0) and np.array_equal(s2, s0 * np.float32(8.0))


def test_dequant_error_within_half_a_step():
    x = _rows(8, 512, 3)
    codes, scale = w8a8.act_quant_e4m3(x)
    xd = w8a8.act_dequant(codes, scale)
    amax = np.abs(x).max(axis=1, keepdims=True).astype(np.float64)
    q = x.astype(np.float64) * 448.0 / amax
    # half an E4M3 step: 2^-4 of the magnitude in the normal range, 2^-10 below
    # it; plus the float32 roundings of inv and q (a few 2^-24 relative)
    bound = np.maximum(np.abs(q) * 2.0 ** -4, 2.0 ** -10) + np.abs(q) * 2.0 ** -21
    assert np.all(np.abs(xd * 448.0 / amax - q) <= bound)


def _weights(n, k, seed):
    r = np.random.default_rng(seed)
    w = r.standard_normal((n, k)) * 0.05
    sc = np.abs(w).max(axis=1) / 448.0
    codes = codecs.e4m3_encode(w / sc[:, None])
    return codes, codecs.bf16_bits(sc)


def test_exact_rows_give_the_w8a16_product():
    # rows built from E4M3 values times 2^-j that reach 448 * 2^-j quantise to
    # themselves, so the W8A8 product is the W8A16 product of the same rows
    r = np.random.default_rng(4)
    m, k, n = 6, 128, 40
    cx = r.integers(0, 256, size=(m, k), dtype=np.uint8)
    cx[(cx & 0x7F) == 0x7F] = 0x10
    cx[:, 5] = 0x7E
    e = np.array([0, -3, 5, -9, 2, -1])
    x = (codecs.e4m3_decode(cx) * np.exp2(e)[:, None]).astype(np.float32)
    codes, scale = w8a8.act_quant_e4m3(x)
    assert np.array_equal(codes, cx)
    assert np.array_equal(scale, np.exp2(e).astype(np.float32))
    wc, ws = _weights(n, k, 5)
    y8 = w8a8.gemm_w8a8(codes, scale, wc, ws)
    y16 = x.astype(np.float64) @ model.weight_eff(wc, ws).T
    np.testing.assert_allclose(y8, y16, rtol=1e-12, atol=1e-12 * np.abs(y16).max())


def test_product_within_the_activation_rounding_bound():
    m, k, n = 7, 320, 48
    x = _rows(m, k, 6)
    wc, ws = _weights(n, k, 7)
    codes, scale = w8a8.act_quant_e4m3(x)
    y8 = w8a8.gemm_w8a8(codes, scale, wc, ws)
    weff = model.weight_eff(wc, ws)
    y16 = x.astype(np.float64) @ weff.T
    err_x = np.abs(w8a8.act_dequant(codes, scale) - x.astype(np.float64))
    bound = err_x @ np.abs(weff).T
    assert np.all(np.abs(y8 - y16) <= bound * (1 + 1e-9) + 1e-12)
    # and the error is not trivially zero (the rows are not representable)
    assert np.abs(y8 - y16).max() > 0


def test_w8a8_depth_golden_files_are_consistent():
    """The full-depth W8A8 golden file and its sensitivity file describe the
    same inputs as the W8A16 golden file; the W8A8 logits differ from the
    W8A16 ones (the reading is applied) by a few percent; the oracle's own
    movement under planted one-ulp disagreements grows with depth."""
    import json
    import os
    gdir = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
    base = json.load(open(os.path.join(gdir, "depth36_qwen3.json")))
    g8 = json.load(open(os.path.join(gdir, "depth36_qwen3_w8a8.json")))
    sens = json.load(open(os.path.join(gdir, "depth36_qwen3_w8a8_sensitivity.json")))
    assert g8["inputs_sha256_16"] == base["inputs_sha256_16"] == sens["inputs_sha256_16"]
    assert g8["taps"] == sens["taps"] == [1, 4, 12, 36]
    for d in g8["taps"]:
        a = np.array(g8["results"][str(d)]["logits"])
        b = np.array(base["results"][g8["case"]][str(d)]["logits"])
        rel = np.max(np.abs(a - b)) / np.max(np.abs(b))
        assert 1e-3 < rel < 0.2, (d, rel)
    for frac, per_depth in sens["fractions"].items():
        v = [per_depth[str(d)] for d in sens["taps"]]
        assert all(x > 0 for x in v) and v == sorted(v), (frac, v)


def test_w8a8_layer_sensitivity_file():
    """The one-layer full-size W8A8 golden file holds the six sampled pairs the
    GPU test checks, each with 8 finite logits, its decision consistent with
    its own logits, and a positive planted-disagreement movement."""
    import json
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "w8a8_layer_sensitivity.json")
    doc = json.load(open(path))
    assert doc["fraction"] == 0.01 and len(doc["pairs"]) == 6
    for p in doc["pairs"].values():
        lg = np.array(p["logits"])
        assert lg.shape == (8,) and np.isfinite(lg).all()
        assert p["decision"] == (0x0F >> int(np.argmax(lg))) & 1
        assert 0 < p["moved_rel"] < 0.5
