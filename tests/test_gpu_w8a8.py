"""GPU parity of the W8A8 path: per-token E4M3 activation quantisation
(codes and scales bit-exact against the oracle) and the fp8 x fp8 GEMM
(fp32-accumulated exact products, bf16 output, against the oracle's float64
product)."""
import numpy as np
import pytest

import workloads as W
from oracle import codecs, model as OM, w8a8 as O8
from tests.gpu_util import bf16_f64, rel_inf, say, u16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    import torch
    assert torch.cuda.is_available()
    from query_aware_prefill_amd import binding
    binding.load()
    return binding


def _dev(a):
    from query_aware_prefill_amd.device import to_device
    return to_device(a)


def _x(r, M, K):
    """bf16 activations with the rows the quantiser has to get right: a zero
    row, a row with -0 entries, a tiny and a huge row, single-spike rows."""
    x = W.draw_bf16(r, (M, K))
    if M >= 6:
        x[0] = 0
        x[1, ::3] = 0x8000                                                    # -0
        x[2] = W.draw_bf16(r, (K,), std=1e-30)
        x[3] = W.draw_bf16(r, (K,), std=1e30)
        x[4] = 0
        x[4, K // 2] = 0xC2F7                                                 # one -123.5
        x[5] = W.draw_bf16(r, (K,), std=0.02)
    return x


def _quant(B, x):
    import torch
    M, K = x.shape
    codes = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    scale = torch.empty(M, dtype=torch.float32, device="cuda")
    B.quail_act_quant_e4m3(_dev(x), codes, scale)
    torch.cuda.synchronize()
    return codes, scale


# one wave per row up to 4096 values; one workgroup per row up to 16384
# (4104, 9728); beyond that the one-wave kernel reads the row twice (16392)
@pytest.mark.parametrize("M,K", [(1, 8), (6, 64), (37, 2560), (9, 4096), (7, 4104), (11, 9728), (6, 16392)])
def test_act_quant_bit_exact(B, M, K):
    say("act quant", M, K)
    r = np.random.default_rng(M * 31 + K)
    x = _x(r, M, K)
    codes, scale = _quant(B, x)
    ref_c, ref_s = O8.act_quant_e4m3(codecs.bf16_value(x).astype(np.float32))
    got_c = codes.cpu().numpy()
    got_s = scale.cpu().numpy()
    bad = np.argwhere(got_c != ref_c)
    assert bad.size == 0, (bad[:5], got_c[tuple(bad[0])], ref_c[tuple(bad[0])])
    assert np.array_equal(got_s.view(np.uint32), ref_s.view(np.uint32))


def _weights(r, N, K):
    w = W.draw_fp8_codes(r, (N, K))
    s = W.bf16_bits_from_f32((0.0002 * (1 + r.random(N))).astype(np.float32))
    return w, s


def _gemm(B, codes, scale, w, s):
    import torch
    M, N = codes.shape[0], w.shape[0]
    y = torch.empty((M, N), dtype=torch.int16, device="cuda")
    B.quail_gemm_w8a8(codes, scale, _dev(w), _dev(s), y)
    torch.cuda.synchronize()
    return bf16_f64(u16(y))


def test_gemm_w8a8_decodes_every_code_exactly(B):
    """Activation codes = identity (code 0x38 = 1.0), scales 1: y[m][n] =
    decode(w[n][m]) exactly."""
    say("gemm w8a8 exact decode")
    M = K = 128
    N = 256
    w = (np.arange(N * K, dtype=np.uint32) % 256)
    w = np.where((w & 0x7F) == 0x7F, 0, w).astype(np.uint8).reshape(N, K)
    xc = np.zeros((M, K), np.uint8)
    xc[np.arange(M), np.arange(M)] = 0x38
    got = _gemm(B, _dev(xc), _dev(np.ones(M, np.float32)), w, np.full(N, 0x3F80, np.uint16))
    assert np.array_equal(got, codecs.e4m3_decode(w).T)


@pytest.mark.parametrize("M,N,K", [(1, 256, 128), (33, 256, 256), (257, 512, 384), (300, 768, 2560),
                                   (511, 1024, 1024)])
def test_gemm_w8a8_matches_oracle(B, M, N, K):
    say("gemm w8a8", M, N, K)
    r = np.random.default_rng(M * 7 + N + K + 1)
    x = _x(r, M, K)
    ref_c, ref_s = O8.act_quant_e4m3(codecs.bf16_value(x).astype(np.float32))
    codes, scale = _quant(B, x)
    assert np.array_equal(codes.cpu().numpy(), ref_c)
    w, s = _weights(r, N, K)
    got = _gemm(B, codes, scale, w, s)
    ref = codecs.bf16_round(O8.gemm_w8a8(ref_c, ref_s, w, s))
    # rows of very different magnitude: the measure is taken per row
    for m in range(M):
        if np.abs(ref[m]).max() == 0:
            assert not np.any(got[m])
            continue
        err = rel_inf(got[m], ref[m])
        assert err < 8e-3, (m, err)


@pytest.mark.parametrize("N,K", [(6144, 2560), (2560, 4096), (19456, 2560), (2560, 9728)])
def test_gemm_w8a8_qwen3_shapes_sampled_rows(B, N, K):
    """The four projection shapes of the Qwen3-4B layer at M = 4096 tokens;
    64 sampled rows against the oracle, and the W8A8 result within the
    activation-rounding bound of the W8A16 product of the same bf16 rows."""
    say("gemm w8a8 qwen3 shape", N, K)
    M = 4096
    r = np.random.default_rng(N + K + 2)
    x = W.draw_bf16(r, (M, K))
    codes, scale = _quant(B, x)
    w, s = _weights(r, N, K)
    got = _gemm(B, codes, scale, w, s)
    rows = np.sort(r.choice(M, 64, replace=False))
    xs = codecs.bf16_value(x[rows]).astype(np.float32)
    rc, rs = O8.act_quant_e4m3(xs)
    assert np.array_equal(codes.cpu().numpy()[rows], rc)
    ref = codecs.bf16_round(O8.gemm_w8a8(rc, rs, w, s))
    err = rel_inf(got[rows], ref)
    say("  rel err vs W8A8 oracle", err)
    assert err < 8e-3
    weff = OM.weight_eff(w, s)
    y16 = xs.astype(np.float64) @ weff.T
    bound = np.abs(O8.act_dequant(rc, rs) - xs) @ np.abs(weff).T
    # the oracle's bound plus the bf16 rounding of the output and fp32 sums
    assert np.all(np.abs(got[rows] - y16) <= bound + np.abs(y16) * 2.0 ** -8 + 1e-3 * np.abs(y16).max())
    say("  rel err vs W8A16 product", rel_inf(got[rows], y16))


def test_gemm_w8a8_many_tiles_ragged(B):
    """More tiles than one wave of workgroups and a ragged last token tile;
    sampled rows and the last 16 rows against the oracle."""
    M, N, K = 3000, 19456, 2560
    say("gemm w8a8 many tiles", M, N, K)
    r = np.random.default_rng(M + N + K)
    x = W.draw_bf16(r, (M, K))
    codes, scale = _quant(B, x)
    w, s = _weights(r, N, K)
    got = _gemm(B, codes, scale, w, s)
    rows = np.unique(np.concatenate([r.choice(M - 16, 48, replace=False), np.arange(M - 16, M)]))
    rc, rs = O8.act_quant_e4m3(codecs.bf16_value(x[rows]).astype(np.float32))
    ref = codecs.bf16_round(O8.gemm_w8a8(rc, rs, w, s))
    err = rel_inf(got[rows], ref)
    say("  rel err", err)
    assert err < 8e-3
