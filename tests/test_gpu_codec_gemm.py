"""GPU parity: the E4M3 codec of the fp8 KV writer (bit-exact, exhaustive) and
the W8A16 GEMM (exact decode; fp32-accumulated products against the oracle)."""
import numpy as np
import pytest

import workloads as W
from oracle import codecs, model as OM
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


def test_fp8_decode_all_codes(B):
    import torch
    say("fp8 decode: 256 codes")
    codes = np.arange(256, dtype=np.uint8)
    out = torch.empty(256, dtype=torch.float32, device="cuda")
    B.quail_fp8_e4m3_decode(_dev(codes), 1.0, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    ref = codecs.e4m3_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


@pytest.mark.parametrize("scale", [1.0, 2.0, 0.25])
def test_fp8_encode_all_bf16_patterns(B, scale):
    import torch
    say("fp8 encode: 65536 bf16 patterns, scale", scale)
    bits = np.arange(1 << 16, dtype=np.uint32)
    x = (bits << 16).view(np.float32)
    x = x[~np.isnan(x)].copy()
    codes = torch.empty(x.size, dtype=torch.uint8, device="cuda")
    B.quail_fp8_e4m3_encode(torch.from_numpy(x).cuda(), scale, codes)
    torch.cuda.synchronize()
    got = codes.cpu().numpy()
    ref = codecs.e4m3_encode(x.astype(np.float64) / scale)
    assert np.array_equal(got, ref), np.flatnonzero(got != ref)[:10]


def test_gemm_decodes_every_code_exactly(B):
    """x = identity, scale = 1: y[m][n] = decode(w[n][m]) exactly."""
    import torch
    say("gemm exact decode")
    K = M = 64
    N = 256
    codes = np.arange(N * K, dtype=np.uint32) % 256
    codes = np.where((codes & 0x7F) == 0x7F, 0, codes).astype(np.uint8).reshape(N, K)
    x = np.zeros((M, K), np.uint16)
    x[np.arange(64), np.arange(64)] = 0x3F80
    scale = np.full(N, 0x3F80, np.uint16)
    y = torch.empty((M, N), dtype=torch.int16, device="cuda")
    B.quail_gemm_w8a16(_dev(x), _dev(codes), _dev(scale), y)
    torch.cuda.synchronize()
    got = bf16_f64(u16(y))
    ref = codecs.e4m3_decode(codes).T
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("M,N,K", [(1, 128, 64), (33, 128, 128), (257, 256, 192), (300, 384, 2560),
                                   (511, 1024, 1024)])
def test_gemm_matches_oracle(B, M, N, K):
    import torch
    say("gemm", M, N, K)
    r = np.random.default_rng(M * 7 + N + K)
    x = W.draw_bf16(r, (M, K))
    w = W.draw_fp8_codes(r, (N, K))
    s = W.bf16_bits_from_f32((0.0002 * (1 + r.random(N))).astype(np.float32))
    y = torch.empty((M, N), dtype=torch.int16, device="cuda")
    B.quail_gemm_w8a16(_dev(x), _dev(w), _dev(s), y)
    torch.cuda.synchronize()
    ref = codecs.bf16_round(codecs.bf16_value(x) @ OM.weight_eff(w, s).T)
    err = rel_inf(bf16_f64(u16(y)), ref)
    say("  rel err", err)
    assert err < 2e-2
    assert err < 8e-3   # one bf16 rounding plus fp32 accumulation, in practice


@pytest.mark.parametrize("N,K", [(6144, 2560), (2560, 4096), (19456, 2560), (2560, 9728)])
def test_gemm_qwen3_shapes_sampled_rows(B, N, K):
    """The four projection shapes of the Qwen3-4B layer at M = 4096 tokens;
    64 sampled rows are checked against the oracle."""
    import torch
    say("gemm qwen3 shape", N, K)
    M = 4096
    r = np.random.default_rng(N + K)
    x = W.draw_bf16(r, (M, K))
    w = W.draw_fp8_codes(r, (N, K))
    s = W.bf16_bits_from_f32((0.0002 * (1 + r.random(N))).astype(np.float32))
    y = torch.empty((M, N), dtype=torch.int16, device="cuda")
    B.quail_gemm_w8a16(_dev(x), _dev(w), _dev(s), y)
    torch.cuda.synchronize()
    rows = np.sort(r.choice(M, 64, replace=False))
    ref = codecs.bf16_round(codecs.bf16_value(x[rows]) @ OM.weight_eff(w, s).T)
    err = rel_inf(bf16_f64(u16(y)[rows]), ref)
    say("  rel err", err)
    assert err < 8e-3


@pytest.mark.parametrize("N,K,M", [(19456, 2560, 3000), (2560, 9728, 8200)])
def test_gemm_many_tiles_per_workgroup_ragged(B, N, K, M):
    """More output tiles than workgroups (each workgroup runs several tiles in
    a row) with a ragged last token tile; sampled rows and the last 16 rows
    are checked against the oracle."""
    import torch
    say("gemm many tiles", M, N, K)
    r = np.random.default_rng(M + N + K)
    x = W.draw_bf16(r, (M, K))
    w = W.draw_fp8_codes(r, (N, K))
    s = W.bf16_bits_from_f32((0.0002 * (1 + r.random(N))).astype(np.float32))
    y = torch.empty((M, N), dtype=torch.int16, device="cuda")
    B.quail_gemm_w8a16(_dev(x), _dev(w), _dev(s), y)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([r.choice(M - 16, 48, replace=False), np.arange(M - 16, M)]))
    ref = codecs.bf16_round(codecs.bf16_value(x[rows]) @ OM.weight_eff(w, s).T)
    err = rel_inf(bf16_f64(u16(y)[rows]), ref)
    say("  rel err", err)
    assert err < 8e-3
