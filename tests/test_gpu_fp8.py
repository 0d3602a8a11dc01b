"""FP8 GEMM through the C ABI against the CPU oracle's E4M3 emulation:
quantisation codes and scales bit for bit (the codes are integers decided
in float32 on both sides), the GEMM in its three output modes over ragged
shapes and K of 1, 2, 3 and 24 tiles, and sampled rows at the full FFN
up-projection shape."""
import numpy as np
import pytest

import oracle.wan_oracle as O
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _bf16(a):
    return synth.bf16_round(np.asarray(a, np.float32))


def _decode(q):
    """E4M3 bytes (torch uint8 on the device) -> float64 numpy."""
    return q.cpu().view(torch.float8_e4m3fn).to(torch.float64).numpy()


# Accumulation bound of the FP8 GEMM, relative to the sum of |products|: the
# E4M3 products are exact; one v_mfma_scale_f32_32x32x64_f8f6f4 sums its 64
# products to about 2^-15 of their absolute sum (measured on the chip: at most
# 2.9e-5 over 600k outputs), bounded here by 2^-13; the float32 accumulation
# across the K/64 instructions adds at most K 2^-24.
def _rel_bound(K):
    return 2.0 ** -13 + K * 2.0 ** -24


def _acc_bound(x, w, K):
    qx, sx = O.quantize_rows_fp8(x)
    qw, sw = O.quantize_tensor_fp8(w)
    return _rel_bound(K) * (np.abs(qx) @ np.abs(qw).T) * sx[:, None] * sw + 1e-7


def _quant_rows(x_np):
    import video_diffusion_transformer_block_amd as W
    M, K = x_np.shape
    x = torch.from_numpy(x_np).to(torch.bfloat16).cuda()
    q = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    s = torch.empty(M, dtype=torch.float32, device="cuda")
    W.quantize_rows_fp8(x, q, s)
    return q, s


def _quant_tensor(w_np):
    import video_diffusion_transformer_block_amd as W
    w = torch.from_numpy(w_np).to(torch.bfloat16).cuda()
    q = torch.empty(w.shape, dtype=torch.uint8, device="cuda")
    s = torch.empty(1, dtype=torch.float32, device="cuda")
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    W.quantize_tensor_fp8(w, q, s, ws)
    return q, s


def test_quantize_rows_and_tensor_bit_exact():
    print("fp8 quantisation", flush=True)
    rng = np.random.default_rng(60)
    x = _bf16(rng.standard_normal((300, 1536)) * np.exp(rng.uniform(-6, 6, (300, 1)))).astype(np.float32)
    x[7] = 0.0
    q, s = _quant_rows(x)
    torch.cuda.synchronize()
    qo, so = O.quantize_rows_fp8(x)
    assert np.array_equal(_decode(q), qo), "per-token codes"
    assert np.array_equal(s.cpu().numpy().astype(np.float64), so), "per-token scales"
    w = _bf16(rng.standard_normal((640, 1536)) * 0.02).astype(np.float32)
    qw, sw = _quant_tensor(w)
    torch.cuda.synchronize()
    qwo, swo = O.quantize_tensor_fp8(w)
    assert np.array_equal(_decode(qw), qwo), "per-tensor codes"
    assert float(sw.cpu()[0]) == swo, "per-tensor scale"


@pytest.mark.parametrize("M,N,K", [(300, 640, 1536), (1, 256, 64), (257, 300, 128), (513, 512, 192)])
@pytest.mark.parametrize("mode", [0, 1, 2])
def test_linear_fp8_vs_oracle(M, N, K, mode):
    import video_diffusion_transformer_block_amd as W
    from tests.gpu_util import assert_parity
    print(f"fp8 linear M={M} N={N} K={K} mode={mode}", flush=True)
    rng = np.random.default_rng(61 + M + N + K + mode)
    x = _bf16(rng.standard_normal((M, K))).astype(np.float32)
    w = _bf16(rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    b = _bf16(rng.standard_normal(N) * 0.02).astype(np.float32)
    qx, sx = _quant_rows(x)
    qw, sw = _quant_tensor(w)
    y = torch.empty((M, N), dtype=torch.float32 if mode == 1 else torch.bfloat16, device="cuda")
    bd = torch.from_numpy(b).to(torch.bfloat16).cuda()
    W.linear_fp8_fwd(qx, sx, qw, sw, bd, y, M, N, K, mode)
    torch.cuda.synchronize()
    g = y.float().cpu().numpy()
    o = O.linear_fp8(x, w, b)
    if mode == 2:
        o = O.gelu_tanh(o)
    if mode == 1:     # float32 output: only the float32 accumulation order differs
        excess = np.abs(g - o) - _acc_bound(x, w, K)
        assert np.max(excess) <= 0, np.max(np.abs(g - o))
    else:             # bf16 output rounding
        assert_parity(g, o, 1e-2, 4e-3, f"fp8 linear mode {mode}")


def test_linear_fp8_full_ffn_shape_sampled_rows():
    """The FFN up-projection of the 1.3B block (M = 32760, N = 8960, K = 1536):
    the whole GEMM on the GPU, 64 sampled rows in the oracle (per-token scales
    make rows independent)."""
    import video_diffusion_transformer_block_amd as W
    M, N, K = 32760, 8960, 1536
    print(f"fp8 linear full FFN shape {M}x{N}x{K}", flush=True)
    g = torch.Generator(device="cpu").manual_seed(62)
    x = torch.randn((M, K), generator=g).to(torch.bfloat16)
    w = (torch.randn((N, K), generator=g) * 0.02).to(torch.bfloat16)
    b = (torch.randn(N, generator=g) * 0.02).to(torch.bfloat16)
    xd, wd, bd = x.cuda(), w.cuda(), b.cuda()
    qx = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    sx = torch.empty(M, dtype=torch.float32, device="cuda")
    W.quantize_rows_fp8(xd, qx, sx)
    qw = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    sw = torch.empty(1, dtype=torch.float32, device="cuda")
    W.quantize_tensor_fp8(wd, qw, sw, torch.empty(256, dtype=torch.uint8, device="cuda"))
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    W.linear_fp8_fwd(qx, sx, qw, sw, bd, y, M, N, K, 1)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(63).choice(M, 64, replace=False))
    rows[-1] = M - 1
    xs = x[rows].float().numpy()
    wf = w.float().numpy()
    qwo, swo = O.quantize_tensor_fp8(wf)
    qxo, sxo = O.quantize_rows_fp8(xs)
    o = (qxo @ qwo.T) * sxo[:, None] * swo + b.float().numpy()[None, :]
    gs = y[torch.from_numpy(rows).cuda()].cpu().numpy()
    bound = _rel_bound(K) * (np.abs(qxo) @ np.abs(qwo).T) * sxo[:, None] * swo + 1e-7
    assert np.max(np.abs(gs - o) - bound) <= 0, np.max(np.abs(gs - o))
