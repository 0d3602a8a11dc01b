"""Kernel-level parity: the HIP attention and GEMM against the CPU oracle,
called through the C ABI (wan_attention_fwd, wan_linear_fwd)."""
import numpy as np
import pytest

import oracle.wan_oracle as O
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


C_LOG2 = np.log2(np.e) / np.sqrt(128.0)   # the pre-scaled query's factor


def _attn_gpu(q, k, v, H, q_scaled=False):
    import video_diffusion_transformer_block_amd as W
    from tests.gpu_util import DEV
    B, Lq, D = q.shape
    Lk = k.shape[1]
    Lkp = (Lk + 63) // 64 * 64
    vt = np.zeros((D, B * Lkp), np.float32)
    for b in range(B):
        vt[:, b * Lkp:b * Lkp + Lk] = v[b].T
    tq = torch.from_numpy(q.reshape(B * Lq, D)).to(torch.bfloat16).to(DEV)
    tk = torch.from_numpy(k.reshape(B * Lk, D)).to(torch.bfloat16).to(DEV)
    tv = torch.from_numpy(vt).to(torch.bfloat16).to(DEV)
    to = torch.empty((B * Lq, D), dtype=torch.bfloat16, device=DEV)
    W.attention_fwd(tq, D, tk, D, tv, B * Lkp, Lkp, to, D, B, H, Lq, Lk, q_scaled=q_scaled)
    torch.cuda.synchronize()
    return to.float().cpu().numpy().reshape(B, Lq, D)


def _attn_oracle(q, k, v, H):
    return np.stack([O.multihead(q[b], k[b], v[b], H) for b in range(q.shape[0])])


CASES = [  # B, H, Lq, Lk
    (1, 1, 1, 1), (1, 2, 200, 64), (2, 2, 300, 100), (1, 3, 513, 257), (2, 1, 256, 600),
    (1, 2, 70, 4), (1, 1, 1000, 1000),
    # key-tile counts 2 .. 5 exercise every tail of the two-tile pipeline
    (1, 1, 64, 128), (1, 1, 96, 150), (1, 2, 100, 250), (1, 1, 40, 320),
]


@pytest.mark.parametrize("B,H,Lq,Lk", CASES)
def test_attention_stress(B, H, Lq, Lk):
    print(f"attention stress B={B} H={H} Lq={Lq} Lk={Lk}", flush=True)
    from tests.gpu_util import assert_parity
    q, k, v = synth.attention_inputs(1, B, H, Lq, Lk)
    g = _attn_gpu(q, k, v, H)
    o = _attn_oracle(q, k, v, H)
    assert_parity(g, o, 3e-2, 1e-2, f"attention {B},{H},{Lq},{Lk}")


def test_attention_rows_sum_to_one():
    """V = 1 -> O = 1 (probabilities normalised) on peaked logits."""
    print("attention V=1", flush=True)
    q, k, v = synth.attention_inputs(2, 1, 2, 300, 500, qk_std=3.0)
    g = _attn_gpu(q, k, np.ones_like(v), 2)
    assert np.max(np.abs(g - 1.0)) <= 4e-3


# a block of keys whose logits jump far above everything before it, so that
# the running max must be raised mid-stream (the kernel takes the first
# tile's max and raises it only when a probability passes 2^16): in the 2nd
# tile, in the steady-state loop, in the last ragged tile, and in the first
# tile (later tiles then sit far below the max)
OUTLIER_CASES = [  # Lq, Lk, first outlier key, last outlier key + 1
    (200, 150, 64, 100), (300, 600, 300, 340), (130, 600, 580, 600), (100, 500, 0, 20),
]


@pytest.mark.parametrize("q_scaled", [False, True])
@pytest.mark.parametrize("Lq,Lk,k0,k1", OUTLIER_CASES)
def test_attention_raises_running_max(Lq, Lk, k0, k1, q_scaled):
    print(f"attention outlier keys {k0}..{k1} of {Lk}, Lq={Lq}, q_scaled={q_scaled}", flush=True)
    from tests.gpu_util import assert_parity
    q, k, v = synth.attention_inputs(3, 1, 2, Lq, Lk)
    k[:, k0:k1] *= 4.0     # logits x4 (std 16): far past 2^16 in probability
    if q_scaled:           # the kernel reads q' = bf16(q c); the exact answer is that of q' / c
        q = synth.bf16_round(q * np.float32(C_LOG2))
        qo = q.astype(np.float64) / C_LOG2
    else:
        qo = q
    g = _attn_gpu(q, k, v, 2, q_scaled)
    o = _attn_oracle(qo, k, v, 2)
    assert_parity(g, o, 3e-2, 1e-2, f"attention outliers {k0}..{k1}")
    g1 = _attn_gpu(q, k, np.ones_like(v), 2, q_scaled)
    assert np.max(np.abs(g1 - 1.0)) <= 4e-3


@pytest.mark.parametrize("B,H,Lq,Lk", [(2, 2, 300, 100), (1, 1, 1000, 1000), (1, 2, 100, 250)])
def test_attention_prescaled_query(B, H, Lq, Lk):
    """q_scaled = 1: the query holds q log2(e)/sqrt(128), as the block's
    query projections write it."""
    print(f"attention pre-scaled q B={B} H={H} Lq={Lq} Lk={Lk}", flush=True)
    from tests.gpu_util import assert_parity
    q, k, v = synth.attention_inputs(4, B, H, Lq, Lk)
    qs = synth.bf16_round(q * np.float32(C_LOG2))
    g = _attn_gpu(qs, k, v, H, True)
    o = _attn_oracle(qs.astype(np.float64) / C_LOG2, k, v, H)
    assert_parity(g, o, 3e-2, 1e-2, f"attention pre-scaled {B},{H},{Lq},{Lk}")


@pytest.mark.parametrize("M,N,K", [(1, 64, 64), (77, 128, 64), (300, 256, 192), (513, 320, 64), (257, 512, 1280),
                                   (512, 1536, 1536)])
@pytest.mark.parametrize("mode", [0, 1, 2])
def test_linear(M, N, K, mode):
    print(f"linear M={M} N={N} K={K} mode={mode}", flush=True)
    import video_diffusion_transformer_block_amd as W
    from tests.gpu_util import DEV, assert_parity
    x, w, b = synth.linear_inputs(3, M, N, K)
    tx = torch.from_numpy(x).to(torch.bfloat16).to(DEV)
    tw = torch.from_numpy(w).to(torch.bfloat16).to(DEV)
    tb = torch.from_numpy(b).to(torch.bfloat16).to(DEV)
    ty = torch.empty((M, N), dtype=torch.float32 if mode == 1 else torch.bfloat16, device=DEV)
    W.linear_fwd(tx, tw, tb, ty, M, N, K, mode)
    torch.cuda.synchronize()
    ref = O.linear(x, w, b)
    if mode == 2:
        ref = O.gelu_tanh(ref)
    tol = 1e-4 if mode == 1 else 3e-2
    assert_parity(ty.float().cpu().numpy(), ref, tol, 1e-2 if mode != 1 else 1e-5, f"linear {mode}")


@pytest.mark.parametrize("B,L,d,branch", [(2, 300, 1536, 0), (1, 257, 1536, 1), (1, 77, 384, -1),
                                          (2, 50, 200, 0)])
def test_ln_modulate(B, L, d, branch):
    """wan_ln_modulate_fwd: LayerNorm (+ the block's modulation of one branch)
    to bf16, against the oracle's layer_norm / modulate; d = 200 takes the
    generic kernel."""
    print(f"ln_modulate B={B} L={L} d={d} branch={branch}", flush=True)
    import video_diffusion_transformer_block_amd as W
    from tests.gpu_util import DEV, assert_parity
    g = np.random.default_rng([B, L, d])
    x = (g.standard_normal((B, L, d)) * 1.5 + 0.3).astype(np.float32)
    mod = (g.standard_normal((B, 6 * d)) * 0.3).astype(np.float32)
    tx, tm = torch.from_numpy(x).to(DEV), torch.from_numpy(mod).to(DEV)
    h = torch.empty((B * L, d), dtype=torch.bfloat16, device=DEV)
    W.ln_modulate_fwd(tx, B, L, d, tm if branch >= 0 else None, branch, 1e-6, h)
    torch.cuda.synchronize()
    ref = O.layer_norm(x, 1e-6)
    if branch >= 0:
        sh, sc = (0, d) if branch == 0 else (3 * d, 4 * d)
        ref = np.stack([O.modulate(ref[b], mod[b, sh:sh + d], mod[b, sc:sc + d]) for b in range(B)])
    assert_parity(h.float().cpu().numpy().reshape(B, L, d), ref, 3e-2, 1e-2, "ln_modulate")
