"""GPU parity of LoRA dropout against the oracle (oracle/dropout.py).

The dropped adapter input (mask and scaling) is unique, so qlora_lora_dropout
must equal the oracle bit for bit, for several probabilities, seeds (64-bit
included) and sizes. The layer with dropout is compared like the plain
layer (max|G - R| / RMS(R) <= 2e-2 against the float64 oracle with the same
mask) on every forward path (GEMV, batched decode, large M) and both dX
paths (the GEMM with an fp32 addend, and the fp32 main product combined
with the masked term), with recomputed and passed T, bf16 gradients, and a
LLaMA-7B linear at 8192 tokens (whole outputs). With p = 0 the forward and
the adapter gradients equal the layer without dropout bit for bit.
"""

import numpy as np
import pytest

from bit_nf4_quantized_amd import workloads
from oracle import dropout, linear, nf4
from gpu_util import check_output, gpu_quantize, require_gpu, say

pytestmark = pytest.mark.gpu
TOL = 2e-2


@pytest.fixture(scope="module")
def api():
    return require_gpu()


@pytest.mark.parametrize("p,seed,M,K", [
    (0.1, 1, 64, 512),
    (0.05, 0xDEADBEEFCAFEF00D, 33, 1024),   # 64-bit seed: both key words
    (0.5, 7, 8, 64),
    (0.0, 3, 16, 128),
    (0.9, 2 ** 40 + 5, 200, 448),
])
def test_dropped_input_bit_exact(api, p, seed, M, K):
    import torch

    say(f"dropout input p={p} seed={seed} {M}x{K}")
    rng = np.random.default_rng(M + K)
    X = workloads.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    Xd = api.qlora_lora_dropout(api.to_device_bf16(X), p, seed)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(api.to_host_bits(Xd), dropout.drop_input(X, p, seed))


def run(api, inp, p, seed, need_bwd=True, use_T=True, grad_dtype=None):
    import torch

    q, _ = gpu_quantize(api, inp.W)
    X, L1, L2 = (api.to_device_bf16(a) for a in (inp.X, inp.L1, inp.L2))
    Y, T = api.qlora_linear_fwd(q, X, L1, L2, inp.s, want_T=True, dropout=(p, seed))
    out = {"Y": api.to_host_bits(Y), "T": api.to_host_bits(T)}
    if need_bwd:
        dY = api.to_device_bf16(inp.dY)
        dX, dL1, dL2 = api.qlora_linear_bwd(q, X, dY, L1, L2, inp.s, T=T if use_T else None,
                                            grad_dtype=grad_dtype, dropout=(p, seed))
        torch.cuda.synchronize()
        out.update(dX=api.to_host_bits(dX), dL1=dL1.float().cpu().numpy(), dL2=dL2.float().cpu().numpy())
    return out


def oracle(inp, p, seed, need_bwd=True):
    Wd = nf4.dequantize(nf4.quantize(inp.W), inp.W.shape)
    Y, T = dropout.linear_fwd(inp.X, Wd, inp.L1, inp.L2, inp.s, p, seed)
    ref = {"Y": Y, "T": T}
    if need_bwd:
        dX, dL1, dL2 = dropout.linear_bwd(inp.X, Wd, inp.L1, inp.L2, inp.s, inp.dY, p, seed)
        ref.update(dX=dX, dL1=dL1, dL2=dL2)
    return ref


def compare(got, ref, label):
    for k, R in ref.items():
        check_output(label, k, got[k], R)


@pytest.mark.parametrize("M,K,N,r,p", [
    (200, 320, 192, 16, 0.1),     # large M, dX GEMM with the fp32 addend (N % 64 == 0)
    (200, 320, 136, 16, 0.05),    # large M, ragged N: fp32 main product + masked combine
    (8, 1024, 520, 64, 0.1),      # GEMV forward, small-M backward
    (64, 512, 256, 64, 0.1),      # batched-decode forward, GEMM dX
    (130, 448, 328, 72, 0.3),     # rank above 64: generic adapter products
    (130, 256, 64 * 193, 16, 0.1),  # dX GEMM with the fp32 addend over N >= 12288 (three B buffers)
])
def test_linear_with_dropout(api, M, K, N, r, p):
    say(f"dropout linear M={M} K={K} N={N} r={r} p={p}")
    rng = np.random.default_rng(M * 3 + K + N)
    inp = workloads.draw_linear(rng, workloads.LinearShape("t", K, N), M, r, 0.5, "normal", 0.02, True)
    seed = 1000 + M
    ref = oracle(inp, p, seed)
    compare(run(api, inp, p, seed), ref, f"{M}x{K}x{N}")
    compare(run(api, inp, p, seed, use_T=False), ref, f"{M}x{K}x{N} recomputed T")


def test_bf16_gradients_with_dropout(api):
    import torch

    say("dropout linear, bf16 adapter gradients")
    rng = np.random.default_rng(5)
    inp = workloads.draw_linear(rng, workloads.LinearShape("t", 256, 192), 96, 16, 0.5, "normal", 0.02, True)
    ref = oracle(inp, 0.1, 77)
    got = run(api, inp, 0.1, 77, grad_dtype=torch.bfloat16)
    compare(got, ref, "bf16 grads")


def test_p_zero_matches_the_plain_layer(api):
    import torch

    say("dropout p = 0 against the plain layer")
    rng = np.random.default_rng(6)
    inp = workloads.draw_linear(rng, workloads.LinearShape("t", 256, 192), 96, 16, 0.5, "normal", 0.02, True)
    q, _ = gpu_quantize(api, inp.W)
    X, L1, L2, dY = (api.to_device_bf16(a) for a in (inp.X, inp.L1, inp.L2, inp.dY))
    Y0, T0 = api.qlora_linear_fwd(q, X, L1, L2, inp.s, want_T=True)
    Y1, T1 = api.qlora_linear_fwd(q, X, L1, L2, inp.s, want_T=True, dropout=(0.0, 123))
    _, a1, a2 = api.qlora_linear_bwd(q, X, dY, L1, L2, inp.s, T=T0)
    dX1, b1, b2 = api.qlora_linear_bwd(q, X, dY, L1, L2, inp.s, T=T1, dropout=(0.0, 123))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(api.to_host_bits(Y0), api.to_host_bits(Y1))
    np.testing.assert_array_equal(api.to_host_bits(T0), api.to_host_bits(T1))
    np.testing.assert_array_equal(a1.cpu().numpy(), b1.cpu().numpy())
    np.testing.assert_array_equal(a2.cpu().numpy(), b2.cpu().numpy())
    Wd = nf4.dequantize(nf4.quantize(inp.W), inp.W.shape)
    dXr, _, _ = linear.linear_bwd(inp.X, Wd, inp.L1, inp.L2, inp.s, inp.dY)
    check_output("p = 0", "dX", api.to_host_bits(dX1), dXr)


def test_dropout_full_size(api):
    """A LLaMA-7B linear at 8192 tokens with p = 0.1: every output whole
    against oracle.dropout (same mask, float64)."""
    shp, inp = workloads.layer_linear("llama7b-layer", 0)
    p, seed = 0.1, 2024
    say(f"dropout full size {shp.name}: M={inp.X.shape[0]} K={shp.K} N={shp.N} p={p}")
    got = run(api, inp, p, seed)
    compare(got, oracle(inp, p, seed), f"full-size {shp.name}")
