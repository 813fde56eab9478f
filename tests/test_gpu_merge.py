"""GPU parity of the adapter merge (qlora_merge_adapters) against the oracle
(oracle/merge.py).

The merged weight is bf16(Wd + s (L1 L2)^T). The GPU sums the rank-r
product in fp32 on MFMA, so it is not bit-exact; every element must lie
within half a bf16 ulp of the float64 value plus the fp32 error bound of
that sum (2 r 2^-24 sum_j |L1 L2| s, and one fp32 rounding each of s D and
of the addition), and at least 99.9 % of the elements must equal the
oracle's correctly rounded value. With zero adapters the merge must equal
the standalone dequantisation bit for bit, and the forward product through
the merged weight must match the layer within 2e-2. Shapes cover ragged
tiles (N not a multiple of 32, K not of 256, r not of 32), r = 256, the
other data types and no double quantisation, and a full LLaMA-7B MLP weight
(11008 x 4096, r = 64) on sampled rows.
"""

import numpy as np
import pytest

from bit_nf4_quantized_amd import workloads
from oracle import linear, merge, nf4, qtypes
from gpu_util import gpu_quantize, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    return require_gpu()


def bf16_ulp(bits):
    e = (bits.astype(np.int64) >> 7) & 0xFF
    return np.ldexp(1.0, np.maximum(e, 1) - 127 - 7)


def check_merged(got_bits, Wd_bits, L1, L2, s, r):
    exact = merge.merge_exact(Wd_bits, L1, L2, s)
    got = nf4.bf16_bits_to_f32(got_bits).astype(np.float64)
    absprod = np.abs(linear.widen(L1)) @ np.abs(linear.widen(L2))
    t = abs(s) * (linear.widen(L1) @ linear.widen(L2)).T
    eps = abs(s) * 2 * r * 2.0 ** -24 * absprod.T + 2.0 ** -24 * (np.abs(t) + np.abs(exact)) * 1.01
    bound = 0.5 * bf16_ulp(got_bits) + eps
    bad = np.abs(got - exact) > bound
    assert not bad.any(), (np.argwhere(bad)[:5], got[bad][:5], exact[bad][:5])
    same = np.mean(got_bits == merge.merge(Wd_bits, L1, L2, s))
    say(f"  merged: {100 * same:.4f} % equal to the correctly rounded value")
    assert same >= 0.999


def draw(rng, N, K, r, wstd=0.02, astd=0.01):
    W = workloads.random_weight(rng, N * K, "normal", wstd).reshape(N, K)
    L1 = workloads.to_bf16_bits(astd * rng.standard_normal((K, r)).astype(np.float32))
    L2 = workloads.to_bf16_bits(astd * rng.standard_normal((r, N)).astype(np.float32))
    return W, L1, L2


@pytest.mark.parametrize("N,K,r,s,name,dq", [
    (64, 256, 8, 2.0, "nf4", True),
    (40, 320, 24, 0.5, "nf4", True),        # ragged tiles in n and k; r not a multiple of 32
    (96, 1024, 256, 0.25, "nf4", True),     # largest rank
    (72, 576, 64, 1.0, "nf4", False),       # no double quantisation
    (32, 512, 16, 1.0, "int4", True),
    (48, 448, 40, 1.0, "fp4_e2m1", True),
])
def test_merge(api, N, K, r, s, name, dq):
    import torch

    say(f"merge {N}x{K} r={r} s={s} {name} dq={dq}")
    rng = np.random.default_rng(N * 7 + K + r)
    W, L1, L2 = draw(rng, N, K, r, astd=0.05)
    tab = qtypes.codebook(name)
    q, _ = gpu_quantize(api, W, qtype=name, double_quant=dq)
    M = api.qlora_merge_adapters(q, api.to_device_bf16(L1), api.to_device_bf16(L2), s)
    torch.cuda.synchronize()
    Wd = nf4.dequantize(nf4.quantize(W, tab, double_quant=dq), (N, K), tab)
    check_merged(api.to_host_bits(M), Wd, L1, L2, s, r)


def test_merge_zero_adapters_is_the_dequantisation(api):
    import torch

    say("merge with zero adapters")
    rng = np.random.default_rng(3)
    W, L1, L2 = draw(rng, 80, 640, 16)
    q, _ = gpu_quantize(api, W)
    M = api.qlora_merge_adapters(q, api.to_device_bf16(np.zeros_like(L1)), api.to_device_bf16(L2), 3.0)
    M0 = api.qlora_merge_adapters(q, api.to_device_bf16(L1), api.to_device_bf16(L2), 0.0)
    D = api.qlora_dequantize(q)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(api.to_host_bits(M), api.to_host_bits(D))
    np.testing.assert_array_equal(api.to_host_bits(M0), nf4.dequantize(nf4.quantize(W), W.shape))


def test_forward_through_merged_weight_matches_the_layer(api):
    import torch

    say("forward through the merged weight, 64 tokens, 256 -> 512, r = 32")
    rng = np.random.default_rng(4)
    inp = workloads.draw_linear(rng, workloads.LinearShape("t", 256, 512), 64, 32, 0.5, "normal", 0.02, False)
    q, _ = gpu_quantize(api, inp.W)
    L1, L2, X = (api.to_device_bf16(a) for a in (inp.L1, inp.L2, inp.X))
    M = api.qlora_merge_adapters(q, L1, L2, inp.s)
    Yl, _ = api.qlora_linear_fwd(q, X, L1, L2, inp.s)
    Ym = (X.float() @ M.float().t()).to(torch.bfloat16)
    torch.cuda.synchronize()
    Wd = nf4.dequantize(nf4.quantize(inp.W), inp.W.shape)
    R, _ = linear.linear_fwd(inp.X, Wd, inp.L1, inp.L2, inp.s)
    for label, Y in (("merged", Ym), ("layer", Yl)):
        err = linear.rel_err(api.to_host_bits(Y), R)
        say(f"  {label} Y: err {err:.5f}")
        assert err <= 2e-2


def test_merge_full_size_sampled_rows(api):
    import torch

    N, K, r, s = 11008, 4096, 64, 0.25
    say(f"merge full size {N}x{K} r={r}")
    rng = np.random.default_rng(11)
    W, L1, L2 = draw(rng, N, K, r)
    q, _ = gpu_quantize(api, W)
    M = api.qlora_merge_adapters(q, api.to_device_bf16(L1), api.to_device_bf16(L2), s)
    torch.cuda.synchronize()
    rows = np.sort(rng.choice(N, 64, replace=False))
    rows[-1] = N - 1
    qt = nf4.quantize(W)
    Wd = nf4.dequantize(qt, (N, K))[rows]
    check_merged(api.to_host_bits(M[rows.tolist()]), Wd, L1, L2[:, rows], s, r)
