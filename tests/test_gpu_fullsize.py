"""GPU parity at the benchmark's full sizes, in the launch configuration the
benchmark times: 8192 tokens through LLaMA-7B-shaped linears (normal weights
with 0.1 % outliers x10), a LLaMA-33B-shaped linear with Student-t weights,
and the decode-style GEMV at M in {1, 4, 16}.

The oracle checks sampled rows of Y and dX (row m of either depends on row m
of the input only) and the full adapter gradients dL1 and dL2 (float64).
"""

import numpy as np
import pytest

from bit_nf4_quantized_amd import workloads
from oracle import linear, nf4
from gpu_util import gpu_quantize, require_gpu, say

pytestmark = pytest.mark.gpu
TOL = 2e-2


@pytest.fixture(scope="module")
def api():
    return require_gpu()


def report(label, k, G, R):
    err = linear.rel_err(G, R)
    say(f"  {label} {k}: err {err:.5f}")
    assert err <= TOL, (label, k, err)


@pytest.mark.parametrize("name,index", [("llama7b-layer", 0), ("llama7b-layer", 4), ("llama7b-layer", 6),
                                        ("llama33b-layer", 4)])
def test_layer_linear_full_size(api, name, index):
    import torch

    shp, inp = workloads.layer_linear(name, index)
    M = inp.X.shape[0]
    say(f"full-size {name} {shp.name}: M={M} K={shp.K} N={shp.N}")
    q, _ = gpu_quantize(api, inp.W)
    X, L1, L2, dY = (api.to_device_bf16(a) for a in (inp.X, inp.L1, inp.L2, inp.dY))
    Y, T = api.qlora_linear_fwd(q, X, L1, L2, inp.s, want_T=True)
    dX, dL1, dL2 = api.qlora_linear_bwd(q, X, dY, L1, L2, inp.s, T=T)
    torch.cuda.synchronize()
    Wd = nf4.dequantize(nf4.quantize(inp.W), inp.W.shape)
    rows = np.sort(np.random.default_rng(index).choice(M, 48, replace=False))
    Yr = linear.linear_fwd_rows(inp.X, Wd, inp.L1, inp.L2, inp.s, rows)
    report(shp.name, "Y rows", api.to_host_bits(Y[rows.tolist()]), Yr)
    dXr = linear.linear_bwd_dx_rows(Wd, inp.L1, inp.L2, inp.s, inp.dY, rows)
    report(shp.name, "dX rows", api.to_host_bits(dX[rows.tolist()]), dXr)
    Xf, dYf = linear.widen(inp.X), linear.widen(inp.dY)
    L1f, L2f = linear.widen(inp.L1), linear.widen(inp.L2)
    U = dYf @ L2f.T
    report(shp.name, "dL1", dL1.cpu().numpy(), inp.s * (Xf.T @ U))
    report(shp.name, "dL2", dL2.cpu().numpy(), inp.s * ((Xf @ L1f).T @ dYf))


@pytest.mark.parametrize("K,N", [(4096, 11008), (11008, 4096)])
@pytest.mark.parametrize("M", [1, 4, 16])
def test_gemv_full_size(api, K, N, M):
    import torch

    say(f"gemv full size K={K} N={N} M={M}")
    inp = workloads.gemv_inputs(K, N, M)
    q, _ = gpu_quantize(api, inp.W)
    X, L1, L2 = (api.to_device_bf16(a) for a in (inp.X, inp.L1, inp.L2))
    Y, _ = api.qlora_linear_fwd(q, X, L1, L2, inp.s)
    torch.cuda.synchronize()
    Wd = nf4.dequantize(nf4.quantize(inp.W), inp.W.shape)
    R, _ = linear.linear_fwd(inp.X, Wd, inp.L1, inp.L2, inp.s)
    report(f"gemv {K}->{N} M={M}", "Y", api.to_host_bits(Y), R)
