"""GPU test of qlora_linear_fwd_noalloc, the decode-path forward (M <= 16)
that allocates nothing: it must give the same bits as qlora_linear_fwd (the
same kernels on a caller workspace), on two calls in a row, the second with
a smaller input (the library-held scratch keeps the first call's contents),
and stay within 2e-2 of the float64 oracle. Run alone in a fresh process and
after the other GPU tests.
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


def one_call(api, K, N, M, r, seed):
    import torch

    rng = np.random.default_rng(seed)
    inp = workloads.draw_linear(rng, workloads.LinearShape("t", K, N), M, r, 0.25, "normal", 0.02, False)
    q, _ = gpu_quantize(api, inp.W)
    X, L1, L2 = (api.to_device_bf16(a) for a in (inp.X, inp.L1, inp.L2))
    Y_ref, T_ref = api.qlora_linear_fwd(q, X, L1, L2, inp.s, want_T=True)
    Y = torch.full((M, N), 7.0, dtype=torch.bfloat16, device="cuda")
    T = torch.full((M, r), 7.0, dtype=torch.bfloat16, device="cuda")
    api.qlora_linear_fwd_noalloc(q, X, L1, L2, inp.s, Y, T)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(api.to_host_bits(Y), api.to_host_bits(Y_ref))
    np.testing.assert_array_equal(api.to_host_bits(T), api.to_host_bits(T_ref))
    Wd = nf4.dequantize(nf4.quantize(inp.W), inp.W.shape)
    R, _ = linear.linear_fwd(inp.X, Wd, inp.L1, inp.L2, inp.s)
    err = linear.rel_err(api.to_host_bits(Y), R)
    say(f"  noalloc K={K} N={N} M={M} r={r}: bit-equal to qlora_linear_fwd, err {err:.5f}")
    assert err <= TOL


def test_noalloc_matches_workspace_forward_twice(api):
    say("qlora_linear_fwd_noalloc: two calls, the second smaller")
    one_call(api, 11008, 4096, 16, 256, 1)     # the largest scratch of this test
    one_call(api, 1024, 520, 3, 16, 2)         # smaller: stale scratch contents from the first call


def test_noalloc_llama_shapes(api):
    say("qlora_linear_fwd_noalloc: LLaMA-7B decode shapes")
    for K, N in ((4096, 11008), (11008, 4096)):
        for M in (1, 4, 16):
            one_call(api, K, N, M, 64, K + M)


def test_noalloc_refuses_m_above_16(api):
    """M > 16 is refused on the host (QLORA_ERR_SHAPE) before any launch.
    Shapes whose scratch exceeds the library's array are refused on the
    host too; tests/test_abi.py checks that without a GPU (it needs no
    device buffers, and no call here passes buffers smaller than a shape
    the library would accept)."""
    import torch

    inp = workloads.draw_linear(np.random.default_rng(3), workloads.LinearShape("t", 512, 256), 32, 8, 0.5,
                                "normal", 0.02, False)
    q, _ = gpu_quantize(api, inp.W)
    X, L1, L2 = (api.to_device_bf16(a) for a in (inp.X, inp.L1, inp.L2))
    Y = torch.empty((32, 256), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(api.QLoRAError) as ei:
        api.qlora_linear_fwd_noalloc(q, X, L1, L2, inp.s, Y)      # M = 32 > 16
    assert ei.value.status == api.QLORA_ERR_SHAPE
