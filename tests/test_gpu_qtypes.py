"""GPU parity of the alternative 4-bit data types (Int4, FP4 E2M1, FP4 E3M0).

The library's quantiser, dequantiser, linear forward/backward and small-M
GEMV are table-driven; these tests run them with the three other 4-bit
tables that the pages compare with NF4 (diycv.top, section 实验设置与主要结果
item 1) and compare with the oracle (oracle/qtypes.py) on the same seeded
inputs: codes, DQ constants and dequantised bf16 bit for bit, linear outputs
and gradients within 2e-2 of the fp64 oracle normalised by the output RMS.
"""

import numpy as np
import pytest

from bit_nf4_quantized_amd import workloads
from oracle import linear, nf4, qtypes
from gpu_util import assert_quant_equal, check_output, gpu_quantize, require_gpu, say

pytestmark = pytest.mark.gpu
TOL = 2e-2
TYPES = ["int4", "fp4_e2m1", "fp4_e3m0"]


@pytest.fixture(scope="module")
def api():
    return require_gpu()


def oracle_quant(W, name):
    qt = nf4.quantize(W, qtypes.codebook(name))
    return {"codes": qt["codes"], "absmax8": qt["absmax8"], "scale2": qt["scale2"], "mean": qt["mean"]}, qt


@pytest.mark.parametrize("name", TYPES)
@pytest.mark.parametrize("rows,cols,kind,bf16", [
    (300, 211, "normal", False),        # ragged: short last block and group
    (512, 512, "student-t4", True),     # bf16 input
    (64, 1024, "normal", False),
])
def test_quantize_dequantize_bit_exact(api, name, rows, cols, kind, bf16):
    import torch

    say(f"{name} quantize {rows}x{cols} {kind} bf16={bf16}")
    rng = np.random.default_rng(rows * 3 + cols + len(name))
    W = workloads.random_weight(rng, rows * cols, kind).reshape(rows, cols)
    W[: min(rows, 2), :] = 0.0                            # zero blocks
    src = W
    if bf16:  # the device gets bf16 bits; the oracle their exact fp32 values
        src = nf4.bf16_rne(W)
        W = nf4.bf16_bits_to_f32(src).reshape(rows, cols)
    q, got = gpu_quantize(api, src, bf16=bf16, qtype=name)
    ref, qt = oracle_quant(W, name)
    assert_quant_equal(got, ref)
    deq = api.to_host_bits(api.qlora_dequantize(q))
    torch.cuda.synchronize()
    want = nf4.dequantize(qt, (rows, cols), qtypes.codebook(name))
    np.testing.assert_array_equal(deq.reshape(rows, cols), want)


def run_linear(api, inp, name, need_bwd=True):
    import torch

    q, _ = gpu_quantize(api, inp.W, qtype=name)
    X, L1, L2 = api.to_device_bf16(inp.X), api.to_device_bf16(inp.L1), api.to_device_bf16(inp.L2)
    Y, T = api.qlora_linear_fwd(q, X, L1, L2, inp.s, want_T=need_bwd)
    out = {"Y": api.to_host_bits(Y)}
    if need_bwd:
        dY = api.to_device_bf16(inp.dY)
        dX, dL1, dL2 = api.qlora_linear_bwd(q, X, dY, L1, L2, inp.s, T=T)
        torch.cuda.synchronize()
        out.update(dX=api.to_host_bits(dX), dL1=dL1.cpu().numpy(), dL2=dL2.cpu().numpy())
    return out


def oracle_linear(inp, name, need_bwd=True):
    tab = qtypes.codebook(name)
    Wd = nf4.dequantize(nf4.quantize(inp.W, tab), inp.W.shape, tab)
    Y, _ = linear.linear_fwd(inp.X, Wd, inp.L1, inp.L2, inp.s)
    ref = {"Y": Y}
    if need_bwd:
        dX, dL1, dL2 = linear.linear_bwd(inp.X, Wd, inp.L1, inp.L2, inp.s, inp.dY)
        ref.update(dX=dX, dL1=dL1, dL2=dL2)
    return ref


def compare(got, ref, label):
    for k, R in ref.items():
        check_output(label, k, got[k], R)


@pytest.mark.parametrize("name", TYPES)
def test_linear_fwd_bwd(api, name):
    say(f"{name} linear 200x320x136 r=16")
    rng = np.random.default_rng(41 + len(name))
    inp = workloads.draw_linear(rng, workloads.LinearShape("t", 320, 136), 200, 16, 0.5, "normal", 0.02, True)
    compare(run_linear(api, inp, name), oracle_linear(inp, name), f"{name} linear")


@pytest.mark.parametrize("name", TYPES)
@pytest.mark.parametrize("M", [1, 4])
def test_gemv(api, name, M):
    say(f"{name} gemv M={M}")
    rng = np.random.default_rng(51 + M + len(name))
    inp = workloads.draw_linear(rng, workloads.LinearShape("t", 1024, 520), M, 64, 0.25, "normal", 0.02, False)
    compare(run_linear(api, inp, name, need_bwd=False), oracle_linear(inp, name, need_bwd=False), f"{name} gemv")


# ---- without double quantisation --------------------------------------------------------

@pytest.mark.parametrize("name", ["nf4", "int4"])
def test_no_dq_quantize_dequantize_bit_exact(api, name):
    import torch

    say(f"{name} without DQ: quantize 300x211")
    rng = np.random.default_rng(61 + len(name))
    W = workloads.random_weight(rng, 300 * 211, "normal").reshape(300, 211)
    W[:1, :] = 0.0
    q, got = gpu_quantize(api, W, qtype=name, double_quant=False)
    tab = qtypes.codebook(name)
    qt = nf4.quantize(W, tab, double_quant=False)
    np.testing.assert_array_equal(got["codes"], qt["codes"])
    np.testing.assert_array_equal(got["absmax32"].view(np.uint32), qt["absmax32"].view(np.uint32))
    deq = api.to_host_bits(api.qlora_dequantize(q))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(deq.reshape(300, 211), nf4.dequantize(qt, (300, 211), tab))


def run_linear_nodq(api, inp, name, need_bwd):
    import torch

    q, _ = gpu_quantize(api, inp.W, qtype=name, double_quant=False)
    X, L1, L2 = api.to_device_bf16(inp.X), api.to_device_bf16(inp.L1), api.to_device_bf16(inp.L2)
    Y, T = api.qlora_linear_fwd(q, X, L1, L2, inp.s, want_T=need_bwd)
    out = {"Y": api.to_host_bits(Y)}
    if need_bwd:
        dY = api.to_device_bf16(inp.dY)
        dX, dL1, dL2 = api.qlora_linear_bwd(q, X, dY, L1, L2, inp.s, T=T)
        torch.cuda.synchronize()
        out.update(dX=api.to_host_bits(dX), dL1=dL1.cpu().numpy(), dL2=dL2.cpu().numpy())
    return out


def oracle_linear_nodq(inp, name, need_bwd):
    tab = qtypes.codebook(name)
    Wd = nf4.dequantize(nf4.quantize(inp.W, tab, double_quant=False), inp.W.shape, tab)
    Y, _ = linear.linear_fwd(inp.X, Wd, inp.L1, inp.L2, inp.s)
    ref = {"Y": Y}
    if need_bwd:
        dX, dL1, dL2 = linear.linear_bwd(inp.X, Wd, inp.L1, inp.L2, inp.s, inp.dY)
        ref.update(dX=dX, dL1=dL1, dL2=dL2)
    return ref


@pytest.mark.parametrize("M,K,N,r", [
    (200, 320, 136, 16),     # large-M path (dequantise + GEMM)
    (1, 1024, 520, 64),      # byte-table GEMV
    (4, 64 * 9, 264, 8),     # register-ring GEMV (K % 128 == 64)
])
def test_no_dq_linear(api, M, K, N, r):
    say(f"nf4 without DQ: linear {M}x{K}x{N} r={r}")
    need_bwd = M > 16
    rng = np.random.default_rng(71 + M + K)
    inp = workloads.draw_linear(rng, workloads.LinearShape("t", K, N), M, r, 0.5, "normal", 0.02, need_bwd)
    compare(run_linear_nodq(api, inp, "nf4", need_bwd), oracle_linear_nodq(inp, "nf4", need_bwd), f"no-DQ {M}x{K}x{N}")
