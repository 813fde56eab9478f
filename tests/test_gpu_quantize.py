"""GPU parity of NF4 + DQ quantisation and of the standalone dequant.

Codes, E4M3 constants, second-level scales, the mean and the dequantised
bf16 weights are unique under the method's steps, so the HIP results must
equal the oracle's bit for bit: on the 512x512 workload, on ragged sizes
(short last block and short last DQ group), on bf16 inputs, on special
tensors (all zero, a single block, constructed ties) and on full LLaMA-7B,
-33B and -65B weight shapes.
"""

import numpy as np
import pytest

from bit_nf4_quantized_amd import workloads
from oracle import nf4
from gpu_util import assert_quant_equal, gpu_quantize, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    return require_gpu()


def check_roundtrip(api, W, bf16=False, shape=None):
    w32 = nf4.bf16_bits_to_f32(W) if bf16 else W
    ref = nf4.quantize(w32)
    q, got = gpu_quantize(api, W.reshape(shape) if shape else W, bf16)
    assert_quant_equal(got, ref)
    d = api.qlora_dequantize(q)
    np.testing.assert_array_equal(api.to_host_bits(d).reshape(-1), nf4.dequantize(ref))
    return q


def test_tiny_512(api):
    say("quantize tiny-512")
    inp = workloads.tiny_512()
    check_roundtrip(api, inp.W)


@pytest.mark.parametrize("rows,cols", [(1, 1), (1, 63), (3, 21), (5, 64 * 256 // 5 + 7), (7, 64 * 256 + 3),
                                       (100, 100), (257, 64), (64, 16384 * 3 + 64 * 5 + 9), (33, 4097)])
def test_ragged_shapes(api, rows, cols):
    say(f"quantize ragged {rows}x{cols}")
    rng = np.random.default_rng(rows * 100003 + cols)
    W = workloads.random_weight(rng, rows * cols).reshape(rows, cols)
    check_roundtrip(api, W)


@pytest.mark.parametrize("kind", ["normal", "student-t4"])
def test_bf16_input(api, kind):
    say(f"quantize bf16 {kind}")
    rng = np.random.default_rng(77)
    W = workloads.to_bf16_bits(workloads.random_weight(rng, 300 * 700, kind).reshape(300, 700))
    check_roundtrip(api, W, bf16=True)


def test_special_tensors(api):
    say("quantize special tensors")
    check_roundtrip(api, np.zeros((64, 300), np.float32))
    rng = np.random.default_rng(1)
    check_roundtrip(api, workloads.random_weight(rng, 64).reshape(1, 64))
    # zero blocks among live ones, subnormal blocks, exact codebook multiples
    W = workloads.random_weight(rng, 64 * 512).reshape(64, 512)
    W[3, :] = 0.0
    W[5, :64] = 1e-39
    W[7, :64] = (np.tile(nf4.nf4_codebook(), 4) * np.float32(0.037)).astype(np.float32)
    check_roundtrip(api, W)


def test_constructed_ties(api):
    say("quantize ties")
    q = nf4.nf4_codebook()
    m = nf4.nf4_midpoints(q)
    W = np.zeros((4, 64), np.float32)
    W[:, 0] = 1.0
    k = 1
    for j in range(15):
        f = np.float32(m[j])
        below = np.nextafter(f, np.float32(-2)) if f > m[j] else f
        above = np.nextafter(below, np.float32(2))
        for v in (below, above, f):
            W[k // 63, 1 + k % 63] = v
            k += 1
    check_roundtrip(api, W)


def test_determinism(api):
    say("quantize determinism")
    rng = np.random.default_rng(5)
    W = workloads.random_weight(rng, 2048 * 1024).reshape(2048, 1024)
    _, a = gpu_quantize(api, W)
    _, b = gpu_quantize(api, W)
    assert_quant_equal(a, b)


@pytest.mark.parametrize("name,index", [("llama7b-layer", 0), ("llama7b-layer", 4), ("llama7b-layer", 6),
                                        ("llama33b-layer", 0)])
def test_full_size_layer_weights(api, name, index):
    shp = workloads.WORKLOADS[name]["linears"][index]
    say(f"quantize full {name} {shp.name} {shp.N}x{shp.K}")
    W = workloads.layer_weight(name, index)
    check_roundtrip(api, W)


def test_llama65b_shape_bf16(api):
    shp = workloads.LLAMA65B[0]
    say(f"quantize llama65b q {shp.N}x{shp.K} (fp32 and bf16)")
    W = workloads.quantize_weight(shp, 4, 0)
    check_roundtrip(api, W)
    check_roundtrip(api, workloads.to_bf16_bits(W), bf16=True)
