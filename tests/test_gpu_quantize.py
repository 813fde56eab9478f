"""GPU parity of NF4 + DQ quantisation and of the standalone dequant.

Codes, E4M3 constants, second-level scales, the mean and the dequantised
bf16 weights are unique under the method's steps, so the HIP results must
equal the oracle's bit for bit: on the 512x512 workload, on ragged sizes
(short last block and short last DQ group), on bf16 inputs, on special
tensors (all zero, a single block, constructed ties) and on full LLaMA-7B,
-33B and -65B weight shapes (the 22016-wide 65B MLP weights from fp32 and
from bf16 included).
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


@pytest.mark.parametrize("index", [4, 6], ids=["gate-22016x8192", "down-8192x22016"])
@pytest.mark.parametrize("bf16", [False, True], ids=["fp32", "bf16"])
def test_llama65b_22016_wide(api, index, bf16):
    """The 22016-wide LLaMA-65B MLP weights (the tensors the 65B quantise
    pass spends most of its bytes on), whole, from fp32 and from bf16."""
    shp = workloads.LLAMA65B[index]
    say(f"quantize llama65b {shp.name} {shp.N}x{shp.K} ({'bf16' if bf16 else 'fp32'})")
    W = workloads.quantize_weight(shp, 4, index)
    check_roundtrip(api, workloads.to_bf16_bits(W) if bf16 else W, bf16=bf16)


def batch_host(q):
    """Host copies of one batch output (codes and block constants)."""
    from gpu_util import nf4_host

    return nf4_host(q)


@pytest.mark.parametrize("bf16", [False, True], ids=["fp32", "bf16"])
def test_batch_mixed_shapes(api, bf16):
    """qlora_quantize_batch over ragged, tiny, empty and group-spanning
    tensors in one pass (one with fp32 block constants, no DQ): every tensor
    bit-exact with the oracle, as if quantised alone."""
    import torch

    shapes = [(1, 63), (5, 64 * 256 // 5 + 7), (0, 17), (257, 64), (33, 4097), (100, 100), (64, 16384 + 9),
              (3, 21)]
    say(f"quantize batch of {len(shapes)} ({'bf16' if bf16 else 'fp32'})")
    rng = np.random.default_rng(4242 + bf16)
    hostW, devW = [], []
    for rows, cols in shapes:
        W = workloads.random_weight(rng, rows * cols, "student-t4").reshape(rows, cols)
        if bf16:
            W = workloads.to_bf16_bits(W)
            devW.append(api.to_device_bf16(W))
        else:
            devW.append(torch.from_numpy(np.ascontiguousarray(W)).cuda())
        hostW.append(nf4.bf16_bits_to_f32(W) if bf16 else W)
    nodq = 5                                           # the 100 x 100 tensor keeps fp32 constants
    outs = [api.NF4Tensor.empty(r, c, "cuda", "nf4", k != nodq) for k, (r, c) in enumerate(shapes)]
    api.qlora_quantize_batch(devW, outs=outs)
    torch.cuda.synchronize()
    for k, (W, q) in enumerate(zip(hostW, outs)):
        if W.size == 0:
            continue
        got = batch_host(q)
        if k == nodq:
            ref = nf4.quantize(W, double_quant=False)
            np.testing.assert_array_equal(got["codes"], ref["codes"])
            np.testing.assert_array_equal(got["absmax32"].view(np.uint32), ref["absmax32"].view(np.uint32))
        else:
            assert_quant_equal(got, nf4.quantize(W))


def test_batch_llama65b_layer_equals_single_calls(api):
    """The seven LLaMA-65B linears of one layer (809.5M weights) in one batch,
    from fp32 and from bf16: every output equal, byte for byte, to the
    single-tensor call (itself bit-exact with the oracle on these shapes,
    test_llama65b_22016_wide and test_llama65b_shape_bf16)."""
    import torch

    Ws = [torch.from_numpy(workloads.quantize_weight(shp, 4, i)).cuda() for i, shp in enumerate(workloads.LLAMA65B)]
    for bf16 in (False, True):
        say(f"quantize batch llama65b layer ({'bf16' if bf16 else 'fp32'})")
        src = [W.to(torch.bfloat16) for W in Ws] if bf16 else Ws
        outs = api.qlora_quantize_batch(src)
        for W, qb in zip(src, outs):
            qs = api.qlora_quantize(W)
            torch.cuda.synchronize()
            numel = W.numel()
            nb = -(-numel // 64)
            ng = -(-nb // 256)
            assert torch.equal(qb.codes[: numel // 2], qs.codes[: numel // 2])
            assert torch.equal(qb.absmax8[:nb], qs.absmax8[:nb])
            assert torch.equal(qb.scale2[:ng].view(torch.int32), qs.scale2[:ng].view(torch.int32))
            assert torch.equal(qb.mean.view(torch.int32), qs.mean.view(torch.int32))
        del outs


@pytest.mark.parametrize("qtype", ["int4", "fp4_e2m1", "fp4_e3m0"])
def test_batch_other_types_equal_single_calls(api, qtype):
    """A batch of another 4-bit type (one threshold table per launch), with
    and without DQ: byte-equal to qlora_quantize on each tensor alone (which
    test_gpu_qtypes.py pins to the oracle bit for bit)."""
    import torch

    say(f"quantize batch {qtype}")
    rng = np.random.default_rng(5151)
    shapes = [(300, 700), (64, 16384 + 64), (7, 64 * 256 + 3)]
    Ws = [torch.from_numpy(workloads.random_weight(rng, r * c, "student-t4").reshape(r, c)).cuda() for r, c in shapes]
    for dq in (True, False):
        outs = api.qlora_quantize_batch(Ws, qtype=qtype, double_quant=dq)
        for W, qb in zip(Ws, outs):
            qs = api.qlora_quantize(W, qtype=qtype, double_quant=dq)
            torch.cuda.synchronize()
            numel = W.numel()
            nb = -(-numel // 64)
            assert torch.equal(qb.codes[: (numel + 1) // 2], qs.codes[: (numel + 1) // 2])
            if dq:
                ng = -(-nb // 256)
                assert torch.equal(qb.absmax8[:nb], qs.absmax8[:nb])
                assert torch.equal(qb.scale2[:ng].view(torch.int32), qs.scale2[:ng].view(torch.int32))
                assert torch.equal(qb.mean.view(torch.int32), qs.mean.view(torch.int32))
            else:
                assert torch.equal(qb.absmax32[:nb].view(torch.int32), qs.absmax32[:nb].view(torch.int32))


def test_batch_of_sixteen(api):
    """The largest batch, 16 tensors of assorted small shapes (one of them
    one weight long), each bit-exact with the oracle."""
    import torch

    say("quantize batch of 16")
    rng = np.random.default_rng(1616)
    shapes = [(1 + int(rng.integers(0, 40)), 1 + int(rng.integers(0, 3000))) for _ in range(15)] + [(1, 1)]
    hostW = [workloads.random_weight(rng, r * c).reshape(r, c) for r, c in shapes]
    outs = api.qlora_quantize_batch([torch.from_numpy(W).cuda() for W in hostW])
    torch.cuda.synchronize()
    for W, q in zip(hostW, outs):
        assert_quant_equal(batch_host(q), nf4.quantize(W))
