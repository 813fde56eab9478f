"""GPU parity of the blockwise Int8 absmax codec (qlora_int8_quantize /
qlora_int8_dequantize) against the oracle (oracle/int8.py).

Codes, block absmax values and dequantised values (fp32 and bf16) are
unique under the codec's steps, so they are compared bit for bit: every
block size, ragged tails (a short last block; lanes and waves past the end),
fp32 and bf16 inputs, zero and tiny blocks, and, at the LLaMA-65B weight
size (22016 x 8192), a sample of 4096 whole blocks that the oracle
recomputes one by one (the blocks are independent).
"""

import numpy as np
import pytest

from bit_nf4_quantized_amd import workloads
from oracle import int8, nf4
from gpu_util import require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    return require_gpu()


def run(api, x, block, bf16=False):
    import torch

    t = api.to_device_bf16(x) if bf16 else torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()
    codes, absmax = api.qlora_int8_quantize(t.reshape(-1), block)
    f32 = api.qlora_int8_dequantize(codes, absmax, block)
    b16 = api.qlora_int8_dequantize(codes, absmax, block, dtype=torch.bfloat16)
    torch.cuda.synchronize()
    return (codes.cpu().numpy(), absmax.cpu().numpy(), f32.cpu().numpy(),
            b16.view(torch.int16).cpu().numpy().view(np.uint16))


def check(api, x, block, bf16=False):
    xf = nf4.bf16_bits_to_f32(x) if bf16 else x
    ref = int8.quantize(xf, block)
    codes, absmax, f32, b16 = run(api, x, block, bf16)
    np.testing.assert_array_equal(codes, ref["codes"])
    np.testing.assert_array_equal(absmax.view(np.uint32), ref["absmax"].view(np.uint32))
    np.testing.assert_array_equal(f32.view(np.uint32), int8.dequantize_f32(ref).view(np.uint32))
    np.testing.assert_array_equal(b16, int8.dequantize_bf16(ref))


@pytest.mark.parametrize("block", [64, 128, 256, 512, 1024, 2048, 4096])
@pytest.mark.parametrize("numel", [1, 63, 4096 * 3 + 17, 300 * 211, 512 * 37])
def test_int8_bit_exact(api, block, numel):
    say(f"int8 block={block} numel={numel}")
    rng = np.random.default_rng(block * 7 + numel)
    x = workloads.random_weight(rng, numel, "student-t4")
    check(api, x, block)


@pytest.mark.parametrize("block", [64, 1024])
def test_int8_bf16_input(api, block):
    say(f"int8 bf16 input block={block}")
    rng = np.random.default_rng(31 + block)
    x = workloads.to_bf16_bits(workloads.random_weight(rng, 512 * 41 + 9, "normal", 1.0))
    check(api, x, block, bf16=True)


def test_int8_zero_tiny_and_ties(api):
    say("int8 zero, tiny and tie blocks")
    x = np.zeros(64 * 6 + 9, np.float32)
    x[64] = np.float32(2.0 ** -121)                   # zero block by the limit
    x[128] = np.float32(2.0 ** -120)                  # just an ordinary block
    x[129] = np.float32(-2.0 ** -121)
    x[192:201] = [127.0, 2.5, 3.5, -2.5, 0.5, 1.5, 126.5, -0.49, 100.25]   # factor exactly 1: ties
    x[256:261] = [1.0, -0.5, 0.25, 0.75, -1.0]
    x[320] = np.float32(3.0e38)                       # near the fp32 maximum
    x[321] = np.float32(-1.0e38)
    x[384 + 8] = np.float32(-3.0)                     # the short last block
    check(api, x, 64)


def test_int8_full_size_sampled_blocks(api):
    import torch

    rows, cols, block = 22016, 8192, 64
    say(f"int8 full size {rows}x{cols} block={block}")
    rng = np.random.default_rng(65)
    W = workloads.draw_weight(rng, rows, cols, "normal", 0.015)
    t = torch.from_numpy(W).cuda().reshape(-1)
    codes, absmax = api.qlora_int8_quantize(t, block)
    f32 = api.qlora_int8_dequantize(codes, absmax, block)
    torch.cuda.synchronize()
    nb = W.size // block
    pick = np.sort(rng.choice(nb, 4096, replace=False))
    pick[-1] = nb - 1
    flat = W.reshape(-1)
    idx = (pick[:, None] * block + np.arange(block)[None, :]).reshape(-1)
    ref = int8.quantize(flat[idx], block)             # the picked blocks, one after another
    got_codes = codes.cpu().numpy()[idx]
    np.testing.assert_array_equal(got_codes, ref["codes"])
    np.testing.assert_array_equal(absmax.cpu().numpy()[pick].view(np.uint32), ref["absmax"].view(np.uint32))
    np.testing.assert_array_equal(f32.cpu().numpy()[idx].view(np.uint32), int8.dequantize_f32(ref).view(np.uint32))


def test_int8_empty(api):
    import torch

    x = torch.empty(0, dtype=torch.float32, device="cuda")
    codes, absmax = api.qlora_int8_quantize(x, 256)
    assert codes.numel() == 0 and absmax.numel() == 0
    assert api.qlora_int8_dequantize(codes, absmax, 256).numel() == 0
