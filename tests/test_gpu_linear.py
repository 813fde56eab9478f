"""GPU parity of the QLoRA linear forward and backward (and the small-M GEMV).

Outputs are compared element by element with the float64 oracle on the same
seeded inputs: err = max|G - R| / RMS(R) <= 2e-2 for Y, dX, dL1 and dL2 (bf16
operands, fp32 accumulation, one final bf16 rounding; the bf16 rounding of
the oracle output itself is printed as the floor). Exact identities pin the
fused dequantisation inside the GEMMs: with a one-hot input and a zero
adapter, Y and dX reproduce the standalone dequantised weight exactly.
"""

import numpy as np
import pytest

from bit_nf4_quantized_amd import workloads
from oracle import linear, nf4
from gpu_util import check_output, gpu_quantize, require_gpu, say

pytestmark = pytest.mark.gpu
TOL = 2e-2


@pytest.fixture(scope="module")
def api():
    return require_gpu()


def dev(api, bits):
    return api.to_device_bf16(bits)


def run_case(api, inp: workloads.LinearInputs, need_bwd=True, use_T=True):
    import torch

    q, _ = gpu_quantize(api, inp.W)
    X, L1, L2 = dev(api, inp.X), dev(api, inp.L1), dev(api, inp.L2)
    Y, T = api.qlora_linear_fwd(q, X, L1, L2, inp.s, want_T=need_bwd and use_T)
    out = {"Y": api.to_host_bits(Y)}
    if need_bwd:
        dY = dev(api, inp.dY)
        dX, dL1, dL2 = api.qlora_linear_bwd(q, X, dY, L1, L2, inp.s, T=T if use_T else None)
        torch.cuda.synchronize()
        out.update(dX=api.to_host_bits(dX), dL1=dL1.cpu().numpy(), dL2=dL2.cpu().numpy())
    return out


def oracle_case(inp):
    qt = nf4.quantize(inp.W)
    Wd = nf4.dequantize(qt, inp.W.shape)
    Y, _ = linear.linear_fwd(inp.X, Wd, inp.L1, inp.L2, inp.s)
    ref = {"Y": Y}
    if inp.dY is not None:
        dX, dL1, dL2 = linear.linear_bwd(inp.X, Wd, inp.L1, inp.L2, inp.s, inp.dY)
        ref.update(dX=dX, dL1=dL1, dL2=dL2)
    return ref, Wd


def compare(got, ref, label):
    for k, R in ref.items():
        check_output(label, k, got[k], R)


def case(M, K, N, r, s, seed, kind="normal", std=0.02, with_grad=True):
    rng = np.random.default_rng(seed)
    return workloads.draw_linear(rng, workloads.LinearShape("t", K, N), M, r, s, kind, std, with_grad)


def test_tiny_512(api):
    say("linear tiny-512 (M=64, r=8, s=2)")
    inp = workloads.tiny_512()
    ref, _ = oracle_case(inp)
    compare(run_case(api, inp), ref, "tiny-512")


@pytest.mark.parametrize("M,K,N,r,s,kind", [
    (200, 320, 136, 16, 0.5, "normal"),          # ragged M and N tiles
    (384, 1024, 768, 64, 0.25, "normal"),        # several tiles each way
    (17, 256, 264, 8, 1.0, "student-t4"),        # smallest M above the GEMV (fused one-pass forward)
    (130, 64 * 7, 8 * 41, 256, 0.125, "normal"),  # largest rank, ragged everything
    # more 256x256 tiles than CUs (17 x 17 = 289): 255 full tiles, then the last
    # two tile-columns as 128-row half tiles, with ragged M and N inside them
    (4100, 512, 4160, 16, 0.5, "normal"),
    # 4 x 66 tiles: the last 2 tile-columns as 64-row quarter tiles (ragged M
    # and N inside them); dX: 4 x 2 tiles, no tail split
    (1000, 512, 66 * 256 - 8, 16, 0.5, "normal"),
    # reductions of 12288 and more run with three B stage buffers: the
    # forward (K = 12352) here, and dX (over N = 12352) in the next case
    (300, 64 * 193, 200, 16, 0.5, "normal"),
    (300, 256, 64 * 193, 16, 0.25, "student-t4"),
    # decode sizes (M r <= 256): the adapter's slice sums inside the GEMV, T
    # written by it for the backward. 6 slices (the last one partial) over 8
    # waves with X staged; 19 slices, up to 3 per wave; 4-wave workgroups
    (4, 64 * 41, 200, 64, 0.5, "normal"),
    (3, 64 * 151, 40, 64, 0.25, "student-t4"),
    (4, 64 * 35, 8200, 64, 0.5, "normal"),
    # M r <= 1024: four 16-byte chunks of each slice per lane. 6 slices;
    # 24 slices, 3 per wave (the most a wave takes); 25 slices (one more than
    # 8 waves take: the separate reduction)
    (16, 64 * 45, 136, 64, 0.25, "normal"),
    (12, 64 * 192, 64, 32, 0.5, "student-t4"),
    (12, 64 * 194, 64, 32, 0.5, "normal"),
])
def test_shapes(api, M, K, N, r, s, kind):
    say(f"linear M={M} K={K} N={N} r={r} s={s} {kind}")
    inp = case(M, K, N, r, s, M * 7 + K, kind)
    ref, _ = oracle_case(inp)
    compare(run_case(api, inp), ref, f"{M}x{K}x{N}")
    compare(run_case(api, inp, use_T=False), ref, f"{M}x{K}x{N} recomputed T")


@pytest.mark.parametrize("M", [1, 2, 3, 4, 9, 16])
def test_gemv_small_m(api, M):
    say(f"gemv M={M}")
    inp = case(M, 1024, 520, 64, 0.25, 100 + M, with_grad=False)
    ref, _ = oracle_case(inp)
    compare(run_case(api, inp, need_bwd=False), ref, f"gemv M={M}")


@pytest.mark.parametrize("M,K,N,r", [
    (1, 64 * 9, 264, 8),        # K % 128 == 64: the last k-step is half a step
    (16, 64 * 35, 8 * 13, 256),  # largest rank, ragged rows
    (5, 64, 8, 64),             # one block per row, one partial row tile
])
def test_gemv_ragged(api, M, K, N, r):
    say(f"gemv M={M} K={K} N={N} r={r}")
    inp = case(M, K, N, r, 0.5, 200 + M + K, with_grad=False)
    ref, _ = oracle_case(inp)
    compare(run_case(api, inp, need_bwd=False), ref, f"gemv {M}x{K}x{N} r={r}")


@pytest.mark.parametrize("M,K,N,r", [
    (1, 256, 8200, 64),     # 513 row tiles: 4-wave workgroups, X staged in LDS, ragged last tile
    (16, 1024, 8200, 64),   # 4-wave workgroups, X fragments in registers
    (16, 4096, 200, 72),    # 8-wave workgroups, X in registers, rank above 64
    (3, 2048, 1000, 8),     # 8-wave workgroups, X staged, rank 8
    (2, 128, 40, 256),      # one k-step per row (idle waves), largest rank
    (1, 512, 264, 8),       # single-token kernel, rank 8: columns 8..63 of the LoRA split idle
    (1, 4096, 22528, 16),   # single-token kernel, 88 rows per CU (11 row groups), rank 16
    (1, 16384, 2048, 64),   # single-token kernel, largest K (64 LoRA slices, 32 KB of X)
])
def test_gemv_paths(api, M, K, N, r):
    say(f"gemv path M={M} K={K} N={N} r={r}")
    inp = case(M, K, N, r, 0.25, 300 + M + K + N, with_grad=False)
    ref, _ = oracle_case(inp)
    compare(run_case(api, inp, need_bwd=False), ref, f"gemv {M}x{K}x{N} r={r}")


@pytest.mark.parametrize("M,K,N,r", [
    (24, 64 * 9, 8 * 13, 24),     # ragged 64-row tile, odd number of k-steps, r not a multiple of 64
    (32, 1024, 520, 64),
    (33, 2048, 1000, 72),         # X tile of 64 rows; two LoRA steps
    (64, 4096, 200, 256),         # largest rank: four LoRA steps
    (100, 512, 8 * 300, 16),      # X tile of 128 rows, padded
    (128, 4096, 4096, 64),        # several K-slices per tile
    (128, 64, 64, 8),             # one k-step: a single slice, no reduction
])
def test_mid_m_forward(api, M, K, N, r):
    say(f"mid-M forward M={M} K={K} N={N} r={r}")
    inp = case(M, K, N, r, 0.5, 300 + M + K, with_grad=False)
    ref, _ = oracle_case(inp)
    compare(run_case(api, inp, need_bwd=False), ref, f"mid-M {M}x{K}x{N} r={r}")


@pytest.mark.parametrize("M", [40, 128])
def test_mid_m_one_hot_reproduces_dequant(api, M):
    """Rows of X that are unit vectors with L2 = 0 give rows of the dequantised
    weight exactly, through the K-slices and their reduction."""
    import torch

    say(f"mid-M one-hot rows M={M}")
    K, N = 2048, 200
    rng = np.random.default_rng(12 + M)
    W = workloads.random_weight(rng, N * K, "normal").reshape(N, K)
    q, _ = gpu_quantize(api, W)
    Wd = nf4.bf16_bits_to_f32(nf4.dequantize(nf4.quantize(W), (N, K)))
    ks = rng.choice(K, M, replace=False)
    Xh = np.zeros((M, K), np.float32)
    Xh[np.arange(M), ks] = 1.0
    L1 = workloads.to_bf16_bits(rng.standard_normal((K, 8)).astype(np.float32))
    Y, T = api.qlora_linear_fwd(q, dev(api, workloads.to_bf16_bits(Xh)), dev(api, L1),
                                dev(api, np.zeros((8, N), np.uint16)), 1.0, want_T=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(nf4.bf16_bits_to_f32(api.to_host_bits(Y)), Wd[:, ks].T)
    np.testing.assert_array_equal(api.to_host_bits(T), L1[ks])      # T = X L1 picks rows of L1


def test_lora_only_and_zero_adapter(api):
    say("linear W = 0 (LoRA branch alone) and L2 = 0")
    inp = case(96, 256, 192, 32, 0.75, 5)
    inp.W[:] = 0.0
    ref, _ = oracle_case(inp)
    compare(run_case(api, inp), ref, "W=0")
    inp2 = case(96, 256, 192, 32, 0.75, 6)
    inp2.L2[:] = 0
    ref2, _ = oracle_case(inp2)
    got2 = run_case(api, inp2)
    assert not np.any(got2["dL1"]), "dL1 must be exactly zero when L2 = 0"
    compare(got2, ref2, "L2=0")


def test_one_hot_reproduces_dequant(api):
    """X = I and L2 = 0 give Y = dequant(Wt)^T exactly; dY = I and L1 = 0 give
    dX = dequant(Wt) exactly (the fused dequant equals the standalone one)."""
    import torch

    say("one-hot identities")
    K, N = 256, 192
    rng = np.random.default_rng(11)
    W = workloads.random_weight(rng, N * K, "student-t4").reshape(N, K)
    q, _ = gpu_quantize(api, W)
    Wd = nf4.bf16_bits_to_f32(nf4.dequantize(nf4.quantize(W), (N, K)))
    eyeK = workloads.to_bf16_bits(np.eye(K, dtype=np.float32))
    eyeN = workloads.to_bf16_bits(np.eye(N, dtype=np.float32))
    L1 = workloads.to_bf16_bits(rng.standard_normal((K, 16)).astype(np.float32))
    zero_L2 = np.zeros((16, N), np.uint16)
    Y, _ = api.qlora_linear_fwd(q, dev(api, eyeK), dev(api, L1), dev(api, zero_L2), 1.0)
    Yf = nf4.bf16_bits_to_f32(api.to_host_bits(Y))
    np.testing.assert_array_equal(Yf, Wd.T)
    L2 = workloads.to_bf16_bits(rng.standard_normal((16, N)).astype(np.float32))
    zero_L1 = np.zeros((K, 16), np.uint16)
    dX, _, _ = api.qlora_linear_bwd(q, dev(api, np.zeros((N, K), np.uint16)), dev(api, eyeN), dev(api, zero_L1),
                                    dev(api, L2), 1.0)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(nf4.bf16_bits_to_f32(api.to_host_bits(dX)), Wd)


def test_determinism_and_identities(api):
    import torch

    say("linear determinism and adjoint identity")
    inp = case(256, 512, 384, 32, 0.5, 21)
    a = run_case(api, inp)
    b = run_case(api, inp)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])
    # adjoint identity <dY, Y> = <dX, X> holds to the bf16/fp32 rounding level
    Y = nf4.bf16_bits_to_f32(a["Y"]).astype(np.float64)
    dX = nf4.bf16_bits_to_f32(a["dX"]).astype(np.float64)
    lhs = np.vdot(linear.widen(inp.dY), Y)
    rhs = np.vdot(dX, linear.widen(inp.X))
    assert abs(lhs - rhs) <= 2e-2 * np.sqrt(np.vdot(Y, Y) * np.vdot(linear.widen(inp.dY), linear.widen(inp.dY)) / Y.size)


def test_bf16_gradients(api):
    import torch

    say("bf16 adapter gradients")
    inp = case(128, 256, 128, 16, 0.5, 31)
    ref, _ = oracle_case(inp)
    q, _ = gpu_quantize(api, inp.W)
    X, L1, L2, dY = (dev(api, a) for a in (inp.X, inp.L1, inp.L2, inp.dY))
    _, dL1, dL2 = api.qlora_linear_bwd(q, X, dY, L1, L2, inp.s, need_dX=False, grad_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    check_output("bf16 grads", "dL1", api.to_host_bits(dL1), ref["dL1"])
    check_output("bf16 grads", "dL2", api.to_host_bits(dL2), ref["dL2"])


@pytest.mark.parametrize("M", [8, 96, 384])
def test_side_stream_with_allocation_churn(api, M):
    """Calls on a non-default stream, with allocations churning on the
    default stream meanwhile, give the same bits as calls on the default
    stream: the binding's workspaces and outputs belong to the call's stream,
    so the caching allocator never hands them to other work while the
    library's kernels still use them."""
    import torch

    say(f"side stream + allocation churn M={M}")
    inp = case(M, 1024, 768, 64, 0.25, 300 + M)
    q, _ = gpu_quantize(api, inp.W)
    X, L1, L2, dY = dev(api, inp.X), dev(api, inp.L1), dev(api, inp.L2), dev(api, inp.dY)
    Y0, T0 = api.qlora_linear_fwd(q, X, L1, L2, inp.s, want_T=True)
    dX0, a0, b0 = api.qlora_linear_bwd(q, X, dY, L1, L2, inp.s, T=T0)
    torch.cuda.synchronize()
    ref = [api.to_host_bits(Y0), api.to_host_bits(dX0), a0.cpu().numpy(), b0.cpu().numpy()]
    side = torch.cuda.Stream()          # default priority
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(4):
        Y, T = api.qlora_linear_fwd(q, X, L1, L2, inp.s, want_T=True, stream=side)
        dX, a, b = api.qlora_linear_bwd(q, X, dY, L1, L2, inp.s, T=T, stream=side)
        outs.append((Y, dX, a, b))
        for _ in range(8):              # churn on the default stream
            junk = torch.full((M * 1024 + 4096,), 7.0, device="cuda")
            junk.mul_(3.0)
            del junk
    side.synchronize()
    torch.cuda.synchronize()
    for Y, dX, a, b in outs:
        np.testing.assert_array_equal(api.to_host_bits(Y), ref[0])
        np.testing.assert_array_equal(api.to_host_bits(dX), ref[1])
        np.testing.assert_array_equal(a.cpu().numpy(), ref[2])
        np.testing.assert_array_equal(b.cpu().numpy(), ref[3])


def test_token_rows_beyond_2gb(api):
    """M = 131072 tokens of K = 8192: X and dX hold 2 GiB each, so the dense
    GEMMs run the token rows in two launches (130816 + 256 rows) and the
    adapter products take the generic path. Rows on both sides of the chunk
    boundary are compared with the oracle; dL1 and dL2 are sums over all
    rows, accumulated over row chunks through oracle.linear.linear_bwd."""
    import torch

    M, K, N, r, s = 131072, 8192, 256, 8, 0.5
    say(f"linear with 2 GiB activations: M={M} K={K} N={N} r={r}")
    rng = np.random.default_rng(77)
    inp = workloads.draw_linear(rng, workloads.LinearShape("t", K, N), 8, r, s, "normal", 0.02, True)
    X = workloads.to_bf16_bits(rng.standard_normal((M, K), dtype=np.float32))
    dY = workloads.to_bf16_bits(rng.standard_normal((M, N), dtype=np.float32))
    q, _ = gpu_quantize(api, inp.W)
    Xd, L1, L2, dYd = dev(api, X), dev(api, inp.L1), dev(api, inp.L2), dev(api, dY)
    Y, T = api.qlora_linear_fwd(q, Xd, L1, L2, s, want_T=True)
    dX, dL1, dL2 = api.qlora_linear_bwd(q, Xd, dYd, L1, L2, s, T=T)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 130815, 130816, 130817, 131071])
    Yr = api.to_host_bits(Y[rows.tolist()])
    dXr = api.to_host_bits(dX[rows.tolist()])
    dL1g, dL2g = dL1.cpu().numpy(), dL2.cpu().numpy()
    del Y, T, dX, dL1, dL2, Xd, dYd
    Wd = nf4.dequantize(nf4.quantize(inp.W), inp.W.shape)
    check_output("2 GiB", "Y rows", Yr, linear.linear_fwd_rows(X, Wd, inp.L1, inp.L2, s, rows))
    check_output("2 GiB", "dX rows", dXr, linear.linear_bwd_dx_rows(Wd, inp.L1, inp.L2, s, dY, rows))
    g1 = np.zeros((K, r))
    g2 = np.zeros((r, N))
    for c in range(0, M, 8192):
        _, a, b = linear.linear_bwd(X[c:c + 8192], Wd, inp.L1, inp.L2, s, dY[c:c + 8192])
        g1 += a
        g2 += b
    check_output("2 GiB", "dL1", dL1g, g1)
    check_output("2 GiB", "dL2", dL2g, g2)
