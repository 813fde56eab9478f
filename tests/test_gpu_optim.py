"""GPU parity of the optimiser step (qlora_clip_grad_norm, qlora_adam_step)
against the float64 oracle (oracle/optim.py), and of its two state
placements against each other.

The norm is a float64 sum in a different order from the oracle's, so it
must agree to 1e-12 relative; the clip coefficient to fp32 rounding. Adam
runs in fp32: with the clip coefficient given, m, v and theta must equal
the fp32 evaluation of the update in its written order bit for bit
(tests/adam_fp32.py), and through the whole clip + Adam path each must stay
within the error bound propagated from the fp32 roundings of every step
around the float64 oracle's trajectory. The same steps with m and v in
pinned host memory ("paged out") must give bit-identical results to
device-resident state, and repeated runs must be bit-identical. The bf16
copy of the parameters must be the round-to-nearest-even of the fp32
parameters. At the size of all LLaMA-7B adapters (r = 64 on 7 linears x 32
layers, 160 M values) the oracle checks a sample of elements (the update is
elementwise).
"""

import numpy as np
import pytest

from adam_fp32 import adam_error_bounds, adam_step_fp32
from oracle import nf4, optim
from gpu_util import require_gpu, say

pytestmark = pytest.mark.gpu
LLAMA7B_ADAPTER_PARAMS = 32 * 64 * (4 * (4096 + 4096) + 2 * (4096 + 11008) + (11008 + 4096))


@pytest.fixture(scope="module")
def api():
    return require_gpu()


@pytest.mark.parametrize("n,scale,max_norm", [(1000003, 0.01, 0.3), (3, 1.0, 0.3), (0, 1.0, 0.3),
                                              (4096, 1e-4, 0.3), (777, 2.0, float("inf"))])
def test_clip_norm(api, n, scale, max_norm):
    import torch

    say(f"clip norm n={n}")
    rng = np.random.default_rng(n + 1)
    g = (scale * rng.standard_normal(n)).astype(np.float32)
    coef, norm = api.qlora_clip_grad_norm(torch.from_numpy(g).cuda(), max_norm)
    torch.cuda.synchronize()
    ref_norm = optim.grad_norm(g)
    assert norm.item() == pytest.approx(ref_norm, rel=1e-12, abs=0.0)
    ref = optim.clip_coef(g, max_norm) if np.isfinite(max_norm) else 1.0
    assert coef.item() == pytest.approx(ref, rel=2 ** -23)
    if n:
        gp = torch.from_numpy(g).pin_memory()            # the gradient in pinned host memory
        c2, n2 = api.qlora_clip_grad_norm(gp, max_norm)
        torch.cuda.synchronize()
        assert c2.item() == coef.item() and n2.item() == norm.item()


def adam_run(api, theta0, grads, paged, hp, max_norm=0.3):
    import torch

    n = theta0.size
    theta = torch.from_numpy(theta0.copy()).cuda()
    mk = (lambda: torch.zeros(n, dtype=torch.float32).pin_memory()) if paged else \
         (lambda: torch.zeros(n, dtype=torch.float32, device="cuda"))
    m, v = mk(), mk()
    tb = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    for t, g in enumerate(grads, start=1):
        gd = torch.from_numpy(g).cuda()
        coef, _ = api.qlora_clip_grad_norm(gd, max_norm)
        api.qlora_adam_step(theta, gd, m, v, t, coef=coef, theta_bf16=tb, **hp)
    torch.cuda.synchronize()
    return (theta.cpu().numpy(), m.cpu().numpy(), v.cpu().numpy(),
            tb.view(torch.int16).cpu().numpy().view(np.uint16))


@pytest.mark.parametrize("n,wd", [(100003, 0.0), (4099, 0.01), (5, 0.0)])
def test_adam_steps(api, n, wd):
    say(f"adam n={n} wd={wd}")
    rng = np.random.default_rng(n)
    theta0 = (0.02 * rng.standard_normal(n)).astype(np.float32)
    grads = [(s * rng.standard_normal(n)).astype(np.float32) for s in (0.001, 0.1, 0.5, 0.01, 2.0)]
    hp = dict(lr=2e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=wd)
    th, m, v, tb = adam_run(api, theta0, grads, False, hp)
    # the float64 oracle on the same gradients and clip coefficients, with the
    # hyperparameters the library receives (fp32 values: 0.999 as fp32 is
    # 0.99900001287...); each result within the bound propagated from the
    # fp32 roundings of every step (tests/adam_fp32.py)
    coefs = [optim.clip_coef(g, 0.3) for g in grads]
    rt, rm, rv, et, em, ev = adam_error_bounds(theta0, grads, coefs, hp["lr"], hp["beta1"], hp["beta2"],
                                               hp["eps"], wd)
    for name, got, ref, bound in (("m", m, rm, em), ("v", v, rv, ev), ("theta", th, rt, et)):
        bad = np.abs(got - ref) > bound
        say(f"  {name}: max |err| / bound {np.max(np.abs(got - ref) / bound):.3f}")
        assert not np.any(bad), (name, int(bad.sum()))
    np.testing.assert_array_equal(tb, nf4.bf16_rne(th))        # the bf16 copy of the fp32 parameters
    # paged-out state: identical arithmetic, identical bits; and reruns are identical
    th2, m2, v2, tb2 = adam_run(api, theta0, grads, True, hp)
    for a, b in ((th, th2), (m, m2), (v, v2), (tb, tb2)):
        np.testing.assert_array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                                      b.view(np.uint32) if b.dtype == np.float32 else b)
    th3, _, _, _ = adam_run(api, theta0, grads, False, hp)
    np.testing.assert_array_equal(th.view(np.uint32), th3.view(np.uint32))


@pytest.mark.parametrize("n,wd", [(100003, 0.0), (4099, 0.01), (7, 0.001)])
def test_adam_matches_fp32_evaluation_bit_exact(api, n, wd):
    """With the clip coefficient given (the oracle's, rounded to fp32), the
    kernel's m, v and theta equal the fp32 evaluation of the textbook update
    in the written operation order bit for bit, step after step."""
    import torch

    say(f"adam fp32 bit-exact n={n} wd={wd}")
    rng = np.random.default_rng(n + 17)
    theta0 = (0.02 * rng.standard_normal(n)).astype(np.float32)
    grads = [(s * rng.standard_normal(n)).astype(np.float32) for s in (0.001, 0.1, 0.5, 0.01, 2.0, 3e-5)]
    hp = dict(lr=2e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=wd)
    theta = torch.from_numpy(theta0.copy()).cuda()
    m = torch.zeros(n, dtype=torch.float32, device="cuda")
    v = torch.zeros(n, dtype=torch.float32, device="cuda")
    et, em, ev = theta0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    for t, g in enumerate(grads, start=1):
        c32 = np.float32(optim.clip_coef(g, 0.3))
        coef = torch.tensor([c32], dtype=torch.float32, device="cuda")
        api.qlora_adam_step(theta, torch.from_numpy(g).cuda(), m, v, t, coef=coef, **hp)
        et, em, ev = adam_step_fp32(et, g, em, ev, t, hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], wd, c32)
        torch.cuda.synchronize()
        for name, got, ref in (("m", m, em), ("v", v, ev), ("theta", theta, et)):
            np.testing.assert_array_equal(got.cpu().numpy().view(np.uint32), ref.view(np.uint32),
                                          err_msg=f"{name} step {t}")


def test_adam_full_adapter_size_sampled(api):
    import torch

    n = LLAMA7B_ADAPTER_PARAMS
    say(f"adam + clip at the LLaMA-7B adapter size, n={n}")
    gen = torch.Generator(device="cuda").manual_seed(7)
    theta = 0.02 * torch.randn(n, device="cuda", generator=gen)
    g = 1e-4 * torch.randn(n, device="cuda", generator=gen)
    m = torch.zeros(n, device="cuda")
    v = torch.zeros(n, device="cuda")
    idx = np.sort(np.random.default_rng(3).choice(n, 20000, replace=False))
    t0, g0 = theta.cpu().numpy(), g.cpu().numpy()
    coef, norm = api.qlora_clip_grad_norm(g, 0.3)
    api.qlora_adam_step(theta, g, m, v, 1, lr=2e-4, coef=coef)
    torch.cuda.synchronize()
    assert norm.item() == pytest.approx(optim.grad_norm(g0), rel=1e-12)
    c = optim.clip_coef(g0, 0.3)
    rt, rm, rv, et, em, ev = adam_error_bounds(t0[idx], [g0[idx]], [c], 2e-4, 0.9, 0.999, 1e-8, 0.0)
    th = theta.cpu().numpy()[idx]
    assert np.all(np.abs(m.cpu().numpy()[idx] - rm) <= em)
    assert np.all(np.abs(v.cpu().numpy()[idx] - rv) <= ev)
    assert np.all(np.abs(th - rt) <= et)
