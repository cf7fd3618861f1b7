"""bf16 weights with no fp32 master copy, trained with the fused step (adamw-sr
page, intro and Correctness: stochastic rounding lets a bf16-only layer train
where round-to-nearest stalls).

Synthetic regression: a teacher W* with entries ~N(0, 1) and inputs
X ~ N(0, 1/d), targets y = X W*^T. The student is a bf16 linear layer
initialised at W* + N(0, 0.05): every weight must move by a few hundredths
while its magnitude is O(1), so one bf16 ulp is 2**-7 .. 2**-6 and a step of
about lr = 5e-4 is far below half an ulp. Three runs from the same start
and the same batches:
  * AdamWSR, rounding "sr"  (bf16 storage only)
  * AdamWSR, rounding "rn"  (bf16 storage only)
  * torch.optim.AdamW on an fp32 copy (a master-weight reference)
Forward and backward run in float32 from the bf16 storage (no bf16 GEMM).
"""

import numpy as np
import pytest
import torch

from adamw_optimizer_stochastic_amd import AdamWSR
from _gpu_util import gpu, require_gpu, announce

pytestmark = gpu
D_IN, D_OUT, BATCH, STEPS, LR = 256, 32, 512, 1500, 5e-4


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _problem(dev):
    g = torch.Generator(device="cpu").manual_seed(1234)
    w_star = torch.randn(D_OUT, D_IN, generator=g)
    w0 = (w_star + 0.05 * torch.randn(D_OUT, D_IN, generator=g))
    xs = [torch.randn(BATCH, D_IN, generator=g) / D_IN ** 0.5 for _ in range(STEPS)]
    return w_star.to(dev), w0.to(dev), [x.to(dev) for x in xs]


def _train(kind, w_star, w0, xs, seed=0):
    dev = w_star.device
    if kind == "fp32":
        w = torch.nn.Parameter(w0.clone())
        opt = torch.optim.AdamW([w], lr=LR, weight_decay=0.0)
    else:
        w = torch.nn.Parameter(w0.to(torch.bfloat16))
        opt = AdamWSR([w], lr=LR, weight_decay=0.0, seed=seed, rounding=kind)
    losses = []
    for x in xs:
        y = x @ w_star.T
        pred = x @ w.float().T
        loss = (pred - y).square().mean()
        opt.zero_grad()
        loss.backward()
        opt.step()
        losses.append(loss.item())
    err = (w.detach().float() - w_star).square().mean().item()
    return np.array(losses), err


def test_sr_trains_bf16_weights_where_rn_stalls():
    dev = torch.device("cuda", 0)
    w_star, w0, xs = _problem(dev)
    announce("bf16 training: sr / rn / fp32")
    sr, err_sr = _train("sr", w_star, w0, xs)
    rn, err_rn = _train("rn", w_star, w0, xs)
    fp, err_fp = _train("fp32", w_star, w0, xs)
    sr2, _ = _train("sr", w_star, w0, xs)
    announce(f"final loss (mean of last 100): sr {sr[-100:].mean():.3e} rn {rn[-100:].mean():.3e} "
             f"fp32 {fp[-100:].mean():.3e}; weight mse sr {err_sr:.3e} rn {err_rn:.3e} fp32 {err_fp:.3e}")
    start = sr[:10].mean()
    # RN: most updates round away; the loss barely moves.
    assert rn[-100:].mean() > 0.5 * start
    # SR: the updates accumulate; the loss falls by more than an order of
    # magnitude and ends far below RN, near the fp32 reference (the bf16
    # grid itself leaves a floor of about ulp**2/12 per weight).
    assert sr[-100:].mean() < 0.1 * start
    assert sr[-100:].mean() < 0.1 * rn[-100:].mean()
    assert err_sr < 0.1 * err_rn
    assert err_sr < 4e-4                       # ~ (2**-7)**2 / 12 * a few
    assert fp[-100:].mean() < sr[-100:].mean()  # the master copy stays the best
    # bitwise reproducible
    assert np.array_equal(sr, sr2)
