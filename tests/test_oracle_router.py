"""Pins of the oracle's router logits (logits = x . W_g^T, the step before routing).

* One-hot router rows pick single hidden-state entries: the logits are those
  bf16 values exactly.
* Against float64 library matmuls (an independent routine) rounded to fp32:
  equal to within one fp32 ulp (both sums are exact to far below that).
* Scaling the router weights by a power of two scales the logits exactly.
A transposed operand, a dropped or doubled term, or a wrong row stride each
fail one of these.
"""
import numpy as np
import torch

import oracle
from synth import gen_router_weights, gen_x


def test_one_hot_rows_select_entries():
    M, E, H = 5, 12, 256
    x = gen_x(H, M, seed=31)
    cols = torch.randperm(H, generator=torch.Generator().manual_seed(31))[:E]
    w = torch.zeros(E, H, dtype=torch.bfloat16)
    w[torch.arange(E), cols] = 1.0
    out = oracle.router_logits(x, w)
    assert np.array_equal(out, x.float()[:, cols].numpy())


def test_matches_float64_library_matmul():
    M, E, H = 7, 64, 2048
    x = gen_x(H, M, seed=32)
    w = gen_router_weights(E, H, seed=32)
    out = oracle.router_logits(x, w)
    ref = (x.double() @ w.double().T).float().numpy()
    ulp = np.spacing(np.abs(ref).astype(np.float32))
    assert (np.abs(out - ref) <= ulp).all()
    assert 0.5 < out.std() < 2.0  # N(0,1/H) router rows give logits of about unit spread


def test_power_of_two_scaling_is_exact():
    M, E, H = 3, 16, 512
    x = gen_x(H, M, seed=33)
    w = gen_router_weights(E, H, seed=33)
    a = oracle.router_logits(x, w)
    b = oracle.router_logits(x, (w.float() * 4.0).to(torch.bfloat16))
    assert np.array_equal(b, a * 4.0)
