"""GPU parity of Eq. (9) mixing (qshift_mix, through the C ABI) against the float64 oracle:
out[j] = X + (1 - mu[j]) X-dagger. The kernel computes in fp32 (one rounding of 1 - mu, of the
product and of the sum, or a fused multiply-add), so each element is within 2 ulp of
|x| + |(1 - mu) x-dagger| of the exact value.
"""
import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu


def _check(x, mu, H, W, shift, gamma):
    import torch

    import linear_complexity_vision_amd as L
    out = L.qshift_mix(torch.from_numpy(x).cuda(), torch.from_numpy(mu).cuda(), H, W, shift, gamma)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    ref = oracle.qshift_mix(x, mu, H, W, shift, gamma)
    xd = oracle.qshift_f64(x, H, W, shift, gamma)
    bound = 2.0 * 2.0 ** -23 * (np.abs(x.astype(np.float64))[None] + np.abs((1.0 - mu.astype(np.float64))[:, None, None, :] * xd[None]))
    bad = np.abs(got - ref) > bound
    assert not bad.any(), f"{bad.sum()} elements outside the fp32 bound"


def test_mix_workload():
    wl = workloads.make(2)
    g = np.random.Generator(np.random.PCG64(77))
    mu = g.uniform(0, 1, (3, wl.C)).astype(np.float32)
    print(f"[case] qshift_mix {wl.name} x, 3 mixes", flush=True)
    _check(wl.x, mu, wl.H, wl.W, wl.shift, wl.gamma)


@pytest.mark.parametrize("B,H,W,C,shift,gamma,J", [
    (1, 5, 7, 100, 2, 0.125, 1), (3, 4, 4, 17, 3, 0.25, 3), (2, 6, 2, 10, 2, 0.2, 8),
    (1, 3, 3, 12, 0, 0.25, 2), (2, 4, 4, 8, 4, 0.25, 3), (1, 64, 64, 96, 1, 0.25, 3),
    (2, 37, 41, 1000, 2, 0.25, 3)])  # odd index divisors, 0.76M items
def test_mix_edge_shapes(B, H, W, C, shift, gamma, J):
    g = np.random.Generator(np.random.PCG64(B * 1000 + H * 100 + W * 10 + C + J))
    x = (g.standard_normal((B, H * W, C)) * 3).astype(np.float32)
    mu = g.uniform(-0.5, 1.5, (J, C)).astype(np.float32)
    mu[0, : min(C, 3)] = [1.0, 0.0, 0.5][: min(C, 3)]
    print(f"[case] qshift_mix B{B} H{H} W{W} C{C} s{shift} g{gamma} J{J}", flush=True)
    _check(x, mu, H, W, shift, gamma)
