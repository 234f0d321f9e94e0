"""CPU check of the rounding bound the GPU invariant tests use (tests/gpu_common.rounding_bound):
an emulation of the 16-bit decode arithmetic -- per 16-token tile, logits in fp32, online
softmax in base 2 with a lazy rescale, weights rounded to the 16-bit type against the running
maximum, fp32 accumulation, pieces of a context cut at arbitrary places merged with the
log-sum-exp rule, output rounded to the 16-bit type -- stays within the bound of the exact
fp64 result for every cut, and two cuts of one context stay within twice it."""

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_common import rounding_bound

LOG2E = 1.4426950408889634


def _emulate(q, k, v, scale, dtype, cuts):
    """One query [Hq, D] over k, v [L, Hkv, D], the context cut into pieces at `cuts`."""
    tdt = getattr(torch, dtype)
    Hq, D = q.shape
    L, Hkv, _ = k.shape
    G = Hq // Hkv
    qf, kf, vf = q.float(), k.float(), v.float()
    out = torch.empty((Hq, D), dtype=tdt)
    bounds = [0] + sorted(cuts) + [L]
    for h in range(Hq):
        g = h // G
        parts = []
        for a, b in zip(bounds[:-1], bounds[1:]):
            m, l, acc = -1e30, torch.tensor(0.0), torch.zeros(D)
            for t0 in range(a, b, 16):
                t1 = min(b, t0 + 16)
                s = (kf[t0:t1, g, :] @ qf[h]) * (scale * LOG2E)
                mx = float(s.max())
                if mx > m + 8.0:
                    alpha = torch.tensor(2.0 ** (m - mx) if m > -1e29 else 0.0, dtype=torch.float32)
                    l, acc, m = l * alpha, acc * alpha, mx
                p = torch.exp2(s - m).to(tdt).float()      # weights rounded to the 16-bit type
                l = l + p.sum()
                acc = acc + p @ vf[t0:t1, g, :]
            parts.append((m, l, acc))
        m, l, acc = parts[0]
        for m2, l2, acc2 in parts[1:]:
            mn = max(m, m2)
            f0 = torch.tensor(2.0 ** (m - mn), dtype=torch.float32)
            f1 = torch.tensor(2.0 ** (m2 - mn), dtype=torch.float32)
            l, acc, m = l * f0 + l2 * f1, acc * f0 + acc2 * f1, mn
        out[h] = (acc / l).to(tdt)
    return out


@pytest.mark.parametrize("dtype", ["bfloat16", "float16"])
def test_emulated_decode_stays_within_the_bound(dtype):
    rng = np.random.default_rng(3)
    tdt = getattr(torch, dtype)
    L, Hq, Hkv, D = 1500, 16, 2, 64
    k = torch.from_numpy(rng.standard_normal((L, Hkv, D), dtype=np.float32)).to(tdt)
    v = torch.from_numpy(rng.standard_normal((L, Hkv, D), dtype=np.float32)).to(tdt)
    q = torch.from_numpy(rng.standard_normal((Hq, D), dtype=np.float32)).to(tdt)
    scale = D ** -0.5
    exact = oracle.decode_attention(q[None], [k], [v], scale)[0]
    bound = rounding_bound(q, k, v, scale, dtype)
    outs = []
    for cuts in ([], [16 * 7], [16 * 30, 16 * 31, 16 * 77], [16 * 50 + 16 * i for i in range(0, 40, 3)]):
        o = _emulate(q, k, v, scale, dtype, cuts).double().numpy()
        assert (np.abs(o - exact) <= bound).all(), (cuts, float((np.abs(o - exact) / bound).max()))
        outs.append(o)
    for o in outs[1:]:
        assert (np.abs(o - outs[0]) <= 2 * bound).all()
    # the bound is not vacuous: well under the 16-bit tolerance of the parity tests
    assert bound.max() < 2e-2


def test_bound_catches_a_dropped_token():
    """A planted mistake (each head's heaviest token left out of the sum, as a gather off by a
    tile would) breaks the bound on some element: the bound is far tighter than the 16-bit
    tolerance of the parity tests and sees a single missing token."""
    rng = np.random.default_rng(4)
    dtype, tdt = "bfloat16", torch.bfloat16
    L, Hq, Hkv, D = 600, 4, 1, 64
    k = torch.from_numpy(rng.standard_normal((L, Hkv, D), dtype=np.float32)).to(tdt)
    v = torch.from_numpy(rng.standard_normal((L, Hkv, D), dtype=np.float32)).to(tdt)
    q = torch.from_numpy(rng.standard_normal((Hq, D), dtype=np.float32)).to(tdt)
    scale = D ** -0.5
    bound = rounding_bound(q, k, v, scale, dtype)
    exact = oracle.decode_attention(q[None], [k], [v], scale)[0]
    z = (k.double()[:, 0, :] @ q.double().T).numpy() * scale     # [L, Hq]
    w = np.exp(z - z.max(axis=0))
    w[w.argmax(axis=0), np.arange(Hq)] = 0.0
    w /= w.sum(axis=0)
    dropped = w.T @ v.double()[:, 0, :].numpy()
    assert all((np.abs(dropped[h] - exact[h]) > bound[h]).any() for h in range(Hq))
