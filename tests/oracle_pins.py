"""Pins for the attention oracle: checks against things other than the oracle itself.

Each ``pin_*`` takes an implementation with the oracle's signature
``impl(q, keys, values, scale) -> [B, Hq, D]`` and raises ``AssertionError`` when the
implementation disagrees with brute force, an independent library routine, a closed form
or a hand-worked fixture.  ``tests/test_oracle_attention.py`` runs them on the oracle and
on deliberately broken copies of it, to show every pin set catches a plausible mistake.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

_MATH_NAMES = {"exp": math.exp, "log": math.log, "e": math.e, "sqrt": math.sqrt}


def _val(x):
    if isinstance(x, str):
        return float(eval(x, {"__builtins__": {}}, _MATH_NAMES))  # hand-written closed forms
    return float(x)


def _arr(nested):
    if isinstance(nested, list):
        return [_arr(x) for x in nested]
    return _val(nested)


def _rand_case(rng, B, Hq, Hkv, D, Lmax, Lmin=1):
    q = rng.standard_normal((B, Hq, D))
    lens = rng.integers(Lmin, Lmax, size=B, endpoint=True)
    keys = [rng.standard_normal((int(L), Hkv, D)) for L in lens]
    values = [rng.standard_normal((int(L), Hkv, D)) for L in lens]
    return q, keys, values


def brute_force(q, keys, values, scale):
    """Scalar loops with math.exp / math.fsum; no numpy arithmetic."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    out = np.zeros((B, Hq, D))
    for s in range(B):
        k = np.asarray(keys[s], dtype=np.float64)
        v = np.asarray(values[s], dtype=np.float64)
        L = k.shape[0]
        if L == 0:
            continue
        Hkv = k.shape[1]
        G = Hq // Hkv
        for h in range(Hq):
            g = h // G
            z = [scale * math.fsum(float(q[s, h, d]) * float(k[t, g, d]) for d in range(D))
                 for t in range(L)]
            m = max(z)
            w = [math.exp(zt - m) for zt in z]
            den = math.fsum(w)
            for d in range(D):
                out[s, h, d] = math.fsum(w[t] * float(v[t, g, d]) for t in range(L)) / den
    return out


def sdpa_reference(q, keys, values, scale):
    """torch's scaled_dot_product_attention in fp64 on the CPU, K/V repeated per group."""
    import torch
    import torch.nn.functional as F

    q = torch.as_tensor(np.asarray(q, dtype=np.float64))
    B, Hq, D = q.shape
    out = torch.zeros((B, Hq, D), dtype=torch.float64)
    for s in range(B):
        k = torch.as_tensor(np.asarray(keys[s], dtype=np.float64))
        v = torch.as_tensor(np.asarray(values[s], dtype=np.float64))
        if k.shape[0] == 0:
            continue
        G = Hq // k.shape[1]
        kk = k.permute(1, 0, 2).repeat_interleave(G, dim=0).unsqueeze(0).contiguous()
        vv = v.permute(1, 0, 2).repeat_interleave(G, dim=0).unsqueeze(0).contiguous()
        qq = q[s].unsqueeze(0).unsqueeze(2).contiguous()  # [1, Hq, 1, D]
        o = F.scaled_dot_product_attention(qq, kk, vv, scale=scale)
        out[s] = o[0, :, 0, :]
    return out.numpy()


# ---------------------------------------------------------------------------- pins
def pin_brute_force(impl, seeds=range(4)):
    for seed in seeds:
        rng = np.random.default_rng(1000 + seed)
        Hkv = int(rng.integers(1, 3))
        G = int(rng.integers(1, 3))
        q, k, v = _rand_case(rng, B=int(rng.integers(1, 4)), Hq=Hkv * G, Hkv=Hkv,
                             D=int(rng.integers(1, 9)), Lmax=6)
        scale = float(rng.uniform(0.1, 1.5))
        got = impl(q, k, v, scale)
        ref = brute_force(q, k, v, scale)
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def pin_sdpa(impl, seeds=range(4)):
    for seed in seeds:
        rng = np.random.default_rng(2000 + seed)
        Hkv = int(rng.integers(1, 4))
        G = int(rng.choice([1, 2, 4]))
        q, k, v = _rand_case(rng, B=3, Hq=Hkv * G, Hkv=Hkv, D=16, Lmax=40)
        scale = 1.0 / math.sqrt(16)
        got = impl(q, k, v, scale)
        np.testing.assert_allclose(got, sdpa_reference(q, k, v, scale), rtol=0, atol=1e-12)


def pin_closed_forms(impl):
    rng = np.random.default_rng(3000)
    B, Hkv, G, D = 2, 2, 2, 8
    Hq = Hkv * G
    q = rng.standard_normal((B, Hq, D))
    # (1) one token: the output is that token's V row, exactly
    k1 = [rng.standard_normal((1, Hkv, D)) for _ in range(B)]
    v1 = [rng.standard_normal((1, Hkv, D)) for _ in range(B)]
    out = impl(q, k1, v1, 0.7)
    for s in range(B):
        for h in range(Hq):
            assert np.array_equal(out[s, h], v1[s][0, h // G]), "L=1 must return the V row"
    # (2) zero query, (3) zero scale, (4) all keys equal: plain mean of the V rows
    L = 9
    k = [rng.standard_normal((L, Hkv, D)) for _ in range(B)]
    v = [rng.standard_normal((L, Hkv, D)) for _ in range(B)]
    mean = [vs.mean(axis=0) for vs in v]
    kconst = [np.broadcast_to(ks[:1], ks.shape).copy() for ks in k]
    for qq, kk, sc in ((np.zeros_like(q), k, 0.5), (q, k, 0.0), (q, kconst, 0.9)):
        out = impl(qq, kk, v, sc)
        for s in range(B):
            for h in range(Hq):
                np.testing.assert_allclose(out[s, h], mean[s][h // G], rtol=0, atol=1e-12)
    # (5) V constant per KV head -> that constant (weights sum to 1, head map h // G)
    c = np.array([3.25, -1.5])
    vconst = [np.broadcast_to(c[None, :, None], (L, Hkv, D)).copy() for _ in range(B)]
    out = impl(q, k, vconst, 0.3)
    for h in range(Hq):
        np.testing.assert_allclose(out[:, h], c[h // G], rtol=0, atol=1e-12)
    # (6) one-hot V rows (D = L): the output is the weight vector; it sums to 1 and
    #     matches softmax of the logits (two-token logistic form checked by the fixtures)
    Lh = 6
    kh = [rng.standard_normal((Lh, 1, Lh))]
    vh = [np.eye(Lh)[:, None, :]]
    qh = rng.standard_normal((1, 1, Lh))
    w = impl(qh, kh, vh, 0.8)[0, 0]
    assert abs(w.sum() - 1.0) < 1e-12 and (w > 0).all()
    z = 0.8 * np.array([math.fsum(qh[0, 0, d] * kh[0][t, 0, d] for d in range(Lh)) for t in range(Lh)])
    for t in range(Lh):
        for u in range(Lh):  # ratio of weights is exp of the logit gap
            assert abs(math.log(w[t] / w[u]) - (z[t] - z[u])) < 1e-12
    # (7) empty context -> zeros
    out = impl(q[:1], [np.zeros((0, Hkv, D))], [np.zeros((0, Hkv, D))], 1.0)
    assert np.array_equal(out, np.zeros_like(out))


def pin_golden(impl):
    with open(os.path.join(GOLDEN, "attention_worked.json"), encoding="utf-8") as f:
        fx = json.load(f)
    for case in fx["cases"]:
        q = np.array(_arr(case["q"]))
        B, Hq, D = q.shape
        keys, values = [], []
        for s in range(B):
            k = np.array(_arr(case["k"][s]), dtype=np.float64)
            v = np.array(_arr(case["v"][s]), dtype=np.float64)
            if k.size == 0:
                k = np.zeros((0, 1, D))
                v = np.zeros((0, 1, D))
            keys.append(k)
            values.append(v)
        exp = np.array(_arr(case["expected"]))
        got = impl(q, keys, values, case["scale"])
        np.testing.assert_allclose(got, exp, rtol=0, atol=1e-14, err_msg=case["name"])


ALL_PINS = (pin_brute_force, pin_sdpa, pin_closed_forms, pin_golden)
