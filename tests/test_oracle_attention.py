"""CPU pins of the fp64 attention oracle (no GPU).

The oracle must pass every pin; each planted mistake (a copy of the oracle with one error)
must fail at least one -- so the pins would catch a dropped term, a wrong sign or index,
a transposed operand or a wrong normalisation in the oracle itself.
"""

import numpy as np
import pytest
import torch

import oracle
from tests import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_passes_pin(pin):
    pin(oracle.decode_attention)


def test_single_head_helper_matches_batched():
    rng = np.random.default_rng(7)
    q, k, v = P._rand_case(rng, B=2, Hq=4, Hkv=2, D=8, Lmax=20)
    full = oracle.decode_attention(q, k, v, 0.4)
    for s in range(2):
        for h in range(4):
            one = oracle.decode_attention_single(q[s, h], k[s][:, h // 2], v[s][:, h // 2], 0.4)
            np.testing.assert_allclose(one, full[s, h], rtol=0, atol=1e-13)


def test_low_precision_inputs_are_upcast_exactly():
    # bf16 / fp16 inputs are widened without rounding before any arithmetic
    rng = np.random.default_rng(8)
    q32 = torch.from_numpy(rng.standard_normal((1, 2, 8), dtype=np.float32))
    k32 = torch.from_numpy(rng.standard_normal((5, 1, 8), dtype=np.float32))
    v32 = torch.from_numpy(rng.standard_normal((5, 1, 8), dtype=np.float32))
    for dt in (torch.bfloat16, torch.float16):
        q, k, v = q32.to(dt), k32.to(dt), v32.to(dt)
        a = oracle.decode_attention(q, [k], [v], 0.3)
        b = oracle.decode_attention(q.double().numpy(), [k.double().numpy()], [v.double().numpy()], 0.3)
        assert np.array_equal(a, b)


# ------------------------------------------------------------------ planted mistakes
def _mutant(kind):
    def impl(q, keys, values, scale):
        q = np.asarray(q, dtype=np.float64)
        B, Hq, D = q.shape
        out = np.zeros((B, Hq, D))
        for s in range(B):
            k = np.asarray(keys[s], dtype=np.float64)
            v = np.asarray(values[s], dtype=np.float64)
            if kind == "swap_kv":
                k, v = v, k
            if kind == "drop_last_token" and k.shape[0] > 1:
                k, v = k[:-1], v[:-1]
            L = k.shape[0]
            if L == 0:
                continue
            Hkv = k.shape[1]
            G = Hq // Hkv
            for h in range(Hq):
                g = (h % Hkv) if kind == "head_map_modulo" else h // G
                sc = 1.0 if kind == "no_scale" else scale
                z = sc * (k[:, g, :] @ q[s, h])
                if kind == "sign_flip":
                    z = -z
                w = np.exp(z - z.max())
                if kind == "no_normalise":
                    out[s, h] = w @ v[:, g, :]
                elif kind == "normalise_by_length":
                    out[s, h] = (w @ v[:, g, :]) / L
                elif kind == "uniform_weights":
                    out[s, h] = v[:, g, :].mean(axis=0)
                else:
                    out[s, h] = (w @ v[:, g, :]) / w.sum()
        return out

    return impl


MUTANTS = ["swap_kv", "drop_last_token", "head_map_modulo", "no_scale", "sign_flip",
           "no_normalise", "normalise_by_length", "uniform_weights"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_planted_mistake_is_caught(kind):
    impl = _mutant(kind)
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin(impl)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin catches the '{kind}' mistake"


def test_mutant_harness_is_faithful_without_a_mistake():
    # the harness above with no mistake planted passes every pin
    for pin in P.ALL_PINS:
        pin(_mutant("none"))
