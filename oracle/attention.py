"""fp64 reference for paged decode attention -- test infrastructure only.

What is computed.  The yunthe.com page "大模型推理显存优化实战：PagedAttention机制原理与
vLLM连续批处理配置", section "PagedAttention分页注意力机制原理", says the attention kernel
looks physical blocks up through the block table and runs attention over those
non-contiguous blocks; the 111cn.net page "大模型推理引擎高频优化：连续批处理、
PagedAttention 与 KV Cache 实战拆解" §3.2 says the block table keeps the logical token
order.  Paging is therefore a storage layout only: the result is ordinary scaled dot-product
attention of the one new query against the sequence's tokens in logical order.  This module
computes exactly that, over contiguous per-sequence K/V that never went through a pool.

The pages do not define the attention arithmetic itself; the readings taken here are:

* one query per sequence (decode), no mask other than the context length;
* query head ``h`` reads KV head ``h // G`` with ``G = Hq / Hkv`` (consecutive query heads
  share a KV head -- the pages never mention grouped queries, this is the convention);
* ``scale`` is a caller argument (the workloads use ``1/sqrt(D)``);
* a context of length 0 gives an all-zero output row.

Inputs may be numpy arrays or torch CPU tensors of any float dtype; they are upcast exactly
to fp64 first, and everything after that is fp64.
"""

from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    """Exact upcast of a numpy array or torch CPU tensor to a float64 numpy array."""
    if hasattr(x, "detach"):  # torch tensor: numpy has no bfloat16, let torch widen it
        import torch

        return x.detach().to(torch.float64).cpu().numpy()
    return np.asarray(x, dtype=np.float64)


def decode_attention_single(q_h, k_g, v_g, scale: float) -> np.ndarray:
    """Attention of one query head over one KV head of one sequence.

    ``q_h``: [D]; ``k_g``, ``v_g``: [L, D].  Returns [D] (fp64).

    Step by step: logits ``z_t = scale * <q, k_t>``; subtract their maximum (changes
    nothing mathematically, keeps ``exp`` finite); weights ``w_t = exp(z_t - max)``; output
    ``sum_t w_t v_t / sum_t w_t``.  ``L == 0`` returns zeros.
    """
    q_h = _f64(q_h)
    k_g = _f64(k_g)
    v_g = _f64(v_g)
    L = k_g.shape[0]
    if L == 0:
        return np.zeros(v_g.shape[1] if v_g.ndim == 2 else q_h.shape[0], dtype=np.float64)
    z = scale * (k_g @ q_h)
    w = np.exp(z - z.max())
    return (w @ v_g) / w.sum()


def decode_attention(q, keys, values, scale: float) -> np.ndarray:
    """Decode attention for a batch of sequences with contiguous, un-paged K/V.

    ``q``: [B, Hq, D].  ``keys[s]``, ``values[s]``: [L_s, Hkv, D] -- the sequence's tokens
    in logical order.  Returns [B, Hq, D] in fp64.

    For every sequence ``s`` and query head ``h`` (with ``g = h // G``):
    ``out[s, h] = softmax_t(scale * K_s[t, g] . q[s, h]) @ V_s[:, g]``, written per KV head
    as one matrix product for the logits and one for the weighted sum.
    """
    qd = _f64(q)
    B, Hq, D = qd.shape
    if len(keys) != B or len(values) != B:
        raise ValueError("need one K and one V array per sequence")
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for s in range(B):
        k = _f64(keys[s])
        v = _f64(values[s])
        L = k.shape[0]
        if L == 0:
            continue  # empty context: zero row
        Hkv = k.shape[1]
        if Hq % Hkv != 0:
            raise ValueError("Hq must be a multiple of Hkv")
        G = Hq // Hkv
        for g in range(Hkv):
            qg = qd[s, g * G:(g + 1) * G, :]          # [G, D] query heads of KV head g
            z = scale * (qg @ k[:, g, :].T)           # [G, L] logits
            z = z - z.max(axis=1, keepdims=True)
            w = np.exp(z)                             # [G, L] unnormalised weights
            out[s, g * G:(g + 1) * G, :] = (w @ v[:, g, :]) / w.sum(axis=1, keepdims=True)
    return out
