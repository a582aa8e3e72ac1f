"""Elementwise kernel feature maps phi applied to queries and keys (fp64).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The glossary page "Lightning Attention" (features list; FAQ Q1) says a kernel
feature map replaces the softmax, so that O_t = sum_j lam^(t-j)
(phi(q_t) . phi(k_j)) v_j, but it never names the map.  Offered here:
  identity : phi(x) = x
  elu1     : phi(x) = elu(x) + 1 = x + 1 (x > 0), exp(x) (x <= 0); phi'(x) = min(1, phi(x))
  relu     : phi(x) = max(x, 0); phi'(x) = 1 (x > 0), 0 (x <= 0)
By the chain rule the gradients with respect to the raw q and k are
phi'(q) * dL/dphi(q) and phi'(k) * dL/dphi(k), elementwise.
"""
from __future__ import annotations

import numpy as np

KINDS = ("identity", "elu1", "relu")


def phi(x, kind: str) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    if kind == "identity":
        return x.copy()
    if kind == "elu1":
        return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))
    if kind == "relu":
        return np.where(x > 0, x, 0.0)
    raise ValueError(f"unknown feature map {kind!r}")


def dphi(x, kind: str) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    if kind == "identity":
        return np.ones_like(x)
    if kind == "elu1":
        return np.where(x > 0, 1.0, np.exp(np.minimum(x, 0.0)))
    if kind == "relu":
        return np.where(x > 0, 1.0, 0.0)
    raise ValueError(f"unknown feature map {kind!r}")
