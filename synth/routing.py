"""Seeded synthetic MoE routing: router logits drawn N(0, 1), top-k experts per
token with softmax weights over the chosen k.

The "TurboEXL3" article (section 3.1 and section 5, model description) routes
each token to 10 of 512 experts with a softmax over the router scores, plus one
shared expert that every token visits.  Here the chosen experts are the k
largest logits (ties go to the lower expert id), their weights are the softmax
of those k logits (the same as a softmax over all experts renormalised over the
chosen ones), computed in float64 and stored as float32, and each token's list
is ordered by descending weight.

This module holds no part of the dequantize/multiply arithmetic: the routing is
an input of the grouped MoE call.
"""

from __future__ import annotations

import numpy as np

from . import rng


def router_logits(t: int, num_experts: int, *, seed: int = rng.BASE_SEED,
                  name: str = "router") -> np.ndarray:
    return rng.normal_matrix(seed, name, t, num_experts, 1.0).astype(np.float32)


def topk_softmax(logits: np.ndarray, k: int):
    """(ids int32 [t][k], weights float32 [t][k])."""
    t, e = logits.shape
    lg = logits.astype(np.float64)
    # stable sort on (-logit) keeps the lower id first among equal logits
    order = np.argsort(-lg, axis=1, kind="stable")[:, :k]
    top = np.take_along_axis(lg, order, axis=1)
    z = np.exp(top - top[:, :1])
    w = z / z.sum(axis=1, keepdims=True)
    return order.astype(np.int32), w.astype(np.float32)


def synthetic_routing(t: int, num_experts: int, k: int, *, seed: int = rng.BASE_SEED,
                      name: str = "router"):
    return topk_softmax(router_logits(t, num_experts, seed=seed, name=name), k)
