"""Seeded synthetic MoE inputs: router logits, and routing tables drawn at
random.

The "TurboEXL3" article (section 3.1 and the model description in section 5)
routes each token to 10 of 512 experts, plus one shared expert that every
token visits.  Two kinds of input are produced here:

* ``router_logits``: logits drawn N(0, 1) per (token, expert), the input of
  the router (top-k and softmax, which the library computes on the GPU and
  the oracle on the CPU);
* ``random_routing``: a routing table that does not come from any router:
  per token, k distinct expert ids drawn uniformly without replacement (a
  partial Fisher-Yates shuffle driven by counter-based uniforms), and k
  positive weights drawn uniformly and divided by their sum.  It has the
  statistics of top-k over i.i.d. logits (every expert equally likely, k
  distinct per token) and is what the grouped-MoE parity tests feed in.

This module holds no part of the method's arithmetic: no ranking of logits,
no softmax, no dequantizing or multiplying.
"""

from __future__ import annotations

import numpy as np

from . import rng


def router_logits(t: int, num_experts: int, *, seed: int = rng.BASE_SEED,
                  name: str = "router") -> np.ndarray:
    """Logits N(0, 1), float32 [t][num_experts]."""
    return rng.normal_matrix(seed, name, t, num_experts, 1.0).astype(np.float32)


def random_routing(t: int, num_experts: int, k: int, *, seed: int = rng.BASE_SEED,
                   name: str = "routing"):
    """(ids int32 [t][k], weights float32 [t][k]): k distinct uniform expert
    ids per token and positive weights that sum to one (up to float32
    rounding)."""
    if not 1 <= k <= num_experts:
        raise ValueError(f"k={k} must lie in 1..{num_experts}")
    u = rng.uniform_matrix(seed, name + "/pick", t, k)
    perm = np.tile(np.arange(num_experts, dtype=np.int64), (t, 1))
    rows = np.arange(t)
    for j in range(k):
        # swap position j with a uniform position in j .. E-1
        r = j + np.minimum((u[:, j] * (num_experts - j)).astype(np.int64), num_experts - j - 1)
        a = perm[rows, j].copy()
        perm[rows, j] = perm[rows, r]
        perm[rows, r] = a
    ids = perm[:, :k].astype(np.int32)
    v = rng.uniform_matrix(seed, name + "/weight", t, k) + 0.05
    w = (v / v.sum(axis=1, keepdims=True)).astype(np.float32)
    return ids, w
