"""Seeded synthetic inputs for the router + align path.

This module holds input recipes only -- none of the routing arithmetic.  Both
the HIP path and the CPU oracle consume the bf16 bit patterns it returns, so
the two sides always see identical inputs.

Recipe (draw order x -> W -> ws -> permutation, numpy default_rng(seed), all
draws in float64, then converted to bf16 by torch's float64 -> bfloat16 cast):

* ``normal``: x ~ N(0, 1); gate rows W and the shared gate row ws ~ N(0, 0.02^2).
* ``int``: x, W, ws = integers uniform in {-3..3} times 2^-4.  Every product is a
  multiple of 2^-8 and every partial sum stays below 2^8 in magnitude, so any
  fp32 or fp64 summation order gives the exact logit, and the bf16 rounding of
  those logits produces many ties (this pins the lowest-id tie rule).
* ``zipf``: ``normal``, then x[:, 0] = 1 and W[e, 0] = ln(E * p(rho_e)) with
  p(rho) = rho^-1.1 / sum_{j=1..E} j^-1.1 and rho a seeded permutation of 1..E,
  so a per-expert offset skews routing the way real prefill routing is skewed.

The workloads stand in for the real activations, captured routing and trained
gate weights the source pages measured with; none of those are available.
"""
from __future__ import annotations

import dataclasses

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    M: int
    E: int
    H: int
    k: int
    shared: bool
    dist: str = "normal"
    scale: float = 1.0
    seed: int = 0

    @property
    def S(self) -> int:
        return self.k + int(self.shared)

    @property
    def num_experts(self) -> int:
        """Expert ids the align step sees (the shared expert is id E)."""
        return self.E + int(self.shared)


# The five workloads: small-M decode router (E=512 routed + 1 shared, top-10,
# H=4096), the same at M=8 on exactly representable inputs, an E=128 top-8
# prefill at M=128 and a skewed one at M=2048, and an M sweep at E=512.
ROUTER_E512_M4 = Workload("router_e512_h4096_k10_m4", 4, 512, 4096, 10, True)
ROUTER_E512_M8_EXACT = Workload("router_e512_h4096_k10_m8_exact", 8, 512, 4096, 10, True, "int")
PREFILL_E128_M128 = Workload("prefill_e128_h2048_k8_m128", 128, 128, 2048, 8, False)
PREFILL_E128_M2048_ZIPF = Workload("prefill_e128_h2048_k8_m2048_zipf", 2048, 128, 2048, 8, False, "zipf")
SWEEP_M = (1, 2, 3, 8, 9, 16, 40, 512, 2048)


def sweep_workload(M: int) -> Workload:
    return Workload(f"router_e512_h4096_k10_m{M}", M, 512, 4096, 10, True)


ALL_WORKLOADS = (ROUTER_E512_M4, ROUTER_E512_M8_EXACT, PREFILL_E128_M128,
                 PREFILL_E128_M2048_ZIPF) + tuple(sweep_workload(m) for m in SWEEP_M)


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float64 array -> bf16 bit patterns (uint16) via torch's cast."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def make_inputs(M: int, E: int, H: int, shared: bool, dist: str = "normal",
                seed: int = 0) -> dict:
    """Returns dict(x=[M, H] uint16, w=[E, H] uint16, ws=[H] uint16 or None)."""
    rng = np.random.default_rng(seed)
    if dist == "int":
        x = rng.integers(-3, 4, size=(M, H)).astype(np.float64) * 2.0 ** -4
        w = rng.integers(-3, 4, size=(E, H)).astype(np.float64) * 2.0 ** -4
        ws = rng.integers(-3, 4, size=H).astype(np.float64) * 2.0 ** -4 if shared else None
    elif dist in ("normal", "zipf"):
        x = rng.standard_normal((M, H))
        w = rng.standard_normal((E, H)) * 0.02
        ws = rng.standard_normal(H) * 0.02 if shared else None
        if dist == "zipf":
            rho = rng.permutation(E) + 1
            j = np.arange(1, E + 1, dtype=np.float64)
            p = rho.astype(np.float64) ** -1.1 / np.sum(j ** -1.1)
            x[:, 0] = 1.0
            w[:, 0] = np.log(E * p)
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    return {
        "x": to_bf16_bits(x),
        "w": to_bf16_bits(w),
        "ws": None if ws is None else to_bf16_bits(ws),
    }


def workload_inputs(wl: Workload) -> dict:
    return make_inputs(wl.M, wl.E, wl.H, wl.shared, wl.dist, wl.seed)
