"""Seeded synthetic inputs for the router workloads.

This module holds no router arithmetic: it draws logits, gradients and
expert biases from numpy's PCG64 generator in fp64 and rounds them to the
storage dtype (fp32 round-to-nearest-even; bf16 round-to-nearest-even from
the fp32 value).  The same bytes feed the HIP kernels and the CPU oracle.

Workloads follow the shapes of the fused-router benchmark tables in
"[Common] Optimize fused router forward/backward kernels" (NVIDIA
TransformerEngine pull request 3012, "Performance" section: T = 8192
tokens, E/K in {512, 2304} x {4, 8, 22, 36}); the pages do not state the
logit distribution, so the recipes below are the ones this library uses.
"""
from dataclasses import dataclass, field

import numpy as np

SOFTMAX = 0
SIGMOID = 1
F32 = 0
BF16 = 1


def normal(seed, shape, std=1.0):
    """fp64 N(0, std^2) draws from PCG64(seed)."""
    return np.random.default_rng(seed).normal(0.0, std, size=shape)


def uniform(seed, shape, lo, hi):
    """fp64 U(lo, hi) draws from PCG64(seed)."""
    return np.random.default_rng(seed).uniform(lo, hi, size=shape)


def to_f32(a):
    """Round to fp32, nearest-even."""
    return np.ascontiguousarray(a, dtype=np.float32)


def f32_to_bf16_bits(a):
    """Round fp32 values to bf16, nearest-even; returns the uint16 bit
    patterns.  Inputs are finite."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits):
    """Exact widening of bf16 bit patterns to fp32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32)
    return (b << np.uint32(16)).view(np.float32)


def storage(a64, dtype):
    """(bytes-array, fp64 value) of a fp64 array rounded to the storage
    dtype: fp32 array for F32, uint16 bf16 bit patterns for BF16."""
    f = to_f32(a64)
    if dtype == F32:
        return f, f.astype(np.float64)
    bits = f32_to_bf16_bits(f)
    return bits, bf16_bits_to_f32(bits).astype(np.float64)


@dataclass
class Workload:
    """One router configuration and the seeds of its synthetic inputs."""
    name: str
    T: int
    E: int
    K: int
    score_fn: int = SOFTMAX
    renorm: bool = False
    num_groups: int = 0
    group_topk: int = 0
    scaling_factor: float = 1.0
    dtype: int = F32
    logit_std: float = 1.0
    bias_range: float = 0.0          # 0 = no bias; else U(-r, r)
    grad_on_map: bool = False        # grad_probs multiplied by the map
    aux: bool = False                # also run the aux-score variant
    aux_renorm: bool = True
    seed_logits: int = 0
    seed_grad: int = 0
    seed_bias: int = 0
    seed_aux_grad: int = 0
    notes: str = field(default="")

    def logits(self):
        return storage(normal(self.seed_logits, (self.T, self.E),
                              self.logit_std), self.dtype)

    def grad(self):
        return storage(normal(self.seed_grad, (self.T, self.E)), self.dtype)

    def aux_grad(self):
        return storage(normal(self.seed_aux_grad, (self.T, self.E)),
                       self.dtype)

    def bias(self):
        """fp32 expert bias [E], or None."""
        if not self.bias_range:
            return None
        return to_f32(uniform(self.seed_bias, (self.E,), -self.bias_range,
                              self.bias_range))


def _wl(i, **kw):
    return Workload(seed_logits=1000 + i, seed_grad=2000 + i,
                    seed_bias=3000 + i, seed_aux_grad=4000 + i, **kw)


# The five router workloads.  "c4_softmax_2304x36" is the headline shape.
WORKLOADS = {
    "c1_softmax_16x2": _wl(1, name="c1_softmax_16x2", T=64, E=16, K=2),
    "c2_softmax_256x4": _wl(2, name="c2_softmax_256x4", T=8192, E=256, K=4,
                            grad_on_map=True),
    "c3_sigmoid_512x22": _wl(3, name="c3_sigmoid_512x22", T=8192, E=512,
                             K=22, score_fn=SIGMOID, renorm=True,
                             scaling_factor=2.5, bias_range=0.1, aux=True),
    "c4_softmax_2304x36": _wl(4, name="c4_softmax_2304x36", T=8192, E=2304,
                              K=36, logit_std=2.0, aux=True),
    "c5_group_sigmoid_256x8_bf16": _wl(
        5, name="c5_group_sigmoid_256x8_bf16", T=16384, E=256, K=8,
        score_fn=SIGMOID, renorm=True, num_groups=8, group_topk=4,
        scaling_factor=2.5, dtype=BF16, bias_range=0.05),
}


def sweep_workload(E, K, score_fn, T=8192):
    """Cell of the T=8192 E/K sweep (softmax without renormalisation, or
    sigmoid with renormalisation), seeded 5000 + E + K."""
    s = 5000 + E + K
    return Workload(name=f"sweep_{'softmax' if score_fn == SOFTMAX else 'sigmoid'}_{E}x{K}",
                    T=T, E=E, K=K, score_fn=score_fn,
                    renorm=(score_fn == SIGMOID), aux=True, seed_logits=s,
                    seed_grad=s + 1, seed_bias=s + 2, seed_aux_grad=s + 3)


# ------------------------------------------------------ aux-loss inputs
#
# The aux loss consumes aux scores [T,E] (probabilities, so non-negative and
# of order 1/E) and per-expert token counts.  Isolated tests draw them
# directly: scores U(0, 2/E) (mean 1/E, like a probability row) and routing
# maps with exactly K ones per row at uniformly random columns.

AUX_LOSS_COEFF = 1e-2    # a typical balancing-loss coefficient


def prob_like(seed, T, E, dtype=F32):
    """(storage, fp64) scores U(0, 2/E) rounded to the storage dtype."""
    return storage(uniform(seed, (T, E), 0.0, 2.0 / E), dtype)


def random_map(seed, T, E, K):
    """uint8 [T,E], exactly K ones per row at columns drawn uniformly
    without replacement (PCG64(seed))."""
    rng = np.random.default_rng(seed)
    m = np.zeros((T, E), np.uint8)
    if T and K:
        cols = np.argpartition(rng.random((T, E)), K - 1, axis=1)[:, :K]
        np.put_along_axis(m, cols, 1, axis=1)
    return m
