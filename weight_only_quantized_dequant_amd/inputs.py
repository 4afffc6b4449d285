"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle checks.

This module holds random-number generation and shapes only. It does no
quantization, packing, rounding rule or product of the method. Both sides (the device
path and the CPU oracle) receive the same arrays from here.

Weights are ``0.02 * N(0,1)`` in fp32 and activations are ``N(0,1)`` rounded to fp16.
This is the random-init stand-in for trained Llama weights: the device path has no
data-dependent branches, so time depends only on shapes and bytes.
"""

import numpy as np

SEED = 0

# Linear shapes (N, K) of the decode layers, by model.
LLAMA2_7B_LINEARS = [
    ("q", 4096, 4096), ("k", 4096, 4096), ("v", 4096, 4096), ("o", 4096, 4096),
    ("gate", 11008, 4096), ("up", 11008, 4096), ("down", 4096, 11008),
]
LLAMA_70B_LINEARS = [
    ("q", 8192, 8192), ("k", 1024, 8192), ("v", 1024, 8192), ("o", 8192, 8192),
    ("gate", 28672, 8192), ("up", 28672, 8192), ("down", 8192, 28672),
]

# Named workloads: format name, list of (N, K), list of M.
WORKLOADS = {
    "w8_single_1024x1024": ("w8", [(1024, 1024)], [1]),
    "llama7b_w4g32_linears": ("w4g32", [(4096, 4096), (11008, 4096), (4096, 11008)], [1]),
    "llama70b_w6e3m2_linears": ("w6e3m2", [(8192, 8192), (1024, 8192), (28672, 8192), (8192, 28672)], [1, 4, 8, 16]),
    # one GPU's shard of the 70B layer under 8-way tensor parallelism: fused q/k/v and gate/up
    # split by output rows (column-parallel), o and down split along K (row-parallel)
    "llama70b_w6e3m2_tp8_shard": ("w6e3m2", [(1280, 8192), (8192, 1024), (3584, 8192), (3584, 8192), (8192, 3584)],
                                  [1, 4, 8, 16]),
    # the same Llama-7B linears with int8 and FP6 weights (the other two formats of the 7B decode sweep)
    "llama7b_w8_linears": ("w8", [(4096, 4096), (11008, 4096), (4096, 11008)], [1, 4, 8, 16]),
    "llama7b_w6e3m2_linears": ("w6e3m2", [(4096, 4096), (11008, 4096), (4096, 11008)], [1, 4, 8, 16]),
    # the Llama-7B linears again with FP4 e2m1 weights (a further bit width)
    "llama7b_w4e2m1_linears": ("w4e2m1", [(4096, 4096), (11008, 4096), (4096, 11008)], [1, 4, 8, 16]),
    # and with FP5 e2m2 weights
    "llama7b_w5e2m2_linears": ("w5e2m2", [(4096, 4096), (11008, 4096), (4096, 11008)], [1, 4, 8, 16]),
    # bfloat16 activations: the Llama-7B W4 and Llama-70B W6 linears (x from the same kind of
    # draws, rounded to bfloat16 by the caller)
    "llama7b_w4g32_bf16_linears": ("w4g32_bf16", [(4096, 4096), (11008, 4096), (4096, 11008)], [1, 4, 8, 16]),
    "llama70b_w6e3m2_bf16_linears": ("w6e3m2_bf16", [(8192, 8192), (1024, 8192), (28672, 8192), (8192, 28672)],
                                     [1, 4, 8, 16]),
    # the Llama-7B linears with int3 weights (a further bit width)
    "llama7b_w3g32_linears": ("w3g32", [(4096, 4096), (11008, 4096), (4096, 11008)], [1, 4, 8, 16]),
    # FP6 in the 2+4 split layout: the same draws as the W6 workloads (same stream), so that the two
    # layouts of one set of weights can be timed side by side
    "llama70b_w6e3m2_p24_linears": ("w6e3m2_p24", [(8192, 8192), (1024, 8192), (28672, 8192), (8192, 28672)],
                                    [1, 4, 8, 16]),
    "llama7b_w6e3m2_p24_linears": ("w6e3m2_p24", [(4096, 4096), (11008, 4096), (4096, 11008)], [1, 4, 8, 16]),
}
# stream index of each workload, so that every workload draws from its own stream
WORKLOAD_STREAM = {"w8_single_1024x1024": 0, "llama7b_w4g32_linears": 1, "llama70b_w6e3m2_linears": 2,
                   "llama70b_w6e3m2_tp8_shard": 3, "llama7b_w4e2m1_linears": 4, "llama7b_w4g32_bf16_linears": 5,
                   "llama70b_w6e3m2_bf16_linears": 6, "llama7b_w5e2m2_linears": 7, "llama7b_w8_linears": 8,
                   "llama7b_w6e3m2_linears": 9, "llama7b_w3g32_linears": 12, "llama70b_w6e3m2_p24_linears": 2,
                   "llama7b_w6e3m2_p24_linears": 9}


# Decode sweeps over a whole random-init model: the linears of one layer, the layer count, and
# the stream its seeded draws come from. Every layer holds a copy of one draw per distinct shape
# (time depends only on shapes and bytes).
SWEEP_MODELS = {
    "llama2_7b": (LLAMA2_7B_LINEARS, 32, 10),
    "llama70b_w6": (LLAMA_70B_LINEARS, 80, 11),
}


def sweep_draws(model, m):
    """{(N, K): (W fp32, x fp16 bits [m, K])} for the distinct linear shapes of a sweep model, the
    i-th shape in sorted order drawn from rng_for(stream, i)."""
    shapes, _, stream = SWEEP_MODELS[model]
    distinct = sorted({(n, k) for _, n, k in shapes})
    return {(n, k): weights_and_x(rng_for(stream, i), n, k, m) for i, (n, k) in enumerate(distinct)}


def sweep_x(draws):
    """The activation rows of each K in a sweep (the x of the first distinct shape with that K)."""
    out = {}
    for (n, k) in sorted(draws):
        out.setdefault(k, draws[(n, k)][1])
    return out


def rng_for(stream, linear):
    """The generator for one linear of one workload."""
    return np.random.default_rng([SEED, stream, linear])


def weights_and_x(rng, n, k, m):
    """Draw W (fp32 [n,k]) first, then x (fp16 bits [m,k]), from one generator."""
    w = 0.02 * rng.standard_normal((n, k), dtype=np.float32)
    x = rng.standard_normal((m, k), dtype=np.float32).astype(np.float16).view(np.uint16)
    return w.astype(np.float32), x


def x_only(rng, m, k):
    return rng.standard_normal((m, k), dtype=np.float32).astype(np.float16).view(np.uint16)


def small_case(seed, n, k, m, scale=0.02):
    """A small seeded case for parity tests."""
    rng = np.random.default_rng([SEED, 100, seed])
    w = (scale * rng.standard_normal((n, k), dtype=np.float32)).astype(np.float32)
    x = rng.standard_normal((m, k), dtype=np.float32).astype(np.float16).view(np.uint16)
    return w, x
