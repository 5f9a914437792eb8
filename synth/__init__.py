"""Seeded synthetic inputs shared by the CPU oracle tests and the HIP path.

This module draws random numbers and nothing else: it holds none of the
arithmetic of softmax, RMSNorm, LayerNorm or cross-entropy.  Both sides of
every parity check take their inputs from here, so the oracle and the GPU
kernels never exchange data except through these arrays.

Generator
---------
SplitMix64 (G. Steele, D. Lea, C. Flood, "Fast splittable pseudorandom number
generators", OOPSLA 2014) used as a counter-based generator: output ``i`` of a
stream is ``mix(state0 + (i + 1) * GOLDEN)``, where ``mix`` is the SplitMix64
finaliser.  Every tensor draws from its own stream, keyed by ``(seed, stream)``:

    state0(seed, stream) = mix(mix(seed) ^ (stream * GOLDEN_2))

* uniform doubles in [0, 1): ``(u >> 11) * 2**-53``
* normals: Box-Muller (G. Box, M. Muller, 1958) on consecutive uniform pairs
  ``(u1, u2)``: ``r = sqrt(-2 ln(1 - u1))``, ``z0 = r cos(2 pi u2)``,
  ``z1 = r sin(2 pi u2)``; computed in double, rounded once to float32 after the
  affine ``mean + std * z``.
* integer labels uniform in ``[lo, hi)``: ``lo + floor(u01 * (hi - lo))``.

Stream ids used by the workloads: x = 0, gamma = 1, beta = 2, labels = 3.
"""
from __future__ import annotations

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
GOLDEN_2 = np.uint64(0xD1B54A32D192ED03)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

STREAM_X = 0
STREAM_GAMMA = 1
STREAM_BETA = 2
STREAM_LABELS = 3
STREAM_RESIDUAL = 4

_CHUNK = 1 << 22  # values generated per numpy pass (bounds temporary memory)


def _mix(z: np.ndarray) -> np.ndarray:
    """SplitMix64 finaliser, elementwise on uint64 (wraps modulo 2**64)."""
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def _mix_scalar(z: int) -> int:
    m = (1 << 64) - 1
    z &= m
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & m
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & m
    return z ^ (z >> 31)


def stream_state(seed: int, stream: int) -> int:
    """Initial SplitMix64 state of ``stream`` under ``seed``."""
    m = (1 << 64) - 1
    return _mix_scalar(_mix_scalar(seed) ^ ((stream * 0xD1B54A32D192ED03) & m))


def raw_u64(seed: int, stream: int, start: int, count: int) -> np.ndarray:
    """Outputs ``start .. start+count-1`` of the stream as uint64."""
    s0 = np.uint64(stream_state(seed, stream))
    with np.errstate(over="ignore"):
        i = np.arange(start + 1, start + 1 + count, dtype=np.uint64)
        return _mix(s0 + i * GOLDEN)


def uniform01(seed: int, stream: int, count: int, start: int = 0) -> np.ndarray:
    """``count`` doubles in [0, 1) with 53 random bits each."""
    out = np.empty(count, dtype=np.float64)
    for a in range(0, count, _CHUNK):
        n = min(_CHUNK, count - a)
        u = raw_u64(seed, stream, start + a, n)
        out[a:a + n] = (u >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)
    return out


def normal_f32(seed: int, stream: int, count: int, mean: float = 0.0,
               std: float = 1.0) -> np.ndarray:
    """``count`` float32 draws of N(mean, std**2) by Box-Muller."""
    out = np.empty(count, dtype=np.float32)
    pairs = (count + 1) // 2
    step = _CHUNK // 2
    for a in range(0, pairs, step):
        n = min(step, pairs - a)
        u = raw_u64(seed, stream, 2 * a, 2 * n)
        u = (u >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)
        u1, u2 = u[0::2], u[1::2]
        r = np.sqrt(-2.0 * np.log1p(-u1))
        t = (2.0 * np.pi) * u2
        z = np.empty(2 * n, dtype=np.float64)
        z[0::2] = r * np.cos(t)
        z[1::2] = r * np.sin(t)
        lo = 2 * a
        hi = min(count, lo + 2 * n)
        out[lo:hi] = (mean + std * z[: hi - lo]).astype(np.float32)
    return out


def uniform_f32(seed: int, stream: int, count: int, lo: float, hi: float) -> np.ndarray:
    """``count`` float32 draws of U(lo, hi)."""
    return (lo + (hi - lo) * uniform01(seed, stream, count)).astype(np.float32)


def labels_i64(seed: int, stream: int, count: int, lo: int, hi: int) -> np.ndarray:
    """``count`` int64 labels uniform in [lo, hi)."""
    u = uniform01(seed, stream, count)
    return (lo + np.floor(u * (hi - lo))).astype(np.int64)


# ---------------------------------------------------------------------------
# The five workloads (shapes and distributions of the pages' held-out cases
# plus the cross-entropy case).  Each returns a dict of numpy arrays.
# ---------------------------------------------------------------------------

def softmax_inputs(rows: int, cols: int, seed: int = 0, std: float = 1.0) -> dict:
    return {"x": normal_f32(seed, STREAM_X, rows * cols, 0.0, std).reshape(rows, cols)}


def rmsnorm_inputs(rows: int, cols: int, seed: int = 0) -> dict:
    return {
        "x": normal_f32(seed, STREAM_X, rows * cols).reshape(rows, cols),
        "gamma": uniform_f32(seed, STREAM_GAMMA, cols, 0.5, 1.5),
    }


def layernorm_inputs(rows: int, cols: int, seed: int = 0, mean: float = 0.0,
                     std: float = 1.0) -> dict:
    return {
        "x": normal_f32(seed, STREAM_X, rows * cols, mean, std).reshape(rows, cols),
        "gamma": uniform_f32(seed, STREAM_GAMMA, cols, 0.5, 1.5),
        "beta": normal_f32(seed, STREAM_BETA, cols, 0.0, 0.1),
    }


def add_layernorm_inputs(rows: int, cols: int, seed: int = 0, mean: float = 0.0,
                         std: float = 1.0) -> dict:
    """Fused residual LayerNorm: x and residual N(mean, std^2) from their own
    streams, gamma and beta as for LayerNorm."""
    d = layernorm_inputs(rows, cols, seed, mean, std)
    d["residual"] = normal_f32(seed, STREAM_RESIDUAL, rows * cols, mean, std).reshape(rows, cols)
    return d


def cross_entropy_inputs(rows: int, cols: int, seed: int = 0, std: float = 2.0) -> dict:
    return {
        "logits": normal_f32(seed, STREAM_X, rows * cols, 0.0, std).reshape(rows, cols),
        "labels": labels_i64(seed, STREAM_LABELS, rows, 0, cols),
    }


#: The five workloads: name -> (op, rows, cols, generator kwargs, eps, policies)
WORKLOADS = {
    "softmax_37x1537": dict(op="softmax", rows=37, cols=1537, gen=dict(std=4.0),
                            eps=None, policies=("unordered_tree",)),
    "rmsnorm_256x3072": dict(op="rmsnorm", rows=256, cols=3072, gen={}, eps=1e-6,
                             policies=("unordered_tree", "ordered_fold")),
    "layernorm_64x12289": dict(op="layernorm", rows=64, cols=12289,
                               gen=dict(mean=3.0, std=2.0), eps=1e-5,
                               policies=("unordered_tree",)),
    "softmax_768x6144": dict(op="softmax", rows=768, cols=6144, gen={}, eps=None,
                             policies=("unordered_tree",)),
    "rmsnorm_768x6144": dict(op="rmsnorm", rows=768, cols=6144, gen={}, eps=1e-6,
                             policies=("unordered_tree",)),
    "layernorm_768x6144": dict(op="layernorm", rows=768, cols=6144, gen={}, eps=1e-5,
                               policies=("unordered_tree",)),
    "cross_entropy_4096x32000": dict(op="cross_entropy", rows=4096, cols=32000,
                                     gen={}, eps=None, policies=("unordered_tree",)),
}

_GEN = {
    "softmax": softmax_inputs,
    "rmsnorm": rmsnorm_inputs,
    "layernorm": layernorm_inputs,
    "cross_entropy": cross_entropy_inputs,
    "add_layernorm": add_layernorm_inputs,
}


def make_inputs(op: str, rows: int, cols: int, seed: int = 0, **kw) -> dict:
    """Inputs of ``op`` at ``rows x cols`` with the workload distributions."""
    return _GEN[op](rows, cols, seed=seed, **kw)


def workload_inputs(name: str, seed: int = 0) -> dict:
    w = WORKLOADS[name]
    return make_inputs(w["op"], w["rows"], w["cols"], seed=seed, **w["gen"])
