"""Seeded synthetic inputs for the BitLinear forward path.

This module only draws random numbers and lays them out in the shapes of the
workloads the BitNet pages describe; it holds none of the method's arithmetic
(no scales, no rounding to codes, no contraction).  Both the CPU oracle and the
GPU path read their inputs from here, so the two sides always see the same
bits.

Streams: every array comes from its own PCG64 stream, addressed by
``SeedSequence(0, spawn_key=(stream, layer, projection, kind, extra))``, with
``stream`` a workload's fixed id, so any single tensor can be regenerated
without drawing the others.

Shapes follow ``nn.Linear``: a weight is ``[N][K]`` (out x in, fp32 row-major),
an activation is ``[M][K]`` carried as bf16 bit patterns (``uint16``).
"""

from __future__ import annotations

import numpy as np

SEED = 0

# kind ids used in spawn keys
_W, _X, _MASK, _FLIP, _COUNT, _GRAD = 0, 1, 2, 3, 4, 5

PROJ_IDS = {"q": 0, "k": 1, "v": 2, "o": 3, "gate": 4, "up": 5, "down": 6, "w": 7}
# which activation each projection consumes (q/k/v share one input, gate/up another)
INPUT_OF = {"q": "qkv", "k": "qkv", "v": "qkv", "o": "o", "gate": "gateup",
            "up": "gateup", "down": "down", "w": "x"}
INPUT_IDS = {"qkv": 0, "o": 1, "gateup": 2, "down": 3, "x": 4}


def _llama_layer(hidden, ffn, kv_out=None):
    kv = hidden if kv_out is None else kv_out
    # (N = out, K = in)
    return {"q": (hidden, hidden), "k": (kv, hidden), "v": (kv, hidden), "o": (hidden, hidden),
            "gate": (ffn, hidden), "up": (ffn, hidden), "down": (hidden, ffn)}


# The five workloads, by what they are.  "stream" is the fixed id in their
# random streams; "layers" is the number of transformer layers whose BitLinear
# tensors take part; "M" lists the token counts; "x" names the activation
# recipe.
WORKLOADS = {
    "linear_256x512": dict(stream=1, name="single BitLinear K=256->N=512, M=32",
                           layers=1, tensors={"w": (512, 256)}, M=(32,), x="channels"),
    "model_16m": dict(stream=2, name="6-layer 16.4M-param model, 42 BitLinear tensors, M=8192 (+ sign-flip tracker)",
                      layers=6, tensors=_llama_layer(256, 512, kv_out=128), M=(8192,), x="channels"),
    "layer_700m": dict(stream=3, name="700M LLaMA-shape layer prefill, M=2048",
                       layers=1, tensors=_llama_layer(1536, 4096), M=(2048,), x="bernoulli"),
    "layer_3b": dict(stream=4, name="3B LLaMA-shape layer decode, M=1/8",
                     layers=1, tensors=_llama_layer(3200, 8640), M=(1, 8), x="plain"),
    "layer_70b": dict(stream=5, name="70B LLaMA-shape layer decode, M=1/16/64",
                      layers=1, tensors=_llama_layer(8192, 28672, kv_out=1024), M=(1, 16, 64), x="plain"),
}


def stream_id(name: str) -> int:
    return WORKLOADS[name]["stream"]


def rng(*key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(SEED, spawn_key=tuple(int(k) for k in key))))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------- generic draws

def gaussian_weight(N: int, K: int, key=(0,), sigma: float = 0.02) -> np.ndarray:
    """fp32 [N][K], sigma * N(0,1) drawn in fp32."""
    w = rng(*key).standard_normal((N, K), dtype=np.float32)
    w *= np.float32(sigma)
    return w


def activation(M: int, K: int, key=(0,), recipe: str = "plain") -> np.ndarray:
    """bf16 bits [M][K]: N(0,1) in fp32, outliers applied, then RNE to bf16.

    recipe "channels": 4 channels drawn without replacement, scaled x20.
    recipe "bernoulli": each element independently (p = 0.001) scaled x50.
    recipe "plain": no outliers.
    """
    g = rng(*key)
    x = g.standard_normal((M, K), dtype=np.float32)
    if recipe == "channels":
        ch = rng(*key, _MASK).choice(K, size=min(4, K), replace=False)
        x[:, ch] *= np.float32(20.0)
    elif recipe == "bernoulli":
        mask = rng(*key, _MASK).random((M, K)) < 0.001
        x[mask] *= np.float32(50.0)
    elif recipe != "plain":
        raise ValueError(recipe)
    return f32_to_bf16_bits(x)


# ---------------------------------------------------------- workload tensors

def workload_weight(name: str, proj: str, layer: int = 0) -> np.ndarray:
    N, K = WORKLOADS[name]["tensors"][proj]
    w = gaussian_weight(N, K, key=(stream_id(name), layer, PROJ_IDS[proj], _W))
    return w


def workload_activation(name: str, proj: str, M: int, layer: int = 0) -> np.ndarray:
    """The activation consumed by ``proj`` (q/k/v share one, gate/up share one)."""
    K = WORKLOADS[name]["tensors"][proj][1]
    inp = INPUT_OF[proj]
    return activation(M, K, key=(stream_id(name), layer, INPUT_IDS[inp] + 16, _X, M), recipe=WORKLOADS[name]["x"])


def workload_tensors(name: str):
    """[(layer, proj, N, K)] in the fixed order layer-major, projection order q k v o gate up down."""
    c = WORKLOADS[name]
    return [(l, p, N, K) for l in range(c["layers"]) for p, (N, K) in c["tensors"].items()]


# --------------------------------------------------------- sign-flip tracker

def flip_snapshots(name: str = "model_16m", frac: float = 0.05):
    """Two flat weight snapshots over all tensors of workload ``name``
    (concatenated in workload_tensors order).  ``curr`` equals ``prev`` with exactly
    round(frac * n_t) entries of each tensor, chosen without replacement,
    sign-negated.  Returns (prev, curr, perturbed_mask)."""
    parts_prev, parts_mask = [], []
    for (l, p, N, K) in workload_tensors(name):
        w = workload_weight(name, p, l).reshape(-1)
        assert np.all(w != 0), "generator produced an exact zero"
        n = w.size
        idx = rng(stream_id(name), l, PROJ_IDS[p], _FLIP).choice(n, size=int(round(frac * n)), replace=False)
        m = np.zeros(n, dtype=bool)
        m[idx] = True
        parts_prev.append(w)
        parts_mask.append(m)
    prev = np.concatenate(parts_prev)
    mask = np.concatenate(parts_mask)
    curr = prev.copy()
    curr[mask] = -curr[mask]
    return prev, curr, mask


def flip_counters(n: int, scenario: int, name: str = "model_16m"):
    """(flip_count int16[n], last_flip int16[n], step).

    scenario 1: counters start at zero, first step after a 100-step warm-up.
    scenario 2: counters pre-seeded (flip_count ~ U{0..900}, last_flip ~ U{0..1000}), step 1000.
    """
    if scenario == 1:
        return np.zeros(n, np.int16), np.zeros(n, np.int16), 101
    g = rng(stream_id(name), 99, 0, _COUNT)
    fc = g.integers(0, 901, size=n, dtype=np.int16)
    lf = g.integers(0, 1001, size=n, dtype=np.int16)
    return fc, lf, 1000


def adam_grad(n: int, step: int, name: str = "model_16m", sigma: float = 2.5e-4) -> np.ndarray:
    """fp32 [n] gradient for optimiser step ``step``: sigma * N(0,1) drawn in
    fp32.  The default sigma puts the global norm of a 16.4M-parameter model
    at about 1, the gradient-clip threshold of the 1-bit training runs."""
    g = rng(stream_id(name), 98, step, _GRAD).standard_normal(n, dtype=np.float32)
    g *= np.float32(sigma)
    return g


def lr_schedule(step: int, peak: float = 3e-4, floor: float = 3e-5, warmup: int = 100, total: int = 1000) -> float:
    """Linear warm-up to ``peak`` over ``warmup`` steps, then cosine decay to
    ``floor`` at ``total`` (the 1-bit training runs' schedule)."""
    if step <= warmup:
        return peak * step / warmup
    u = min(1.0, (step - warmup) / (total - warmup))
    return float(floor + 0.5 * (peak - floor) * (1.0 + np.cos(np.pi * u)))
