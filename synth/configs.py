"""Model shapes of the workloads and their seeded random weights.

Weight layout (shared convention of both sides, data only):
  * every matrix is ``[out_features, in_features]`` row-major;
  * ``w_qkv`` stacks the Q rows (nq*d), then K rows (nkv*d), then V rows
    (nkv*d), heads contiguous inside each block;
  * for the SwiGLU feed-forward ``w1`` stacks the gate rows (F) then the up
    rows (F), so it is ``[2F, H]``;
  * GPT-style layers carry biases and LayerNorm (gamma, beta); Llama-style
    layers carry RMSNorm gamma only and no biases.

Initialisation: every matrix is N(0, s^2) with s = min(0.02, 1/sqrt(fan_in));
embeddings and biases N(0, 0.02^2); norm gains 1 + N(0, 0.1^2) and LayerNorm
shifts N(0, 0.02^2), so that a kernel that drops a gain or a shift is caught by
a parity test.  s = 0.02 for the toy and mini shapes (fan_in <= 2500); for
hidden sizes of 4096 and 12288 the 1/sqrt(fan_in) cap keeps projections near
unit variance -- with 0.02 there, attention scores would have a standard
deviation of ~5 (near one-hot softmax), and the layer output would jump with
single-ulp differences of its inputs.
"""
from dataclasses import dataclass, replace

import numpy as np

from .gen import normal


def init_std(fan_in: int) -> float:
    """Standard deviation of a random weight matrix with ``fan_in`` inputs."""
    return min(0.02, fan_in ** -0.5)


def kv_std(m) -> float:
    """Scale of synthetic cached K/V rows: that of a normalised row times a projection matrix."""
    return min(0.02 * m.H ** 0.5, 1.0)


@dataclass(frozen=True)
class ModelDims:
    name: str
    arch: str          # 'gpt' (LayerNorm, biases, GeLU, learned positions) or 'llama'
    n_layers: int
    H: int
    nq: int
    nkv: int
    d: int
    F: int
    V: int
    max_pos: int = 2048
    eps: float = 1e-5
    rope_theta: float = 500000.0

    @property
    def qkv_out(self) -> int:
        return (self.nq + 2 * self.nkv) * self.d

    @property
    def group(self) -> int:
        return self.nq // self.nkv

    def with_layers(self, n: int) -> "ModelDims":
        return replace(self, n_layers=n)


# 2-layer GPT decoder used for the Figure-5 walk-through (fp32).
TOY = ModelDims("toy-gpt", "gpt", n_layers=2, H=64, nq=4, nkv=4, d=16, F=256, V=256)
# The ~13M-parameter mini model of the CPU measurement (64 decodes).
MINI = ModelDims("mini-gpt", "gpt", n_layers=4, H=256, nq=8, nkv=8, d=32, F=1024, V=4096)
# Llama-3-8B-shaped decoder: GQA 32/8, head_dim 128, SwiGLU 14336, RMSNorm, RoPE.
LLAMA8B = ModelDims("llama3-8b-shape", "llama", n_layers=32, H=4096, nq=32, nkv=8, d=128,
                    F=14336, V=128256, max_pos=0, eps=1e-5, rope_theta=500000.0)
# GPT-175B-shaped single layer (H 12288, 96 heads, FFN 49152, GeLU).
GPT175B_LAYER = ModelDims("gpt175b-layer", "gpt", n_layers=1, H=12288, nq=96, nkv=96, d=128,
                          F=49152, V=0, max_pos=2048)


def qkv_rows(m: ModelDims) -> int:
    return m.qkv_out


def ffn1_rows(m: ModelDims) -> int:
    return 2 * m.F if m.arch == "llama" else m.F


def make_layer_weights(m: ModelDims, seed: int, layer: int, dtype: str) -> dict:
    """Weights of one decoder layer (float32 arrays, ``dtype``-representable)."""
    p = f"L{layer}."
    H, F = m.H, m.F
    w = {}
    w["ln1_g"] = normal(seed, p + "ln1_g", (H,), std=0.1, mean=1.0, dtype=dtype)
    w["w_qkv"] = normal(seed, p + "w_qkv", (m.qkv_out, H), std=init_std(H), dtype=dtype)
    w["w_o"] = normal(seed, p + "w_o", (H, m.nq * m.d), std=init_std(m.nq * m.d), dtype=dtype)
    w["ln2_g"] = normal(seed, p + "ln2_g", (H,), std=0.1, mean=1.0, dtype=dtype)
    w["w1"] = normal(seed, p + "w1", (ffn1_rows(m), H), std=init_std(H), dtype=dtype)
    w["w2"] = normal(seed, p + "w2", (H, F), std=init_std(F), dtype=dtype)
    if m.arch == "gpt":
        w["ln1_b"] = normal(seed, p + "ln1_b", (H,), std=0.02, dtype=dtype)
        w["b_qkv"] = normal(seed, p + "b_qkv", (m.qkv_out,), std=0.02, dtype=dtype)
        w["b_o"] = normal(seed, p + "b_o", (H,), std=0.02, dtype=dtype)
        w["ln2_b"] = normal(seed, p + "ln2_b", (H,), std=0.02, dtype=dtype)
        w["b1"] = normal(seed, p + "b1", (F,), std=0.02, dtype=dtype)
        w["b2"] = normal(seed, p + "b2", (H,), std=0.02, dtype=dtype)
    return w


def make_weights(m: ModelDims, seed: int, dtype: str, layers=None) -> dict:
    """Full model weights: embeddings, ``layers`` (default all), final norm, LM head."""
    w = {"layers": []}
    if m.V > 0:
        w["tok_emb"] = normal(seed, "tok_emb", (m.V, m.H), std=0.02, dtype=dtype)
        w["w_lm"] = normal(seed, "w_lm", (m.V, m.H), std=init_std(m.H), dtype=dtype)
    if m.arch == "gpt" and m.max_pos > 0 and m.V > 0:
        w["pos_emb"] = normal(seed, "pos_emb", (m.max_pos, m.H), std=0.02, dtype=dtype)
    w["lnf_g"] = normal(seed, "lnf_g", (m.H,), std=0.1, mean=1.0, dtype=dtype)
    if m.arch == "gpt":
        w["lnf_b"] = normal(seed, "lnf_b", (m.H,), std=0.02, dtype=dtype)
    for l in (range(m.n_layers) if layers is None else layers):
        w["layers"].append(make_layer_weights(m, seed, l, dtype))
    return w
