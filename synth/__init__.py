"""Seeded synthetic calibration inputs for the AWQ search path.

This module only draws random numbers: it holds none of the method's
arithmetic, so both the CPU oracle's tests and the GPU path can take their
inputs from it without sharing any computation.

Workload being imitated (dev.to "AWQ: How Activation-Aware Quantization Saves
4-bit LLMs", section "Why does naive 4-bit quantization wreck LLM accuracy?"):
transformer activations in which a handful of input channels carry outlier
magnitudes on nearly every token, about 1% of the channels (same page, opening
paragraph and "How does AWQ decide which weights to protect?"), and fp16
weights of 7B/13B-class linear layers.  No corpus or trained weight exists
here, so every tensor is drawn from the recipe below.

Recipe for one searched layer (seed, layer index l):
  1. rng = numpy Generator(PCG64(SeedSequence([seed, l])))
  2. n_o = round(0.01 * in_features) outlier channels, idx = rng.choice(in, n_o)
  3. mult = exp(uniform(ln lo, ln hi)) per outlier channel
  4. Z = standard normal [N, in] (float32); heavy-tailed kind uses sign(Z)|Z|^1.5
  5. per-token scale r = exp(normal(0, 0.3)) only where the layer asks for it,
     from the stream SeedSequence([seed, l, 2])
  6. X = fp16(Z * mult[col] * r[row])
  7. W = fp16(0.02 * standard normal [out, in] (float32)), stream [seed, l, 1]
A cut to fewer tokens or output rows yields exactly the leading rows of the
full tensors.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import Dict, List, Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class LayerSpec:
    """Shape and distribution of one searched linear layer."""

    name: str
    n_tokens: int
    in_features: int
    out_features: int
    kind: str = "normal"          # "normal" or "heavy" (sign(Z)|Z|^1.5)
    outlier_lo: float = 10.0
    outlier_hi: float = 100.0
    token_scale: bool = False     # per-token log-normal(0, 0.3) scale
    layer_index: int = 0

    @property
    def n_outliers(self) -> int:
        # Python's round is half-to-even; 0.01*in never lands on .5 here.
        return int(round(0.01 * self.in_features))


@dataclasses.dataclass(frozen=True)
class ConfigSpec:
    key: int
    workload: str
    seed: int
    layers: List[LayerSpec]


def _cfg() -> Dict[int, ConfigSpec]:
    c: Dict[int, ConfigSpec] = {}
    c[1] = ConfigSpec(1, "single_linear_in512_out512_tok128", 0, [
        LayerSpec("linear", 128, 512, 512)])
    c[2] = ConfigSpec(2, "llama7b_q_proj_in4096_out4096_tok512", 1, [
        LayerSpec("q_proj", 512, 4096, 4096, token_scale=True)])
    c[3] = ConfigSpec(3, "fused_qkv_in4096_out12288_tok2048", 2, [
        LayerSpec("qkv", 2048, 4096, 12288, token_scale=True)])
    c[4] = ConfigSpec(4, "mlp_pair_up4096x11008_down11008x4096_tok2048", 3, [
        LayerSpec("up_gate", 2048, 4096, 11008, token_scale=True, layer_index=0),
        LayerSpec("down", 2048, 11008, 4096, kind="heavy", outlier_lo=10.0,
                  outlier_hi=50.0, layer_index=1)])
    c[5] = ConfigSpec(5, "llama13b_block_h5120_mlp13824_tok4096", 4, [
        LayerSpec("qkv", 4096, 5120, 15360, layer_index=0),
        LayerSpec("o_proj", 4096, 5120, 5120, layer_index=1),
        LayerSpec("gate_up", 4096, 5120, 27648, layer_index=2),
        LayerSpec("down", 4096, 13824, 5120, layer_index=3)])
    return c


CONFIGS: Dict[int, ConfigSpec] = _cfg()


def rng_for(seed: int, layer_index: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, layer_index])))


def make_activations(spec: LayerSpec, seed: int) -> np.ndarray:
    """X [n_tokens, in_features] fp16 following the module recipe."""
    rng = rng_for(seed, spec.layer_index)
    n, k = spec.n_tokens, spec.in_features
    idx = rng.choice(k, spec.n_outliers, replace=False)
    mult = np.exp(rng.uniform(math.log(spec.outlier_lo), math.log(spec.outlier_hi),
                              spec.n_outliers))
    col = np.ones(k, dtype=np.float32)
    col[idx] = mult.astype(np.float32)
    z = rng.standard_normal((n, k), dtype=np.float32)
    if spec.token_scale:
        # own stream: a cut to fewer tokens is then exactly the leading rows
        rrow = np.random.Generator(np.random.PCG64(
            np.random.SeedSequence([seed, spec.layer_index, 2])))
        row = np.exp(rrow.normal(0.0, 0.3, n)).astype(np.float32)
    else:
        row = None
    if spec.kind == "heavy":
        z = np.sign(z) * np.abs(z) ** np.float32(1.5)
    elif spec.kind != "normal":
        raise ValueError(f"unknown activation kind {spec.kind!r}")
    z *= col[None, :]
    if row is not None:
        z *= row[:, None]
    x = z.astype(np.float16)
    if not np.isfinite(x).all():
        raise ValueError("synthetic activations overflowed fp16")
    return x


def make_weights(spec: LayerSpec, seed: int) -> np.ndarray:
    """W [out_features, in_features] fp16, N(0, 0.02)."""
    # a stream of its own, so W does not depend on how many tokens X has
    rng = np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([seed, spec.layer_index, 1])))
    w = rng.standard_normal((spec.out_features, spec.in_features), dtype=np.float32)
    w *= np.float32(0.02)
    return w.astype(np.float16)


def make_layer(config: int, layer: int = 0, *, n_tokens: Optional[int] = None,
               out_features: Optional[int] = None):
    """(spec, X, W) for a configuration's layer, optionally cut to fewer tokens/rows.

    A cut keeps the distribution (same seed stream, same outlier channels) and
    is how the small parity cases are made from the large configurations.
    """
    cfg = CONFIGS[config]
    spec = cfg.layers[layer]
    if n_tokens is not None or out_features is not None:
        spec = dataclasses.replace(
            spec, n_tokens=n_tokens or spec.n_tokens,
            out_features=out_features or spec.out_features)
    return spec, make_activations(spec, cfg.seed), make_weights(spec, cfg.seed)


def make_custom(n_tokens: int, in_features: int, out_features: int, seed: int, *,
                kind: str = "normal", token_scale: bool = False,
                outlier_lo: float = 10.0, outlier_hi: float = 100.0):
    spec = LayerSpec("custom", n_tokens, in_features, out_features, kind=kind,
                     outlier_lo=outlier_lo, outlier_hi=outlier_hi, token_scale=token_scale)
    return spec, make_activations(spec, seed), make_weights(spec, seed)


def digest(*arrays: np.ndarray) -> str:
    """SHA-256 over the raw bytes of the given arrays (input manifest)."""
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()
