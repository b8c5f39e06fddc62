"""Seeded synthetic inputs for the GPT-2 forward: weights, token ids, attention Q/K/V.

This module draws random numbers and fixes their storage precision. It holds none of the
forward's arithmetic, imports nothing else from this package, and is the only code that the
CPU oracle and the GPU path share (both receive exactly the arrays made here).

Recipe (the init the GPT-2 pages describe; "复现GPT-2 124M" §2.4 and §2.1):
  * every Linear weight and both embedding tables (wte, wpe) ~ N(0, 0.02);
  * the two residual-output projections of each block (attn.c_proj.w, mlp.c_proj.w) have their
    standard deviation divided by sqrt(2 * n_layer);
  * Linear biases 0, LayerNorm gamma 1 and beta 0;
  * token ids uniform over [0, n_vocab).
The "perturbed" variant additionally draws biases ~ N(0, 0.02), gamma ~ 1 + N(0, 0.1),
beta ~ N(0, 0.02) from its own stream, so that the bias and affine paths are exercised.

Generator: numpy Generator(PCG64(seed)); seeds 0 (weights), 1 (tokens), 2 (attention Q/K/V),
3 (perturbation extras), 4 (sampling inputs). Tensors are drawn one after another in the fixed tensor order below as
float64 normals, rounded to float32 (round-to-nearest-even), and, for a bf16 model, rounded once
more to bf16 (round-to-nearest-even) and kept as bf16-exact float32 values. The double rounding
is deliberate and is the definition of the weights: both sides receive the same values.
"""
from __future__ import annotations

import dataclasses

import numpy as np

SEED_WEIGHTS = 0
SEED_TOKENS = 1
SEED_ATTENTION = 2
SEED_PERTURB = 3
SEED_SAMPLING = 4


@dataclasses.dataclass(frozen=True)
class ModelShape:
    """Hyper-parameters of one GPT-2 size (the pages' GPT2Config fields)."""

    n_vocab: int = 50257
    n_ctx: int = 1024
    d_model: int = 768
    n_head: int = 12
    n_layer: int = 12
    d_mlp: int = 3072
    ln_eps: float = 1e-5

    @property
    def d_head(self) -> int:
        return self.d_model // self.n_head


GPT2_SMALL = ModelShape()
GPT2_MEDIUM = ModelShape(d_model=1024, n_head=16, n_layer=24, d_mlp=4096)
GPT2_XL = ModelShape(d_model=1600, n_head=25, n_layer=48, d_mlp=6400)


def tensor_specs(s: ModelShape):
    """The fixed tensor order: list of (name, shape, kind).

    kind is one of "emb" (N(0,0.02)), "w" (N(0,0.02)), "w_res" (N(0,0.02/sqrt(2L))),
    "bias" (0), "gamma" (1), "beta" (0). Linear weights are [out, in] (y = x W^T + b).
    lm_head has no tensor of its own: it is wte.
    """
    d, f = s.d_model, s.d_mlp
    specs = [("wte", (s.n_vocab, d), "emb"), ("wpe", (s.n_ctx, d), "emb")]
    for l in range(s.n_layer):
        p = f"h.{l}."
        specs += [
            (p + "ln_1.w", (d,), "gamma"), (p + "ln_1.b", (d,), "beta"),
            (p + "attn.c_attn.w", (3 * d, d), "w"), (p + "attn.c_attn.b", (3 * d,), "bias"),
            (p + "attn.c_proj.w", (d, d), "w_res"), (p + "attn.c_proj.b", (d,), "bias"),
            (p + "ln_2.w", (d,), "gamma"), (p + "ln_2.b", (d,), "beta"),
            (p + "mlp.c_fc.w", (f, d), "w"), (p + "mlp.c_fc.b", (f,), "bias"),
            (p + "mlp.c_proj.w", (d, f), "w_res"), (p + "mlp.c_proj.b", (d,), "bias"),
        ]
    specs += [("ln_f.w", (d,), "gamma"), ("ln_f.b", (d,), "beta")]
    return specs


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns bf16-exact float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    out = r.astype(np.uint32).view(np.float32)
    # keep NaN payloads quiet rather than letting the carry turn them into Inf
    nan = np.isnan(a)
    if nan.any():
        out = out.copy()
        out[nan] = np.float32(np.nan)
    return out


def make_weights(s: ModelShape, bf16: bool, perturbed: bool = False, seed: int = SEED_WEIGHTS):
    """Return an ordered dict name -> float32 array (bf16-exact when bf16=True)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    prng = np.random.Generator(np.random.PCG64(SEED_PERTURB)) if perturbed else None
    std = 0.02
    std_res = 0.02 / np.sqrt(2.0 * s.n_layer)
    out = {}
    for name, shape, kind in tensor_specs(s):
        if kind in ("emb", "w"):
            z = rng.standard_normal(shape) * std
        elif kind == "w_res":
            z = rng.standard_normal(shape) * std_res
        elif kind == "gamma":
            z = np.ones(shape) + (prng.standard_normal(shape) * 0.1 if perturbed else 0.0)
        else:  # bias, beta
            z = prng.standard_normal(shape) * 0.02 if perturbed else np.zeros(shape)
        a = z.astype(np.float32)
        if bf16:
            a = round_bf16(a)
        out[name] = a
    return out


def make_tokens(B: int, T: int, n_vocab: int = 50257, seed: int = SEED_TOKENS) -> np.ndarray:
    """Token ids uniform over [0, n_vocab), int32 [B, T]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(0, n_vocab, size=(B, T)).astype(np.int32)


def make_qkv(B: int, H: int, T: int, dh: int, bf16: bool = True, seed: int = SEED_ATTENTION):
    """Q, K, V i.i.d. N(0, 1), each [B, H, T, dh] float32 (bf16-exact when bf16=True)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for _ in range(3):
        a = rng.standard_normal((B, H, T, dh)).astype(np.float32)
        out.append(round_bf16(a) if bf16 else a)
    return tuple(out)


def make_sampling_inputs(B: int, V: int, n_hist: int = 0, std: float = 2.0, n_peaked: int = 0,
                         seed: int = SEED_SAMPLING):
    """Inputs of the next-token sampler: logits float32 [B, V] ~ N(0, std^2), where the first
    n_peaked rows also get 5 dominant tokens (+N(8, 1) on 5 distinct random ids, a peaked next-token
    distribution); u float32 [B] uniform over [0, 1); history int32 [B, n_hist] uniform ids over
    [0, V) (the tokens seen so far). Drawn in that order from one stream."""
    rng = np.random.Generator(np.random.PCG64(seed))
    logits = rng.standard_normal((B, V)) * std
    for b in range(min(n_peaked, B)):
        ids = rng.choice(V, size=min(5, V), replace=False)
        logits[b, ids] += rng.normal(8.0, 1.0, size=ids.shape)
    u = rng.random(B).astype(np.float32)
    u = np.minimum(u, np.float32(1.0) - np.float32(2.0 ** -24))  # float32 rounding must not reach 1
    hist = rng.integers(0, V, size=(B, n_hist)).astype(np.int32)
    return logits.astype(np.float32), u, hist
