"""Seeded synthetic inputs for the masked-diffusion denoising step.

This module only draws numbers: model shapes, random-init weights, random
prompts, random lock bitmasks and random K/V caches.  It holds none of the
method's arithmetic (no normalisation, attention, softmax, locking or commit
rule), so that the CPU oracle and the GPU engine can both be fed from it
without sharing any computation.

Recipe (NumPy ``default_rng``; every tensor drawn in a fixed order):

* weights: seed 0.  Matrices ~ N(0, 0.02) in float32, drawn in the order
  tok_emb, then per layer (attn_norm, w_qkv, w_o, ffn_norm, w_gate, w_up,
  w_down), then final_norm, lm_head.  Norm gains are 1 + gain_std * N(0, 1).
  For bf16 models every value is rounded to the nearest bfloat16
  (ties to even) and kept as the float32 that holds it exactly.
* prompts: sequence b uses seed [1, b]; tokens uniform over [0, V-1), i.e.
  never the mask token V-1.
* active-set choice: seed 2; cache contents: seed 3; activations: seed 4.

Matrix layouts are "output-major": a linear map y = x W^T stores W as
[out_features][in_features], rows contiguous along the input dimension.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

WEIGHT_STD = 0.02


@dataclasses.dataclass(frozen=True)
class ModelShape:
    n_layers: int
    d_model: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    d_ff: int
    vocab: int
    bf16: bool
    rope_base: float = 10000.0
    rms_eps: float = 1e-5

    @property
    def mask_id(self) -> int:
        return self.vocab - 1

    @property
    def qkv_out(self) -> int:
        return (self.n_heads + 2 * self.n_kv_heads) * self.head_dim


@dataclasses.dataclass(frozen=True)
class RunShape:
    batch: int
    seq_len: int
    prompt_len: int
    steps: int
    block_len: int  # generated positions per semi-autoregressive block


# Lock settings.  "natural" is the configured gate (KL <= 1e-3 and
# max-prob >= 0.9 for 2 consecutive steps); "kl_only" drops the confidence
# gate; "scheduled" accepts every defined KL (eps = +inf, tau = 0), so a
# decoded position locks on its second step with a real input token;
# "vanilla" never locks (plain full-recompute decoding).
LOCK_SETTINGS = {
    "natural": dict(policy="test", kl_eps=1e-3, conf_tau=0.9, n_consec=2,
                    lock_prompt_after_first_step=1),
    "kl_only": dict(policy="test", kl_eps=1e-3, conf_tau=0.0, n_consec=2,
                    lock_prompt_after_first_step=1),
    "scheduled": dict(policy="test", kl_eps=float("inf"), conf_tau=0.0,
                      n_consec=2, lock_prompt_after_first_step=1),
    "vanilla": dict(policy="none", kl_eps=-1.0, conf_tau=0.0, n_consec=2,
                    lock_prompt_after_first_step=0),
    # the natural lock test with the SlowFast sampler ([SF] §2) in place of the
    # semi-autoregressive block schedule; thresholds at the pages' 0.9, the
    # stage limits of [SF] §4 (8 exploratory steps, window 2, variance 1.0)
    "slowfast": dict(policy="test", kl_eps=1e-3, conf_tau=0.9, n_consec=2,
                     lock_prompt_after_first_step=1, sampler="slowfast", sf_k=3, sf_kmax=8,
                     sf_whist=2, sf_tau_conv=0.9, sf_tau_high=0.9, sf_var=1.0),
    # the scheduled lock test with the drift-aware refresh of locked positions
    # (Polestar page, Polestar-Cache): each step the 8 locked positions of a
    # sequence with the largest drift are recomputed, and one whose drift
    # exceeds 1e-3 (the KL level of the lock test) is unlocked; the budget is
    # a run choice (the page gives none)
    "refresh": dict(policy="test", kl_eps=float("inf"), conf_tau=0.0, n_consec=2,
                    lock_prompt_after_first_step=1, refresh_budget=8, refresh_eps=1e-3),
}


def _tiny() -> (ModelShape, RunShape):
    return (ModelShape(2, 64, 4, 4, 16, 172, 256, bf16=False),
            RunShape(1, 32, 8, 16, 24))


def _llada(L=32) -> ModelShape:
    return ModelShape(L, 4096, 32, 32, 128, 12288, 126464, bf16=True)


CONFIGS: Dict[str, tuple] = {
    # 2-layer fp32 model, one sequence of 32 (8 prompt + 24 masked), 16 steps.
    "tiny": _tiny(),
    # LLaDA-8B shape, one sequence of 512 (128 prompt + 384 masked), 128 steps.
    "llada8b": (_llada(), RunShape(1, 512, 128, 128, 384)),
    # Dream-7B shape (GQA 28/4), 8 sequences of 1024, 256 steps.
    "dream7b": (ModelShape(28, 3584, 28, 4, 128, 18944, 152064, bf16=True),
                RunShape(8, 1024, 256, 256, 768)),
    # LLaDA-8B shape, 4 sequences of 4096, 512 steps in blocks of 256.
    "longctx": (_llada(), RunShape(4, 4096, 1024, 512, 256)),
}

# One bf16 transformer layer at LLaDA width, for kernel isolation.
LAYER_ISOLATION = dict(shape=_llada(L=1), cache_len=1024,
                       active_fractions=(1.0, 0.5, 0.25, 0.1, 0.02))


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Nearest bfloat16 value (ties to even) of float32 data, as float32.

    Used only to make generated inputs bf16-representable."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    out = r.astype(np.uint32).view(np.float32)
    nan = np.isnan(a)
    if nan.any():
        out = out.copy()
        out[nan] = np.nan
    return out


def gen_weights(shape: ModelShape, seed: int = 0, gain_std: float = 0.1,
                layers: Optional[List[int]] = None) -> Dict[str, object]:
    """Random-init weights as float32 host arrays.

    Returns a dict with tok_emb [V][d], final_norm [d], lm_head [V][d] and
    a list ``layers`` of dicts: attn_norm [d], w_qkv [(nq+2nkv)*hd][d],
    w_o [d][nq*hd], ffn_norm [d], w_gate [d_ff][d], w_up [d_ff][d],
    w_down [d][d_ff].  ``layers`` (a list of layer indices) keeps only those
    layers' matrices; the draw order, and so every value, is unchanged.
    """
    rng = np.random.default_rng(seed)
    d, dff, V = shape.d_model, shape.d_ff, shape.vocab
    qo = shape.n_heads * shape.head_dim

    def mat(rows, cols, keep=True):
        if not keep:
            # advance the stream exactly as a real draw would
            rng.standard_normal((rows, cols), dtype=np.float32)
            return None
        w = rng.standard_normal((rows, cols), dtype=np.float32) * np.float32(WEIGHT_STD)
        return round_to_bf16(w) if shape.bf16 else w

    def gain(keep=True):
        g = (1.0 + gain_std * rng.standard_normal(d)).astype(np.float32)
        if not keep:
            return None
        return round_to_bf16(g) if shape.bf16 else g

    out: Dict[str, object] = {}
    out["tok_emb"] = mat(V, d)
    lay = []
    for li in range(shape.n_layers):
        keep = layers is None or li in layers
        ent = dict(
            attn_norm=gain(keep),
            w_qkv=mat(shape.qkv_out, d, keep),
            w_o=mat(d, qo, keep),
            ffn_norm=gain(keep),
            w_gate=mat(dff, d, keep),
            w_up=mat(dff, d, keep),
            w_down=mat(d, dff, keep),
        )
        lay.append(ent if keep else None)
    out["layers"] = lay
    out["final_norm"] = gain()
    out["lm_head"] = mat(V, d)
    return out


def gen_prompts(shape: ModelShape, run: RunShape) -> np.ndarray:
    """int32 [B][P] prompt tokens, uniform over [0, V-1)."""
    rows = []
    for b in range(run.batch):
        rng = np.random.default_rng([1, b])
        rows.append(rng.integers(0, shape.vocab - 1, size=run.prompt_len, dtype=np.int64))
    return np.asarray(rows, dtype=np.int32).reshape(run.batch, run.prompt_len)


def gen_active_rows(n: int, m: int, seed: int = 2) -> np.ndarray:
    """Sorted int32 positions of a uniform random subset of size m of [0, n)."""
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(n, size=m, replace=False)).astype(np.int32)


def gen_lock_bits(batch: int, seq_len: int, p_locked: float, seed: int = 2) -> np.ndarray:
    """uint64 [B][ceil(N/64)] bitmask; bit (pos % 64) of word pos // 64."""
    rng = np.random.default_rng(seed)
    words = (seq_len + 63) // 64
    bits = rng.random((batch, seq_len)) < p_locked
    out = np.zeros((batch, words), dtype=np.uint64)
    for b in range(batch):
        for p in np.nonzero(bits[b])[0]:
            out[b, p // 64] |= np.uint64(1) << np.uint64(p % 64)
    return out


def gen_normal(shape, seed: int, std: float = 1.0, bf16: bool = False) -> np.ndarray:
    rng = np.random.default_rng(seed)
    a = (rng.standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float32)
    return round_to_bf16(a) if bf16 else a
