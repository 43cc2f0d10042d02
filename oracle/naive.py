"""O2: vanilla masked-diffusion decoding by plain full recompute (NumPy, fp64).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Written independently
of ``oracle.cpp``: every step runs the whole transformer over all N positions
with dense N x N bidirectional attention and no K/V cache, which is the
baseline sampler the SureLock page describes in its §1 Problem statement
("Stopping Computation for Converged Tokens in Masked Diffusion-LM
Decoding").  The unmasking rule is the confidence-ranked top-k inside
semi-autoregressive blocks named on the SlowFast page ("Accelerating
Diffusion LLMs with SlowFast Sampling"), §1 and §2.

``generate_loops`` is a third version in pure Python loops (no vectorised
attention or matmul) for brute force on tiny shapes.
"""
from __future__ import annotations

import math
from typing import Dict, List

import numpy as np


def _bf16(a: np.ndarray) -> np.ndarray:
    """Round float64 data to bf16 precision (8 significant bits, ties to even)."""
    a = np.asarray(a, dtype=np.float64)
    m, e = np.frexp(a)
    scale = np.ldexp(np.ones_like(a), e - 8)
    with np.errstate(invalid="ignore"):
        r = np.rint(a / scale) * scale
    return np.where(np.isfinite(a) & (a != 0), r, a)


def _rms(x, g, eps):
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * g


def _rope_all(u, base):
    """u [N][heads][hd]; rotates row n by its position n (half-split pairs)."""
    if base <= 0:
        return u
    n, _, hd = u.shape
    half = hd // 2
    inv = base ** (-2.0 * np.arange(half) / hd)
    ang = np.arange(n)[:, None] * inv[None, :]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    a, b = u[..., :half], u[..., half:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def forward_full(shape, W: Dict, tokens: np.ndarray) -> np.ndarray:
    """Logits [N][V] for one sequence, every position recomputed."""
    st = _bf16 if shape.bf16 else (lambda a: a)
    d, nq, nkv, hd = shape.d_model, shape.n_heads, shape.n_kv_heads, shape.head_dim
    N = tokens.shape[0]
    h = W["tok_emb"][tokens].astype(np.float64)
    for lay in W["layers"]:
        a = st(_rms(h, lay["attn_norm"].astype(np.float64), shape.rms_eps))
        qkv = a @ lay["w_qkv"].astype(np.float64).T
        q = qkv[:, : nq * hd].reshape(N, nq, hd)
        k = qkv[:, nq * hd: (nq + nkv) * hd].reshape(N, nkv, hd)
        v = qkv[:, (nq + nkv) * hd:].reshape(N, nkv, hd)
        q = st(_rope_all(q, shape.rope_base))
        k = st(_rope_all(k, shape.rope_base))
        v = st(v)
        rep = nq // nkv
        kk = np.repeat(k, rep, axis=1)  # head h uses kv head h // rep
        vv = np.repeat(v, rep, axis=1)
        s = np.einsum("ihc,jhc->hij", q, kk) / math.sqrt(hd)
        s = s - s.max(axis=-1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=-1, keepdims=True)
        o = st(np.einsum("hij,jhc->ihc", p, vv).reshape(N, nq * hd))
        h = h + o @ lay["w_o"].astype(np.float64).T
        a2 = st(_rms(h, lay["ffn_norm"].astype(np.float64), shape.rms_eps))
        g = a2 @ lay["w_gate"].astype(np.float64).T
        u = a2 @ lay["w_up"].astype(np.float64).T
        act = st(g / (1.0 + np.exp(-g)) * u)
        h = h + act @ lay["w_down"].astype(np.float64).T
    af = st(_rms(h, W["final_norm"].astype(np.float64), shape.rms_eps))
    z = af @ W["lm_head"].astype(np.float64).T
    z[:, shape.mask_id] = -np.inf
    return z


def _k_for_step(run, t):
    G = run.seq_len - run.prompt_len
    nblk = -(-G // run.block_len)
    for b in range(nblk):
        t0, t1 = run.steps * b // nblk, run.steps * (b + 1) // nblk
        if t0 <= t < t1:
            lo = run.prompt_len + b * run.block_len
            hi = min(run.seq_len, lo + run.block_len)
            Gb, Tb, s = hi - lo, t1 - t0, t - t0
            return lo, hi, Gb * (s + 1) // Tb - Gb * s // Tb
    return 0, 0, 0


def _commit(shape, run, t, x, z):
    lo, hi, k = _k_for_step(run, t)
    zz = z.copy()
    zz[:, shape.mask_id] = -np.inf
    mx = zz.max(axis=1)
    lse = mx + np.log(np.exp(zz - mx[:, None]).sum(axis=1))
    am = zz.argmax(axis=1)  # first maximum
    conf = np.exp(mx - lse)
    cand = [i for i in range(lo, hi) if x[i] == shape.mask_id]
    cand.sort(key=lambda i: (-conf[i], i))
    x = x.copy()
    for i in cand[:k]:
        x[i] = am[i]
    return x, conf, am


def generate(shape, W: Dict, run, prompts: np.ndarray) -> Dict[str, List]:
    """Vanilla decoding of every sequence: per-step logits and tokens."""
    out = {"logits": [], "tokens": []}
    xs = []
    for b in range(run.batch):
        x = np.full(run.seq_len, shape.mask_id, dtype=np.int64)
        x[: run.prompt_len] = prompts[b]
        xs.append(x)
    for t in range(run.steps):
        zs, new = [], []
        for b in range(run.batch):
            z = forward_full(shape, W, xs[b])
            x, _, _ = _commit(shape, run, t, xs[b], z)
            zs.append(z)
            new.append(x)
        xs = new
        out["logits"].append(np.stack(zs))
        out["tokens"].append(np.stack(xs).astype(np.int32))
    return out


# --- pure-Python loops, tiny shapes only -----------------------------------

def forward_loops(shape, W, tokens) -> List[List[float]]:
    st = (lambda v: float(_bf16(np.float64(v)))) if shape.bf16 else (lambda v: v)
    d, nq, nkv, hd, dff, V = (shape.d_model, shape.n_heads, shape.n_kv_heads, shape.head_dim,
                              shape.d_ff, shape.vocab)
    N = len(tokens)

    def rms(vec, g):
        ms = sum(v * v for v in vec) / len(vec)
        inv = 1.0 / math.sqrt(ms + shape.rms_eps)
        return [st(vec[c] * inv * float(g[c])) for c in range(len(vec))]

    def mv(Wm, vec):
        return [sum(float(Wm[o][c]) * vec[c] for c in range(len(vec))) for o in range(len(Wm))]

    def rot(vec, pos):
        if shape.rope_base <= 0:
            return vec
        half = len(vec) // 2
        out = list(vec)
        for j in range(half):
            ang = pos * shape.rope_base ** (-2.0 * j / len(vec))
            out[j] = vec[j] * math.cos(ang) - vec[j + half] * math.sin(ang)
            out[j + half] = vec[j] * math.sin(ang) + vec[j + half] * math.cos(ang)
        return out

    h = [[float(W["tok_emb"][tok][c]) for c in range(d)] for tok in tokens]
    for lay in W["layers"]:
        qs, ks, vs = [], [], []
        for n in range(N):
            a = rms(h[n], lay["attn_norm"])
            y = mv(lay["w_qkv"], a)
            qs.append([[st(v) for v in rot(y[hh * hd:(hh + 1) * hd], n)] for hh in range(nq)])
            ks.append([[st(v) for v in rot(y[(nq + g) * hd:(nq + g + 1) * hd], n)]
                       for g in range(nkv)])
            vs.append([[st(v) for v in y[(nq + nkv + g) * hd:(nq + nkv + g + 1) * hd]]
                       for g in range(nkv)])
        for n in range(N):
            o = []
            for hh in range(nq):
                g = hh * nkv // nq
                sc = [sum(qs[n][hh][c] * ks[j][g][c] for c in range(hd)) / math.sqrt(hd)
                      for j in range(N)]
                m = max(sc)
                e = [math.exp(s - m) for s in sc]
                den = sum(e)
                o.extend(st(sum(e[j] * vs[j][g][c] for j in range(N)) / den) for c in range(hd))
            dh = mv(lay["w_o"], o)
            h[n] = [h[n][c] + dh[c] for c in range(d)]
        for n in range(N):
            a = rms(h[n], lay["ffn_norm"])
            g = mv(lay["w_gate"], a)
            u = mv(lay["w_up"], a)
            act = [st(g[c] / (1.0 + math.exp(-g[c])) * u[c]) for c in range(dff)]
            dh = mv(lay["w_down"], act)
            h[n] = [h[n][c] + dh[c] for c in range(d)]
    z = []
    for n in range(N):
        a = rms(h[n], W["final_norm"])
        row = mv(W["lm_head"], a)
        row[shape.mask_id] = -math.inf
        z.append(row)
    return z


def generate_loops(shape, W, run, prompts) -> Dict[str, List]:
    out = {"logits": [], "tokens": []}
    xs = []
    for b in range(run.batch):
        x = [shape.mask_id] * run.seq_len
        x[: run.prompt_len] = [int(v) for v in prompts[b]]
        xs.append(x)
    for t in range(run.steps):
        lo, hi, k = _k_for_step(run, t)
        zs = []
        for b in range(run.batch):
            z = forward_loops(shape, W, xs[b])
            zs.append(z)
            best = []
            for i in range(lo, hi):
                if xs[b][i] != shape.mask_id:
                    continue
                row = z[i]
                m = max(row)
                am = row.index(m)
                conf = 1.0 / sum(math.exp(v - m) for v in row if v != -math.inf)
                best.append((-conf, i, am))
            best.sort()
            for _, i, am in best[:k]:
                xs[b][i] = am
        out["logits"].append(np.asarray(zs, dtype=np.float64))
        out["tokens"].append(np.asarray(xs, dtype=np.int32))
    return out
