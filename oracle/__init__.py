"""CPU oracle for the masked-diffusion denoising step with converged-token locking.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code
with the GPU engine (``selective_token_recompute_amd``) and never imports it.

Two independent implementations live here:

* ``oracle.cpp`` (O1, C++, fp64, OpenMP over rows): the SureLock step as the
  pages describe it -- active set, fresh K/V for active rows written into a
  per-layer cache, active queries attending to all N cached positions, the
  posterior statistics, confidence-ranked top-k unmasking and the KL lock
  test.  Wrapped by :class:`Oracle` and the ``unit_*`` functions below.
* ``naive.py`` (O2, NumPy): vanilla full-recompute decoding with dense N x N
  attention and no cache, used to pin O1 with locking off.

Every unit function converts its inputs to float64 and returns float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.cpp")
_LIB = os.path.join(_HERE, "liboracle.so")

POLICY = {"none": 0, "test": 1}
SAMPLER = {"semi_ar": 0, "slowfast": 1}
# SlowFast defaults ([SF] §4 ablation: at most 8 exploratory steps, a history
# window of 2, variance threshold 1.0; the two confidence thresholds and k
# are run choices)
SF_DEFAULTS = dict(sf_k=1, sf_kmax=8, sf_whist=2, sf_tau_conv=0.9, sf_tau_high=0.9, sf_var=1.0)


def build(force: bool = True) -> str:
    """Compile oracle.cpp into liboracle.so with g++ (OpenMP, -O2)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp"
    cmd = ["g++", "-O2", "-mavx2", "-mfma", "-fopenmp", "-fPIC", "-shared", "-std=c++17",
           _SRC, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


class _Model(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("mask_id", ctypes.c_int32),
                ("rope_base", ctypes.c_double), ("rms_eps", ctypes.c_double),
                ("bf16_storage", ctypes.c_int32)]


class _Run(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seq_len", ctypes.c_int32),
                ("prompt_len", ctypes.c_int32), ("steps", ctypes.c_int32),
                ("block_len", ctypes.c_int32), ("kl_eps", ctypes.c_double),
                ("conf_tau", ctypes.c_double), ("n_consec", ctypes.c_int32),
                ("kl_dir", ctypes.c_int32), ("lock_prompt_after_first_step", ctypes.c_int32),
                ("policy", ctypes.c_int32), ("sampler", ctypes.c_int32),
                ("sf_k", ctypes.c_int32), ("sf_kmax", ctypes.c_int32),
                ("sf_whist", ctypes.c_int32), ("sf_tau_conv", ctypes.c_double),
                ("sf_tau_high", ctypes.c_double), ("sf_var", ctypes.c_double),
                ("refresh_budget", ctypes.c_int32), ("refresh_eps", ctypes.c_double)]


_PF = ctypes.POINTER(ctypes.c_float)


class _Weights(ctypes.Structure):
    _fields_ = [("tok_emb", _PF), ("final_norm", _PF), ("lm_head", _PF),
                ("attn_norm", ctypes.POINTER(_PF)), ("w_qkv", ctypes.POINTER(_PF)),
                ("w_o", ctypes.POINTER(_PF)), ("ffn_norm", ctypes.POINTER(_PF)),
                ("w_gate", ctypes.POINTER(_PF)), ("w_up", ctypes.POINTER(_PF)),
                ("w_down", ctypes.POINTER(_PF))]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        vp = ctypes.c_void_p
        i32 = ctypes.c_int32
        L.orc_create.restype = vp
        L.orc_create.argtypes = [ctypes.POINTER(_Model), ctypes.POINTER(_Weights),
                                 ctypes.POINTER(_Run), vp]
        L.orc_destroy.argtypes = [vp]
        L.orc_step.argtypes = [vp]
        L.orc_step_sample.argtypes = [vp, vp, ctypes.c_int]
        L.orc_lock_update.argtypes = [vp, vp, vp, vp, i32, vp, vp]
        for f in ("orc_t", "orc_m", "orc_n_logit_rows", "orc_n_commits"):
            getattr(L, f).argtypes = [vp]
        L.orc_flops.argtypes = [vp]
        L.orc_flops.restype = ctypes.c_double
        for f in ("orc_get_tokens", "orc_get_locked", "orc_get_cnt", "orc_get_frozen",
                  "orc_get_sf", "orc_get_has_prev", "orc_get_drift", "orc_get_refresh"):
            getattr(L, f).argtypes = [vp, vp]
        L.orc_get_rows.argtypes = [vp, vp, vp, vp]
        L.orc_get_stats.argtypes = [vp, vp, vp, vp, vp, vp]
        L.orc_get_logits.argtypes = [vp, vp, vp]
        L.orc_get_commits.argtypes = [vp, vp, vp, vp]
        L.orc_get_kv.argtypes = [vp, ctypes.c_int, vp, vp]
        L.orc_bf16_round.argtypes = [ctypes.c_double]
        L.orc_bf16_round.restype = ctypes.c_double
        L.orc_unit_rmsnorm.argtypes = [vp, vp, ctypes.c_int, ctypes.c_int, ctypes.c_double, vp]
        L.orc_unit_rope.argtypes = [vp, vp, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_double]
        L.orc_unit_linear.argtypes = [vp, vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]
        L.orc_unit_attention.argtypes = [vp, vp, vp, vp] + [ctypes.c_int] * 6 + [vp]
        L.orc_unit_vocab_stats.argtypes = [vp, vp, vp, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp]
        L.orc_unit_schedule.argtypes = [ctypes.POINTER(_Run), ctypes.c_int, vp]
        L.orc_unit_lock_transition.argtypes = [ctypes.POINTER(_Model), ctypes.POINTER(_Run),
                                               ctypes.c_int, ctypes.c_int] + [vp] * 12
        L.orc_unit_refresh_select.argtypes = [ctypes.POINTER(_Run), vp, vp, vp]
        L.orc_unit_compact.argtypes = [vp, ctypes.c_int, ctypes.c_int, vp, vp, vp]
        L.orc_unit_slowfast.argtypes = [ctypes.POINTER(_Run)] + [ctypes.c_int] * 3 + [vp] * 9
        L.orc_num_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


def make_model(shape) -> _Model:
    return _Model(shape.n_layers, shape.d_model, shape.n_heads, shape.n_kv_heads,
                  shape.head_dim, shape.d_ff, shape.vocab, shape.mask_id,
                  float(shape.rope_base), float(shape.rms_eps), 1 if shape.bf16 else 0)


def make_run(run, lock: Dict) -> _Run:
    return _Run(run.batch, run.seq_len, run.prompt_len, run.steps, run.block_len,
                float(lock["kl_eps"]), float(lock["conf_tau"]), int(lock["n_consec"]),
                int(lock.get("kl_dir", 0)), int(lock["lock_prompt_after_first_step"]),
                POLICY[lock["policy"]], SAMPLER[lock.get("sampler", "semi_ar")],
                *[type(v)(lock.get(k, v)) for k, v in SF_DEFAULTS.items()],
                int(lock.get("refresh_budget", 0)),
                float(lock.get("refresh_eps", lock["kl_eps"])))


def num_threads() -> int:
    return int(lib().orc_num_threads())


class Oracle:
    """The O1 state machine: ``step()`` then ``lock_update()``, T times."""

    def __init__(self, shape, weights: Dict, run, lock: Dict, prompts: np.ndarray):
        self.shape, self.run, self.lock = shape, run, lock
        L = shape.n_layers
        self._keep = []

        def f(a):
            a = _f32(a)
            self._keep.append(a)
            return ctypes.cast(a.ctypes.data, _PF)

        def arr(key):
            ps = (_PF * L)(*[f(weights["layers"][l][key]) for l in range(L)])
            self._keep.append(ps)
            return ctypes.cast(ps, ctypes.POINTER(_PF))

        self._w = _Weights(f(weights["tok_emb"]), f(weights["final_norm"]),
                           f(weights["lm_head"]), arr("attn_norm"), arr("w_qkv"),
                           arr("w_o"), arr("ffn_norm"), arr("w_gate"), arr("w_up"),
                           arr("w_down"))
        self._m = make_model(shape)
        self._r = make_run(run, lock)
        pr = np.ascontiguousarray(prompts, dtype=np.int32)
        self._keep.append(pr)
        h = lib().orc_create(ctypes.byref(self._m), ctypes.byref(self._w), ctypes.byref(self._r),
                             _ptr(pr))
        if not h:
            raise ValueError("oracle rejected the configuration")
        self._h = ctypes.c_void_p(h)

    def __del__(self):
        if getattr(self, "_h", None):
            lib().orc_destroy(self._h)
            self._h = None

    @property
    def t(self) -> int:
        return lib().orc_t(self._h)

    @property
    def m(self) -> int:
        return lib().orc_m(self._h)

    @property
    def flops(self) -> float:
        return lib().orc_flops(self._h)

    def step(self, sample_rows: Optional[Sequence[int]] = None) -> None:
        if sample_rows is None:
            rc = lib().orc_step(self._h)
        else:
            s = np.ascontiguousarray(sample_rows, dtype=np.int32)
            rc = lib().orc_step_sample(self._h, _ptr(s), len(s))
        if rc != 0:
            raise RuntimeError(f"oracle step failed ({rc})")

    def lock_update(self, commits=None, locked=None, cnt=None) -> None:
        """commits: optional (seq, pos, tok) arrays replacing the top-k choice;
        locked: optional uint8 [B][N] ORed into the lock state; cnt: optional
        int32 [B][N] replacing the counters."""
        keep = []

        def p(a, dt):
            if a is None:
                return None
            a = np.ascontiguousarray(a, dtype=dt)
            keep.append(a)
            return _ptr(a)

        if commits is None:
            cs = cp = ct = None
            n = -1
        else:
            cs, cp, ct = (p(commits[0], np.int32), p(commits[1], np.int32),
                          p(commits[2], np.int32))
            n = len(commits[0])
        rc = lib().orc_lock_update(self._h, cs, cp, ct, n, p(locked, np.uint8), p(cnt, np.int32))
        if rc != 0:
            raise RuntimeError(f"oracle lock_update failed ({rc})")

    def _bn(self):
        return self.run.batch, self.run.seq_len

    def tokens(self) -> np.ndarray:
        out = np.empty(self._bn(), dtype=np.int32)
        lib().orc_get_tokens(self._h, _ptr(out))
        return out

    def locked(self) -> np.ndarray:
        out = np.empty(self._bn(), dtype=np.uint8)
        lib().orc_get_locked(self._h, _ptr(out))
        return out

    def counters(self) -> np.ndarray:
        out = np.empty(self._bn(), dtype=np.int32)
        lib().orc_get_cnt(self._h, _ptr(out))
        return out

    def frozen(self) -> np.ndarray:
        """uint8 [B][N]: positions a SlowFast accelerated stage took out of the
        active set."""
        out = np.empty(self._bn(), dtype=np.uint8)
        lib().orc_get_frozen(self._h, _ptr(out))
        return out

    def has_prev(self) -> np.ndarray:
        """uint8 [B][N]: a previous-step posterior is stored."""
        out = np.empty(self._bn(), dtype=np.uint8)
        lib().orc_get_has_prev(self._h, _ptr(out))
        return out

    def drift(self) -> np.ndarray:
        """float32 [B][N]: each position's KL between its two latest
        posteriors (+inf while undefined)."""
        out = np.empty(self._bn(), dtype=np.float32)
        lib().orc_get_drift(self._h, _ptr(out))
        return out

    def refresh(self) -> np.ndarray:
        """uint8 [B][N]: locked positions the last step recomputed."""
        out = np.empty(self._bn(), dtype=np.uint8)
        lib().orc_get_refresh(self._h, _ptr(out))
        return out

    def sf_state(self) -> np.ndarray:
        """int32 [B][13]: phase, lo, hi, slow_n, hist_n, hist[8] per sequence."""
        out = np.empty((self.run.batch, 13), dtype=np.int32)
        lib().orc_get_sf(self._h, _ptr(out))
        return out

    def rows(self):
        M = self.m
        seq = np.empty(M, np.int32)
        pos = np.empty(M, np.int32)
        real = np.empty(M, np.uint8)
        lib().orc_get_rows(self._h, _ptr(seq), _ptr(pos), _ptr(real))
        return seq, pos, real

    def stats(self) -> Dict[str, np.ndarray]:
        M = self.m
        am = np.empty(M, np.int32)
        conf = np.empty(M, np.float64)
        kl = np.empty(M, np.float64)
        lse = np.empty(M, np.float64)
        hk = np.empty(M, np.uint8)
        lib().orc_get_stats(self._h, _ptr(am), _ptr(conf), _ptr(kl), _ptr(lse), _ptr(hk))
        return dict(argmax=am, conf=conf, kl=kl, lse=lse, has_kl=hk)

    def logits(self):
        R = lib().orc_n_logit_rows(self._h)
        rows = np.empty(R, np.int32)
        z = np.empty((R, self.shape.vocab), np.float64)
        lib().orc_get_logits(self._h, _ptr(rows), _ptr(z))
        return rows, z

    def commits(self):
        n = lib().orc_n_commits(self._h)
        s, p, t = (np.empty(n, np.int32) for _ in range(3))
        lib().orc_get_commits(self._h, _ptr(s), _ptr(p), _ptr(t))
        return s, p, t

    def kv(self, layer: int):
        sh = (self.run.batch, self.shape.n_kv_heads, self.run.seq_len, self.shape.head_dim)
        k = np.empty(sh, np.float64)
        v = np.empty(sh, np.float64)
        lib().orc_get_kv(self._h, layer, _ptr(k), _ptr(v))
        return k, v


# --- the individual steps -----------------------------------------------------

def bf16_round(x: float) -> float:
    return lib().orc_bf16_round(float(x))


def unit_rmsnorm(x, g, eps: float) -> np.ndarray:
    x = _f64(x)
    M, d = x.shape
    g = _f32(g)
    y = np.empty_like(x)
    lib().orc_unit_rmsnorm(_ptr(x), _ptr(g), M, d, float(eps), _ptr(y))
    return y


def unit_rope(u, pos, base: float) -> np.ndarray:
    u = _f64(u).copy()
    M, nh, hd = u.shape
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    lib().orc_unit_rope(_ptr(u), _ptr(pos), M, nh, hd, float(base))
    return u


def unit_linear(x, W) -> np.ndarray:
    x = _f64(x)
    W = _f32(W)
    M, K = x.shape
    N = W.shape[0]
    assert W.shape[1] == K
    y = np.empty((M, N), np.float64)
    lib().orc_unit_linear(_ptr(x), _ptr(W), M, N, K, _ptr(y))
    return y


def unit_attention(q, row_seq, kc, vc) -> np.ndarray:
    """q [M][nq][hd]; kc, vc [B][nkv][N][hd]; row_seq [M] -> o [M][nq][hd]."""
    q = _f64(q)
    kc = _f64(kc)
    vc = _f64(vc)
    M, nq, hd = q.shape
    B, nkv, N, _ = kc.shape
    rs = np.ascontiguousarray(row_seq, dtype=np.int32)
    o = np.empty_like(q)
    lib().orc_unit_attention(_ptr(q), _ptr(rs), _ptr(kc), _ptr(vc), M, B, N, nq, nkv, hd, _ptr(o))
    return o


def unit_vocab_stats(z, prev=None, has_prev=None, mask_id: int = -1, kl_dir: int = 0):
    """z [M][V] logits; prev [M][V] previous log-probabilities (or None)."""
    z = _f64(z)
    M, V = z.shape
    if prev is not None:
        prev = _f64(prev)
        hp = (np.ones(M, np.uint8) if has_prev is None
              else np.ascontiguousarray(has_prev, dtype=np.uint8))
    else:
        hp = None
    lse = np.empty(M)
    am = np.empty(M, np.int32)
    conf = np.empty(M)
    kl = np.empty(M)
    logp = np.empty_like(z)
    lib().orc_unit_vocab_stats(_ptr(z), None if prev is None else _ptr(prev),
                               None if hp is None else _ptr(hp), M, V, mask_id, kl_dir,
                               _ptr(lse), _ptr(am), _ptr(conf), _ptr(kl), _ptr(logp))
    return dict(lse=lse, argmax=am, conf=conf, kl=kl, logp=logp)


def unit_schedule(run, t: int):
    r = make_run(run, dict(kl_eps=0, conf_tau=0, n_consec=1, lock_prompt_after_first_step=0,
                           policy="none"))
    out = np.empty(4, np.int32)
    lib().orc_unit_schedule(ctypes.byref(r), t, _ptr(out))
    return dict(beta=int(out[0]), lo=int(out[1]), hi=int(out[2]), k=int(out[3]))


def unit_lock_transition(shape, run, lock, t, row_seq, row_pos, row_real, argmax, conf, kl,
                         has_kl, x, locked, cnt, refresh=None, drift=None):
    """Commit + lock transition on given statistics.  refresh: optional
    uint8 [B][N] set of locked positions the step recomputed; drift: optional
    float32 [B][N], updated and returned as a fourth value when given."""
    m = make_model(shape)
    r = make_run(run, lock)
    a = [np.ascontiguousarray(row_seq, np.int32), np.ascontiguousarray(row_pos, np.int32),
         np.ascontiguousarray(row_real, np.uint8), np.ascontiguousarray(argmax, np.int32),
         _f64(conf), _f64(kl), np.ascontiguousarray(has_kl, np.uint8)]
    x = np.ascontiguousarray(x, np.int32).copy()
    locked = np.ascontiguousarray(locked, np.uint8).copy()
    cnt = np.ascontiguousarray(cnt, np.int32).copy()
    rf = None if refresh is None else np.ascontiguousarray(refresh, np.uint8)
    dr = None if drift is None else np.ascontiguousarray(drift, np.float32).copy()
    lib().orc_unit_lock_transition(ctypes.byref(m), ctypes.byref(r), t, len(a[0]),
                                   *[_ptr(v) for v in a], _ptr(x), _ptr(locked), _ptr(cnt),
                                   None if rf is None else _ptr(rf),
                                   None if dr is None else _ptr(dr))
    if dr is not None:
        return x, locked, cnt, dr
    return x, locked, cnt


def unit_refresh_select(run, lock, locked, drift) -> np.ndarray:
    """Refresh set (uint8 [B][N]) of a step from the lock state and each
    position's drift: per sequence the refresh_budget locked positions with
    the largest float32 drift, ties to the smaller position."""
    r = make_run(run, lock)
    locked = np.ascontiguousarray(locked, np.uint8)
    drift = np.ascontiguousarray(drift, np.float32)
    out = np.empty(locked.shape, np.uint8)
    lib().orc_unit_refresh_select(ctypes.byref(r), _ptr(locked), _ptr(drift), _ptr(out))
    return out


def unit_slowfast(run, lock, mask_id, pos, argmax, conf, x, frozen, has_prev, state):
    """One SlowFast commit decision for one sequence ([SF] §2): rows (pos
    ascending, argmax, conf) of this step; x, frozen, has_prev [N] and state
    [13] are updated copies.  Returns (commits (pos, tok), x, frozen, has_prev,
    state)."""
    r = make_run(run, lock)
    pos = np.ascontiguousarray(pos, np.int32)
    argmax = np.ascontiguousarray(argmax, np.int32)
    conf = _f64(conf)
    x = np.ascontiguousarray(x, np.int32).copy()
    frozen = np.ascontiguousarray(frozen, np.uint8).copy()
    has_prev = np.ascontiguousarray(has_prev, np.uint8).copy()
    state = np.ascontiguousarray(state, np.int32).copy()
    assert state.shape == (13,) and x.shape == frozen.shape == has_prev.shape
    cp = np.empty(max(1, len(pos)), np.int32)
    ct = np.empty(max(1, len(pos)), np.int32)
    n = lib().orc_unit_slowfast(ctypes.byref(r), int(mask_id), len(x), len(pos), _ptr(pos),
                                _ptr(argmax), _ptr(conf), _ptr(x), _ptr(frozen), _ptr(has_prev),
                                _ptr(state), _ptr(cp), _ptr(ct))
    return (cp[:n], ct[:n]), x, frozen, has_prev, state


def unit_compact(bits, N: int):
    bits = np.ascontiguousarray(bits, dtype=np.uint64)
    B = bits.shape[0]
    seq = np.empty(B * N, np.int32)
    pos = np.empty(B * N, np.int32)
    mb = np.empty(B, np.int32)
    M = lib().orc_unit_compact(_ptr(bits), B, N, _ptr(seq), _ptr(pos), _ptr(mb))
    return seq[:M], pos[:M], mb


def closed_form_flops(shape, m_per_seq: Sequence[int], seq_len: int) -> float:
    """Per-step algorithmic FLOPs of the active-row step: projections and FFN
    on M rows, attention of M queries over N keys, LM head on M rows
    (norms, RoPE, softmax and SiLU excluded)."""
    M = float(sum(m_per_seq))
    d, hd, nq, nkv, dff = (shape.d_model, shape.head_dim, shape.n_heads, shape.n_kv_heads,
                           shape.d_ff)
    proj = d * (nq + 2 * nkv) * hd + nq * hd * d + 3 * d * dff
    attn = 2.0 * seq_len * nq * hd  # per row: QK^T and PV, 2 FLOP per MAC
    return 2.0 * shape.n_layers * (M * proj + M * attn) + 2.0 * M * d * shape.vocab
