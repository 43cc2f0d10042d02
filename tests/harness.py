"""Lockstep GPU-vs-oracle replay harness for step-level parity.

Each step runs on both sides from the same state.  Logits and statistics are
compared within tolerance; the commit and lock decisions must match bit for
bit, except where the oracle's own decision sits inside a margin (near-tied
argmax or confidence ranking, or a lock comparison within 1e-3 of its
threshold): there the oracle's decision is replayed into the engine through
the lock-update override and the replay is counted.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np
import torch

import oracle
import synth
from selective_token_recompute_amd import engine as E

MARGIN = 1e-3  # lock-test margin on |KL - eps| and |conf - tau|


@dataclasses.dataclass
class StepReport:
    t: int
    m: int
    max_dz: float
    z_scale: float
    replayed: bool
    reasons: List[str]
    argmax_mismatch_near_tie: int
    max_dconf: float
    max_dkl: float


def bits_to_bool(bits: np.ndarray, N: int) -> np.ndarray:
    B, W = bits.shape
    out = np.zeros((B, N), dtype=np.uint8)
    u = bits.astype(np.uint64)
    for i in range(N):
        out[:, i] = ((u[:, i // 64] >> np.uint64(i % 64)) & np.uint64(1)).astype(np.uint8)
    return out


def bool_to_bits(locked: np.ndarray) -> np.ndarray:
    B, N = locked.shape
    W = (N + 63) // 64
    out = np.zeros((B, W), dtype=np.uint64)
    for b in range(B):
        for i in np.nonzero(locked[b])[0]:
            out[b, i // 64] |= np.uint64(1) << np.uint64(i % 64)
    return out


def logit_tol(shape, scale: float) -> float:
    return 2e-2 * scale if shape.bf16 else 1e-4 * max(1.0, scale)


def top2_gap(z: np.ndarray, mask_id: int) -> np.ndarray:
    zz = z.copy()
    zz[:, mask_id] = -np.inf
    part = np.partition(zz, -2, axis=1)
    return part[:, -1] - part[:, -2]


def explain_difference(shape, run, lock, t, x_before, x_g, x_o, lk_g, lk_o, cnt_g, cnt_o,
                       seq_o, pos_o, real_o, so, near_tie, dconf, dkl):
    """Asserts that every decision where engine and oracle differ sits inside
    a margin; returns the list of margins used."""
    reasons = set()
    row_of = {(int(b), int(p)): i for i, (b, p) in enumerate(zip(seq_o, pos_o))}
    sch = oracle.unit_schedule(run, t)
    conf_tol = 2.0 * float(dconf.max()) + 1e-7
    diff_tok = np.argwhere(x_g != x_o)
    for b, p in diff_tok:
        i = row_of[(int(b), int(p))]
        orc_committed = x_o[b, p] != x_before[b, p]
        gpu_committed = x_g[b, p] != x_before[b, p]
        if orc_committed and gpu_committed:
            assert near_tie[i], f"step {t}: ({b},{p}) committed a different token outside a tie"
            reasons.add("argmax")
        else:
            sel = (seq_o == b) & (pos_o >= sch["lo"]) & (pos_o < sch["hi"]) & \
                (x_before[b, pos_o] == shape.mask_id)
            c = np.sort(so["conf"][sel])[::-1]
            k = sch["k"]
            assert 0 < k < len(c) and c[k - 1] - c[k] <= conf_tol, \
                f"step {t}: commit set differs at ({b},{p}) outside a confidence tie"
            reasons.add("commit-rank")
    diff_lock = np.argwhere((lk_g != lk_o) | (cnt_g != cnt_o))
    eps, tau = float(lock["kl_eps"]), float(lock["conf_tau"])
    for b, p in diff_lock:
        i = row_of.get((int(b), int(p)))
        assert i is not None and real_o[i] and so["has_kl"][i], \
            f"step {t}: lock state differs at ({b},{p}) where no test applies"
        near_kl = abs(so["kl"][i] - eps) < MARGIN
        near_cf = abs(so["conf"][i] - tau) < MARGIN
        assert near_kl or near_cf, f"step {t}: lock decision differs at ({b},{p}) outside margin"
        reasons.add("lock-margin")
    return sorted(reasons)


def run_lockstep(shape, W: Dict, run, lock: Dict, prompts: np.ndarray, steps: Optional[int] = None,
                 dev_weights: Optional[Dict] = None, check=True) -> List[StepReport]:
    """Runs `steps` steps on engine and oracle in lockstep; asserts parity."""
    dev = torch.device("cuda")
    dw = dev_weights if dev_weights is not None else E.upload_weights(W, shape, dev)
    eng = E.Engine(shape, dw, run, lock, torch.from_numpy(prompts).to(dev))
    orc = oracle.Oracle(shape, W, run, lock, prompts)
    B, N, V = run.batch, run.seq_len, shape.vocab
    reports = []
    T = run.steps if steps is None else steps
    for t in range(T):
        x_before = orc.tokens()
        m_gpu = eng.step()
        orc.step()
        torch.cuda.synchronize()
        seq_o, pos_o, real_o = orc.rows()
        assert m_gpu == orc.m, f"step {t}: active count {m_gpu} vs oracle {orc.m}"
        rs, rp, rr = (a.cpu().numpy() for a in eng.rows())
        assert np.array_equal(rs, seq_o) and np.array_equal(rp, pos_o), f"step {t}: active rows"
        assert np.array_equal(rr.astype(np.uint8), real_o), f"step {t}: real flags"
        _, _, flops = eng.last_step_info()
        cf = oracle.closed_form_flops(shape, [orc.m], N)
        assert abs(flops - cf) <= 1e-9 * max(cf, 1.0), f"step {t}: FLOP count {flops} vs {cf}"
        if orc.m == 0:
            orc.lock_update()
            eng.lock_update()
            continue
        _, zo = orc.logits()
        zg = eng.logits().cpu().numpy()[rs, rp]
        fin = np.isfinite(zo)
        assert np.array_equal(fin, np.isfinite(zg)), f"step {t}: -inf pattern"
        dz = np.abs(np.where(fin, zg - zo, 0.0))
        scale = float(np.abs(zo[fin]).max())
        max_dz = float(dz.max())
        if check:
            assert max_dz <= logit_tol(shape, scale), \
                f"step {t}: logits max|dz|={max_dz:.3g} scale={scale:.3g}"
        so = orc.stats()
        sg = {k: v.cpu().numpy() for k, v in eng.stats().items()}
        row_dz = dz.max(axis=1)
        gap = top2_gap(zo, shape.mask_id)
        near_tie = gap <= np.maximum(2.0 * row_dz, 1e-6 * max(scale, 1.0))
        am_bad = sg["argmax"] != so["argmax"]
        assert not (am_bad & ~near_tie).any(), f"step {t}: argmax differs outside a near tie"
        dconf = np.abs(sg["conf"] - so["conf"])
        assert (dconf <= 1e-5 + 2.0 * so["conf"] * (5e-3 if shape.bf16 else 1e-4)).all() or not check, \
            f"step {t}: conf"
        assert np.array_equal(sg["has_kl"].astype(np.uint8), so["has_kl"]), f"step {t}: has_kl"
        hk = so["has_kl"].astype(bool)
        dkl = np.abs(sg["kl"][hk] - so["kl"][hk]) if hk.any() else np.zeros(1)
        kl_tol = (2e-6 + 1e-3 * np.abs(so["kl"][hk])) if not shape.bf16 else (
            1e-4 + 5e-2 * np.abs(so["kl"][hk]))
        if check and hk.any():
            assert (dkl <= kl_tol).all(), f"step {t}: KL max diff {dkl.max():.3g}"

        # oracle decision (the authority), then the engine's own decision
        orc.lock_update()
        x_o, lk_o, cnt_o = orc.tokens(), orc.locked(), orc.counters()
        cs, cp, ct = orc.commits()
        tok_v, bits_v, cnt_v = eng.tokens(), eng.lock_bits(), eng.counters()
        eng.lock_update()
        torch.cuda.synchronize()
        x_g = tok_v.cpu().numpy()
        lk_g = bits_to_bool(bits_v.cpu().numpy().view(np.uint64), N)
        cnt_g = cnt_v.cpu().numpy()
        reasons = []
        if not (np.array_equal(x_g, x_o) and np.array_equal(lk_g, lk_o)
                and np.array_equal(cnt_g, cnt_o)):
            reasons = explain_difference(shape, run, lock, t, x_before, x_g, x_o, lk_g, lk_o,
                                         cnt_g, cnt_o, seq_o, pos_o, real_o, so, near_tie,
                                         dconf, dkl if hk.any() else None)
            # every difference lies inside a margin: replay the oracle's decision
            # into the engine's state
            tok_v.copy_(torch.from_numpy(x_o).to(tok_v.device))
            bits_v.copy_(torch.from_numpy(bool_to_bits(lk_o).view(np.int64)).to(bits_v.device))
            cnt_v.copy_(torch.from_numpy(cnt_o).to(cnt_v.device))
            torch.cuda.synchronize()
        replay = bool(reasons)
        reports.append(StepReport(t, orc.m, max_dz, scale, replay, reasons,
                                  int((am_bad & near_tie).sum()), float(dconf.max()),
                                  float(dkl.max())))
    eng.close()
    return reports
