"""Lockstep parity of the drift-aware refresh of locked positions.

Polestar page ("Polestar: Drift-Aware Cache Calibration and Token Commitment
...", section "Polestar: The Smart Painter", Polestar-Cache): the cached
positions whose distribution drifts most are recomputed, drift measured by a
KL divergence.  With refresh_budget > 0 the engine, at the start of every
step, recomputes the budget's worth of locked positions per sequence with
the largest drift (the KL between a position's two latest posteriors), and at
the lock update unlocks those whose new drift exceeds refresh_eps.

Each step of these runs compares, beyond the ordinary lockstep checks
(active rows, logits, statistics, tokens, lock bits, counters): the refresh
set bit for bit, and the engine's drift array against the rule applied to
the engine's own statistics.  A refresh set can differ only where the
oracle's drift values at the budget boundary lie within the statistics'
error; the oracle's drift is then replayed ("refresh-rank").  A differing
keep/unlock decision is accepted only within 1e-3 of refresh_eps
("refresh-margin").
"""
import dataclasses

import numpy as np
import pytest

import oracle
import synth
from tests.harness import record, run_lockstep

pytestmark = pytest.mark.gpu

MID = synth.ModelShape(2, 512, 4, 4, 128, 1024, 4096, bf16=True)
MID_RUN = synth.RunShape(2, 192, 64, 32, 64)
DEPTH32 = synth.ModelShape(32, 256, 2, 2, 128, 768, 4096, bf16=True)
RUN = synth.RunShape(1, 512, 128, 128, 384)


def _oracle_counts(shape, W, run, lock, pr, steps):
    """Refreshed positions and refresh unlocks over the oracle's own run."""
    o = oracle.Oracle(shape, W, run, lock, pr)
    n_ref = n_unlock = 0
    for _ in range(steps):
        o.step()
        rf = o.refresh().astype(bool)
        o.lock_update()
        n_ref += int(rf.sum())
        n_unlock += int((rf & (o.locked() == 0)).sum())
    return n_ref, n_unlock


def _check(rec, steps):
    assert rec["steps"] == steps
    why = rec["replay_reasons"]
    assert why.get("argmax", 0) <= max(2, steps // 16), rec
    assert why.get("commit-rank", 0) <= rec["ambiguous_commit_steps"], rec


@pytest.mark.parametrize("setting,budget,eps", [
    ("refresh", 8, 1e-3), ("refresh", 3, 0.0), ("kl_only", 4, 1e-4)])
def test_tiny_fp32_refresh(setting, budget, eps):
    shape, run = synth.CONFIGS["tiny"]
    W = synth.gen_weights(shape)
    pr = synth.gen_prompts(shape, run)
    lock = dict(synth.LOCK_SETTINGS[setting], refresh_budget=budget, refresh_eps=eps)
    n_ref, n_unlock = _oracle_counts(shape, W, run, lock, pr, run.steps)
    assert n_ref > 0
    if eps == 0.0:
        assert n_unlock > 0
    reps = run_lockstep(shape, W, run, lock, pr)
    rec = record(f"tiny/refresh/{setting}/r{budget}/eps{eps:g}", reps, refreshed=n_ref,
                 refresh_unlocks=n_unlock)
    _check(rec, run.steps)


@pytest.mark.parametrize("eps", [1e-3, 0.0])
def test_mid_bf16_refresh(eps):
    W = synth.gen_weights(MID)
    pr = synth.gen_prompts(MID, MID_RUN)
    lock = dict(synth.LOCK_SETTINGS["refresh"], refresh_budget=6, refresh_eps=eps)
    n_ref, n_unlock = _oracle_counts(MID, W, MID_RUN, lock, pr, MID_RUN.steps)
    assert n_ref > 0
    reps = run_lockstep(MID, W, MID_RUN, lock, pr)
    rec = record(f"mid-bf16/refresh/eps{eps:g}", reps, refreshed=n_ref, refresh_unlocks=n_unlock)
    _check(rec, MID_RUN.steps)


@pytest.mark.timeout(1200)
def test_depth32_refresh_lockstep():
    """The LLaDA-8B run shape through 32 bf16 layers at reduced width, with
    the refresh setting (scheduled lock test, 8 refreshed positions per step,
    unlock above a drift of 1e-3), over the first 32 steps."""
    W = synth.gen_weights(DEPTH32)
    pr = synth.gen_prompts(DEPTH32, RUN)
    lock = synth.LOCK_SETTINGS["refresh"]
    steps = 32
    reps = run_lockstep(DEPTH32, W, RUN, lock, pr, steps=steps)
    rec = record("llada-run-shape/depth32/refresh", reps, width=DEPTH32.d_model,
                 layers=DEPTH32.n_layers, seq_len=RUN.seq_len)
    _check(rec, steps)
    # every step after the first recomputes 8 locked positions
    assert all(m >= 8 for m in rec["m_trace"])
