"""Pins of the oracle's drift-aware refresh of locked positions (-m "not gpu").

Polestar page ("Polestar: Drift-Aware Cache Calibration and Token Commitment
...", section "Polestar: The Smart Painter", Polestar-Cache): rather than
keeping every cached position frozen, recompute only the positions whose
understanding drifts most, the drift measured as a KL divergence between the
position's successive distributions.  The oracle's reading: a position's
drift is the KL (run's direction) between its two latest posteriors, float32,
+inf while undefined; each step the refresh_budget locked positions of a
sequence with the largest drift (ties: smaller position) are recomputed; a
recomputed position whose new drift exceeds refresh_eps is unlocked.

What pins it to something other than itself:
- refreshing every locked position and keeping none is vanilla full
  recompute (the independent NumPy O2), to 1e-10 on every logit;
- a refreshed position whose inputs did not change reproduces its cached
  posterior bit for bit: drift exactly 0, and it stays locked;
- each refreshed position's drift is the KL, computed here with scipy,
  between its posterior now and the one it had when it was last computed
  (kept from the run's own trace), in the run's KL direction;
- the selection and the transition on hand-worked cases;
- the invariants of the rule over whole runs.
"""
import dataclasses

import numpy as np
import pytest
import scipy.special

import oracle
import synth
from oracle import naive


@pytest.fixture(scope="module")
def tiny():
    shape, run = synth.CONFIGS["tiny"]
    return shape, run, synth.gen_weights(shape), synth.gen_prompts(shape, run)


def _trace(shape, W, run, lock, prompts, overrides=None):
    o = oracle.Oracle(shape, W, run, lock, prompts)
    out = []
    for t in range(run.steps):
        x_in, lk_in, cnt_in, dr_in = o.tokens(), o.locked(), o.counters(), o.drift()
        o.step()
        seq, pos, real = o.rows()
        st = o.stats()
        z = o.logits()[1]
        rf = o.refresh()
        if overrides and t in overrides:
            o.lock_update(**overrides[t])
        else:
            o.lock_update()
        out.append(dict(t=t, x_in=x_in, locked_in=lk_in, cnt_in=cnt_in, drift_in=dr_in,
                        seq=seq, pos=pos, real=real, stats=st, logits=z, refresh=rf, m=o.m,
                        x_out=o.tokens(), locked_out=o.locked(), cnt_out=o.counters(),
                        drift_out=o.drift()))
    return out


def _finite_diff(a, b):
    a = np.where(np.isinf(a), 0.0, a)
    b = np.where(np.isinf(b), 0.0, b)
    return float(np.abs(a - b).max())


def test_refresh_all_keep_none_is_full_recompute(tiny):
    """Budget N with refresh_eps < 0: every locked position is recomputed at
    every step and unlocked, so every step computes all N positions over a
    fully fresh cache: the logits and tokens of vanilla decoding (O2)."""
    shape, run, W, pr = tiny
    ref = naive.generate(shape, W, run, pr)
    lock = dict(synth.LOCK_SETTINGS["scheduled"], refresh_budget=run.seq_len, refresh_eps=-1.0)
    tr = _trace(shape, W, run, lock, pr)
    assert any(st["refresh"].any() for st in tr), "nothing was refreshed"
    for t, st in enumerate(tr):
        assert st["m"] == run.seq_len
        assert _finite_diff(st["logits"], ref["logits"][t][0]) <= 1e-10
        assert np.array_equal(st["x_out"], ref["tokens"][t])
        # every refreshed position was unlocked by the rule
        assert not (st["refresh"].astype(bool) & st["locked_out"].astype(bool)).any()


def test_budget_zero_is_the_setting_without_refresh(tiny):
    shape, run, W, pr = tiny
    a = _trace(shape, W, run, synth.LOCK_SETTINGS["scheduled"], pr)
    b = _trace(shape, W, run, dict(synth.LOCK_SETTINGS["refresh"], refresh_budget=0), pr)
    for x, y in zip(a, b):
        assert np.array_equal(x["logits"], y["logits"])
        assert np.array_equal(x["x_out"], y["x_out"])
        assert np.array_equal(x["locked_out"], y["locked_out"])
        assert not y["refresh"].any()


def test_refresh_without_change_reproduces_the_cached_posterior(tiny):
    """Step t commits nothing (override) and locks every real position
    (override); step t+1 then recomputes locked positions whose inputs are
    all unchanged: their posterior is bitwise the one cached, drift 0, and
    they stay locked (refresh_eps 0)."""
    shape, run, W, pr = tiny
    lock = dict(synth.LOCK_SETTINGS["kl_only"], refresh_budget=4, refresh_eps=0.0)
    o = oracle.Oracle(shape, W, run, lock, pr)
    N = run.seq_len
    for _ in range(3):  # a few ordinary steps so that some tokens are decoded
        o.step()
        o.lock_update()
    x = o.tokens()
    o.step()
    seq, pos, real = o.rows()
    rows_t, z_t = o.logits()
    # commit nothing; lock every real position of this step
    lk = np.zeros((1, N), np.uint8)
    lk[0, pos[real == 1]] = 1
    o.lock_update(commits=(np.zeros(0), np.zeros(0), np.zeros(0)), locked=lk)
    assert np.array_equal(o.tokens(), x)
    drift_before = o.drift()
    locked_before = o.locked()
    o.step()
    rf = o.refresh()
    assert rf.sum() == 4
    seq2, pos2, _ = o.rows()
    st = o.stats()
    _, z2 = o.logits()
    last = {int(p): i for i, p in enumerate(pos)}
    for i, p in enumerate(pos2):
        if rf[0, p]:
            assert p in last
            assert np.array_equal(z2[i], z_t[last[p]]), "recomputed posterior differs"
            assert st["has_kl"][i] == 1 and st["kl"][i] == 0.0
    # the four chosen: the locked positions with the largest drift (ties:
    # smaller position)
    cand = np.nonzero(locked_before[0])[0]
    order = sorted(cand, key=lambda p: (-float(drift_before[0, p]), p))
    assert sorted(np.nonzero(rf[0])[0].tolist()) == sorted(order[:4])
    o.lock_update()
    assert (o.locked()[rf == 1] == 1).all(), "a drift-0 refresh unlocked its position"
    assert (o.drift()[rf == 1] == 0.0).all()


@pytest.mark.parametrize("kl_dir", [0, 1])
def test_drift_is_kl_against_the_posterior_when_last_computed(tiny, kl_dir):
    shape, run, W, pr = tiny
    lock = dict(synth.LOCK_SETTINGS["refresh"], refresh_budget=3, kl_dir=kl_dir)
    tr = _trace(shape, W, run, lock, pr)
    last = {}  # position -> log-probabilities at its last computation
    n_checked = 0
    for st in tr:
        lp = scipy.special.log_softmax(np.where(np.isinf(st["logits"]), -1e300, st["logits"]),
                                       axis=1)
        keep = np.arange(shape.vocab) != shape.mask_id
        for i, p in enumerate(st["pos"]):
            if st["refresh"][0, p]:
                a, b = lp[i][keep], last[int(p)][keep]
                if kl_dir == 0:
                    kl = float(np.sum(np.exp(a) * (a - b)))
                else:
                    kl = float(np.sum(np.exp(b) * (b - a)))
                assert st["stats"]["kl"][i] == pytest.approx(kl, rel=1e-9, abs=1e-13)
                assert st["drift_out"][0, p] == np.float32(st["stats"]["kl"][i])
                n_checked += 1
            last[int(p)] = lp[i]
    assert n_checked >= 3 * (run.steps - 2)


def test_selection_hand_worked():
    run = synth.RunShape(2, 10, 2, 4, 8)
    lock = dict(synth.LOCK_SETTINGS["refresh"], refresh_budget=3)
    inf = np.inf
    locked = np.array([[1, 1, 0, 1, 1, 0, 1, 1, 0, 0],
                       [0, 1, 0, 0, 0, 0, 0, 0, 0, 1]], np.uint8)
    drift = np.array([[0.5, inf, 9.0, 2e-3, 2e-3, 7.0, 1e-5, inf, 0.0, 0.0],
                      [0.0, 1e-4, 5.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 3e-4]], np.float32)
    sel = oracle.unit_refresh_select(run, lock, locked, drift)
    # sequence 0: +inf at 1 and 7 (1 first), then 0.5 at 0; the unlocked 2 and
    # 5 (drift 9, 7) are not candidates; sequence 1: only two are locked
    assert np.nonzero(sel[0])[0].tolist() == [0, 1, 7]
    assert np.nonzero(sel[1])[0].tolist() == [1, 9]
    # a tie at the boundary goes to the smaller position
    drift[0, [0, 1, 3, 4, 7]] = 1e-3
    sel = oracle.unit_refresh_select(run, dict(lock, refresh_budget=2), locked, drift)
    assert np.nonzero(sel[0])[0].tolist() == [0, 1]
    assert not oracle.unit_refresh_select(run, dict(lock, refresh_budget=0), locked, drift).any()


def test_transition_of_refreshed_rows_hand_worked():
    shape = synth.ModelShape(1, 8, 1, 1, 8, 8, 16, bf16=False)
    run = synth.RunShape(1, 8, 2, 4, 6)
    lock = dict(policy="test", kl_eps=1e-3, conf_tau=0.0, n_consec=2,
                lock_prompt_after_first_step=1, refresh_budget=3, refresh_eps=1e-3)
    mask = shape.mask_id
    x = np.array([[3, 4, 5, 6, mask, mask, 7, mask]], np.int32)
    locked = np.array([[1, 1, 1, 0, 0, 0, 0, 0]], np.uint8)
    cnt = np.array([[0, 0, 2, 1, 0, 0, 1, 0]], np.int32)
    refresh = np.array([[1, 1, 1, 0, 0, 0, 0, 0]], np.uint8)
    drift = np.full((1, 8), np.inf, np.float32)
    drift[0, 2] = 0.25
    rows = [0, 1, 2, 3, 4, 5, 6, 7]
    real = (x[0] != mask).astype(np.uint8)
    # refreshed: 0 kl 5e-4 (stays), 1 kl 2e-3 (unlocked), 2 no KL (unlocked);
    # 3 passes (cnt 1 -> 2, locks); 6 fails (kl 5e-3, cnt -> 0); 4, 5, 7 masked
    kl = [5e-4, 2e-3, 0.0, 1e-4, 0.0, 0.0, 5e-3, 0.0]
    has_kl = [1, 1, 0, 1, 1, 1, 1, 1]
    conf = [0.5] * 8
    argmax = [1] * 8
    x2, lk2, cnt2, dr2 = oracle.unit_lock_transition(
        shape, run, lock, 3, [0] * 8, rows, real, argmax, conf, kl, has_kl, x, locked, cnt,
        refresh=refresh, drift=drift)
    assert lk2.tolist() == [[1, 0, 0, 1, 0, 0, 0, 0]]
    assert cnt2.tolist() == [[0, 0, 0, 2, 0, 0, 0, 0]]
    assert dr2[0].tolist() == [np.float32(5e-4), np.float32(2e-3), np.inf, np.float32(1e-4),
                               0.0, 0.0, np.float32(5e-3), 0.0]
    # without the refresh set the refreshed rows take the ordinary lock test
    _, lk3, cnt3 = oracle.unit_lock_transition(
        shape, run, lock, 3, [0] * 8, rows, real, argmax, conf, kl, has_kl, x, locked, cnt)
    assert lk3.tolist() == [[1, 1, 1, 1, 0, 0, 0, 0]]
    assert cnt3.tolist() == [[1, 0, 0, 2, 0, 0, 0, 0]]


@pytest.mark.parametrize("setting,budget,eps", [("refresh", 8, 1e-3), ("refresh", 3, 0.0),
                                                ("kl_only", 5, 1e-2)])
def test_refresh_invariants(tiny, setting, budget, eps):
    shape, run, W, pr = tiny
    lock = dict(synth.LOCK_SETTINGS[setting], refresh_budget=budget, refresh_eps=eps)
    tr = _trace(shape, W, run, lock, pr)
    any_unlock = False
    for st in tr:
        lin, lout = st["locked_in"].astype(bool), st["locked_out"].astype(bool)
        rf = st["refresh"].astype(bool)
        assert not (rf & ~lin).any(), "refreshed a position that was not locked"
        for b in range(run.batch):
            assert rf[b].sum() == min(budget, lin[b].sum())
        # active set: unlocked or refreshed
        act = np.zeros_like(lin)
        act[st["seq"], st["pos"]] = True
        assert np.array_equal(act, ~lin | rf)
        # a lock is released only at a refreshed position whose drift exceeds
        # refresh_eps (or has no KL)
        released = lin & ~lout
        assert not (released & ~rf).any()
        row = {(int(s), int(p)): i for i, (s, p) in enumerate(zip(st["seq"], st["pos"]))}
        for b, p in zip(*np.nonzero(rf)):
            i = row[(b, p)]
            keep = st["stats"]["has_kl"][i] and st["stats"]["kl"][i] <= eps
            assert lout[b, p] == keep
            any_unlock |= not keep
        # tokens: decoded positions never change; masked positions never lock
        xin, xout = st["x_in"], st["x_out"]
        dec = xin != shape.mask_id
        assert np.array_equal(xin[dec], xout[dec])
        assert not (lout & (xout == shape.mask_id)).any()
    assert (tr[-1]["x_out"] != shape.mask_id).all()
    if eps == 0.0:
        assert any_unlock, "no refreshed position was unlocked"


def test_refresh_with_slowfast_is_rejected(tiny):
    shape, run, W, pr = tiny
    lock = dict(synth.LOCK_SETTINGS["slowfast"], refresh_budget=2, refresh_eps=1e-3)
    with pytest.raises(ValueError):
        oracle.Oracle(shape, W, run, lock, pr)


def test_refresh_bf16_storage_runs_and_keeps_invariants():
    shape, run = synth.CONFIGS["tiny"]
    shape = dataclasses.replace(shape, bf16=True)
    W = synth.gen_weights(shape)
    pr = synth.gen_prompts(shape, run)
    tr = _trace(shape, W, run, synth.LOCK_SETTINGS["refresh"], pr)
    assert any(st["refresh"].any() for st in tr)
    assert (tr[-1]["x_out"] != shape.mask_id).all()
