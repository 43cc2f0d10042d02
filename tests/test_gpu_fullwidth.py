"""Parity at full model width: one layer at the LLaDA-8B and Dream-7B widths
and vocabularies, in the launch configurations the bench times (every GEMM,
attention and vocabulary kernel at its real N, K and V; M = 512 and 384 at
LLaDA width).  The oracle computes the whole layer for all active rows and
the LM head and statistics for all rows (LLaDA width, first step) or a
sample of rows; those rows' logits, argmax, confidence, log-normaliser and
KL, and the layer's K/V cache, are compared with the engine's.

At LLaDA width the first step is complete on the oracle's side, so it keeps
every position's posterior; its own commit decision (top-3, prompt locked)
is applied to both sides, and the second step -- M = 384, where the engine
folds the statistics into the LM-head epilogue -- compares the KL of the
sampled rows against the previous posterior at V = 126464, d = 4096
(SureLock page, §2 Methodology: locking condition)."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from selective_token_recompute_amd import engine as E
from tests.harness import append_record, bool_to_bits, conf_bound, logit_tol, top2_gap

pytestmark = pytest.mark.gpu


def _compare_rows(shape, eng, orc, sample, check_kl):
    rs, rp, _ = (a.cpu().numpy() for a in eng.rows())
    seq_o, pos_o, _ = orc.rows()
    assert np.array_equal(rs, seq_o) and np.array_equal(rp, pos_o)
    rows, zo = orc.logits()
    if sample is not None:
        assert np.array_equal(rows, np.asarray(sample, np.int32))
    zg = eng.logits().cpu().numpy()[rs[rows], rp[rows]].astype(np.float64)
    fin = np.isfinite(zo)
    assert np.array_equal(fin, np.isfinite(zg))
    with np.errstate(invalid="ignore"):  # -inf - -inf at the mask column
        dz = np.abs(np.where(fin, zg - zo, 0.0))
    scale = float(np.abs(zo[fin]).max())
    assert dz.max() <= logit_tol(shape, scale), (dz.max(), scale)
    so = orc.stats()
    sg = {k: v.cpu().numpy() for k, v in eng.stats().items()}
    gap = top2_gap(zo, shape.mask_id)
    near_tie = gap <= np.maximum(2.0 * dz.max(axis=1), 1e-6 * max(scale, 1.0))
    bad = sg["argmax"][rows] != so["argmax"][rows]
    assert not (bad & ~near_tie).any()
    assert np.allclose(sg["lse"][rows], so["lse"][rows], rtol=0, atol=2e-2 * max(scale, 1.0))
    dconf = np.abs(sg["conf"][rows] - so["conf"][rows])
    assert (dconf <= conf_bound(so["conf"][rows], dz.max(axis=1))).all(), \
        (dconf / so["conf"][rows]).max()
    kl_note = ""
    if check_kl:
        hk = so["has_kl"][rows].astype(bool)
        assert np.array_equal(sg["has_kl"][rows].astype(bool), hk)
        if hk.any():
            ko, kg = so["kl"][rows][hk], sg["kl"][rows][hk].astype(np.float64)
            dkl = np.abs(kg - ko)
            # the bf16 bar of the lockstep harness
            assert (dkl <= 1e-4 + 5e-2 * np.abs(ko)).all(), (dkl.max(), ko)
            kl_note = (f" KL rows={int(hk.sum())} KL range=[{ko.min():.3g}, {ko.max():.3g}] "
                       f"max|dKL|={dkl.max():.3g}")
            append_record(dict(name=f"fullwidth/d{shape.d_model}/V{shape.vocab}/kl",
                               M=int(len(rs)), rows=int(hk.sum()), kl_min=float(ko.min()),
                               kl_max=float(ko.max()), max_dkl=float(dkl.max()),
                               max_dz=float(dz.max()), z_scale=scale))
    print(f"\n[fullwidth] M={len(rs)} sample={len(rows)} max|dz|={dz.max():.3g} "
          f"scale={scale:.3g} argmax near-tie differences={int(bad.sum())}{kl_note}", flush=True)
    return int(hk.sum()) if check_kl else 0


def _compare_kv(eng, orc, shape):
    kg, vg = eng.kv_cache()
    for layer in range(shape.n_layers):
        ko, vo = orc.kv(layer)
        got_k = kg[layer].float().cpu().numpy()
        got_v = vg[layer].float().cpu().numpy().transpose(0, 1, 3, 2)
        for got, want in ((got_k, ko), (got_v, vo)):
            scale = float(np.abs(want).max())
            err = np.abs(got - want)
            assert (err <= 2.0 ** -7 * np.abs(want) + 1e-3 * scale).all(), (err.max(), scale)


def _run(shape, run, sample_fn, second_step, full_first=False):
    W = synth.gen_weights(shape)
    pr = synth.gen_prompts(shape, run)
    lock = synth.LOCK_SETTINGS["natural"]
    dev = torch.device("cuda")
    eng = E.Engine(shape, E.upload_weights(W, shape, dev), run, lock,
                   torch.from_numpy(pr).to(dev))
    orc = oracle.Oracle(shape, W, run, lock, pr)
    M0 = eng.step()
    sample = None if full_first else sample_fn(M0)
    orc.step(sample_rows=sample)
    torch.cuda.synchronize()
    _compare_rows(shape, eng, orc, sample, check_kl=True)
    _compare_kv(eng, orc, shape)
    kl_rows = 0
    if second_step:
        if full_first:
            # the oracle's own transition (top-3 commit, prompt locked), applied
            # to the engine as an override so that both sides continue from
            # the same state with a changed context
            orc.lock_update()
            cs, cp, ct = orc.commits()
            assert len(cs) == 3
            eng.lock_update(commits=(cs, cp, ct), lock_bits=bool_to_bits(orc.locked()),
                            counters=orc.counters())
        else:
            # the same decision on both sides: nothing committed, the prompt locked
            locked = np.zeros((run.batch, run.seq_len), np.uint8)
            locked[:, : run.prompt_len] = 1
            none = (np.zeros(0, np.int32),) * 3
            orc.lock_update(commits=none, locked=locked)
            eng.lock_update(commits=none, lock_bits=bool_to_bits(locked))
        M1 = eng.step()
        assert M1 == run.batch * (run.seq_len - run.prompt_len)
        sample = sample_fn(M1)
        orc.step(sample_rows=sample)
        torch.cuda.synchronize()
        # KL is defined where the oracle kept the previous posterior (every
        # position after a complete first step)
        kl_rows = _compare_rows(shape, eng, orc, sample, check_kl=full_first)
        _compare_kv(eng, orc, shape)
    eng.close()
    return kl_rows


def _spread(M, n=8):
    return sorted(set(int(x) for x in np.linspace(0, M - 1, n)))


@pytest.mark.timeout(900)
def test_llada_width_one_layer():
    shape = dataclasses.replace(synth.CONFIGS["llada8b"][0], n_layers=1)
    _, run = synth.CONFIGS["llada8b"]
    kl_rows = _run(shape, run, lambda M: _spread(M, 16), second_step=True, full_first=True)
    assert kl_rows == 16


def test_dream_width_one_layer_batched_gqa():
    shape = dataclasses.replace(synth.CONFIGS["dream7b"][0], n_layers=1)
    run = synth.RunShape(2, 256, 64, 16, 192)
    _run(shape, run, _spread, second_step=False)
