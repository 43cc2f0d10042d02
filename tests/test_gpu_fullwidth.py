"""Parity at full model width: one layer at the LLaDA-8B and Dream-7B widths
and vocabularies, in the launch configurations the bench times (every GEMM,
attention and vocabulary kernel at its real N, K and V; M = 512 and 384 at
LLaDA width).  The oracle computes the whole layer for all active rows and
the LM head and statistics for a sample of rows; those rows' logits,
argmax, confidence and log-normaliser, and the layer's K/V cache, are
compared with the engine's."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from selective_token_recompute_amd import engine as E
from tests.harness import bool_to_bits, logit_tol, top2_gap

pytestmark = pytest.mark.gpu


def _compare_rows(shape, eng, orc, sample, check_kl):
    rs, rp, _ = (a.cpu().numpy() for a in eng.rows())
    seq_o, pos_o, _ = orc.rows()
    assert np.array_equal(rs, seq_o) and np.array_equal(rp, pos_o)
    rows, zo = orc.logits()
    assert np.array_equal(rows, np.asarray(sample, np.int32))
    zg = eng.logits().cpu().numpy()[rs[rows], rp[rows]].astype(np.float64)
    fin = np.isfinite(zo)
    assert np.array_equal(fin, np.isfinite(zg))
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
    assert (np.abs(sg["conf"][rows] - so["conf"][rows]) <= 1e-5 + 1e-2 * so["conf"][rows]).all()
    if check_kl:
        assert np.array_equal(sg["has_kl"][rows].astype(np.uint8), so["has_kl"][rows])
    print(f"\n[fullwidth] M={len(rs)} sample={len(rows)} max|dz|={dz.max():.3g} "
          f"scale={scale:.3g} argmax near-tie differences={int(bad.sum())}", flush=True)


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


def _run(shape, run, sample_fn, second_step):
    W = synth.gen_weights(shape)
    pr = synth.gen_prompts(shape, run)
    lock = synth.LOCK_SETTINGS["natural"]
    dev = torch.device("cuda")
    eng = E.Engine(shape, E.upload_weights(W, shape, dev), run, lock,
                   torch.from_numpy(pr).to(dev))
    orc = oracle.Oracle(shape, W, run, lock, pr)
    M0 = eng.step()
    sample = sample_fn(M0)
    orc.step(sample_rows=sample)
    torch.cuda.synchronize()
    _compare_rows(shape, eng, orc, sample, check_kl=True)
    _compare_kv(eng, orc, shape)
    if second_step:
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
        # the oracle's sampled first step kept no previous posterior: KL not compared
        _compare_rows(shape, eng, orc, sample, check_kl=False)
        _compare_kv(eng, orc, shape)
    eng.close()


def _spread(M, n=8):
    return sorted(set(int(x) for x in np.linspace(0, M - 1, n)))


def test_llada_width_one_layer():
    shape = dataclasses.replace(synth.CONFIGS["llada8b"][0], n_layers=1)
    _, run = synth.CONFIGS["llada8b"]
    _run(shape, run, _spread, second_step=True)


def test_dream_width_one_layer_batched_gqa():
    shape = dataclasses.replace(synth.CONFIGS["dream7b"][0], n_layers=1)
    run = synth.RunShape(2, 256, 64, 16, 192)
    _run(shape, run, _spread, second_step=False)
