"""Checkpoint and resume through the C ABI (dlm_checkpoint_save / load): a
run saved at a step boundary and resumed in a fresh handle, or rewound in the
same handle, continues bitwise as the uninterrupted run did (tokens, lock
bits, counters, SlowFast state, drift and refresh set, per-row statistics,
logits and K/V cache at every later step), with host and device images; plus
the refusals."""
import numpy as np
import pytest
import torch

import synth
from selective_token_recompute_amd import _lib as L
from selective_token_recompute_amd import engine as E

pytestmark = pytest.mark.gpu

MID = synth.ModelShape(2, 512, 4, 4, 128, 1024, 4096, bf16=True)
MID_RUN = synth.RunShape(2, 192, 64, 32, 64)

CASES = {
    "tiny-fp32-natural": (synth.CONFIGS["tiny"][0], synth.CONFIGS["tiny"][1], "natural", 5),
    "mid-bf16-scheduled": (MID, MID_RUN, "scheduled", 7),
    "mid-bf16-slowfast": (MID, MID_RUN, "slowfast", 9),
    "mid-bf16-refresh": (MID, MID_RUN, "refresh", 9),
}


def _bits(t: torch.Tensor) -> torch.Tensor:
    """Raw bytes of a tensor, for bitwise comparison of any dtype."""
    return t.contiguous().view(torch.uint8).cpu()


def _snapshot(eng: E.Engine, with_rows: bool) -> dict:
    s = dict(tokens=eng.tokens(), bits=eng.lock_bits(), counters=eng.counters(),
             frozen=eng.frozen_bits(), sf=eng.sf_state(), has_prev=eng.has_prev(),
             drift=eng.drift(), refresh=eng.refresh_bits())
    kc, vc = eng.kv_cache()
    s.update(kc=kc, vc=vc)
    if with_rows:
        m = eng.m
        rs, rp = (a[:m].long() for a in eng.rows()[:2])
        s["rows"] = torch.stack([rs, rp])
        s["logits"] = eng.logits()[rs, rp]
        for k, v in eng.stats().items():
            s["stat_" + k] = v[:m]
    return {k: _bits(v) for k, v in s.items()}


def _assert_same(a: dict, b: dict, where: str):
    assert a.keys() == b.keys(), where
    for k in a:
        assert torch.equal(a[k], b[k]), f"{where}: {k}"


def _engine(shape, run, lock, W, pr):
    dev = torch.device("cuda")
    return E.Engine(shape, E.upload_weights(W, shape, dev), run, lock,
                    torch.from_numpy(pr).to(dev))


def _run_to_end(eng, t0, steps):
    """Steps t0 .. steps-1; per step the snapshot after dlm_step (rows,
    statistics, logits) and after dlm_lock_update."""
    out = []
    for t in range(t0, steps):
        eng.step()
        mid = _snapshot(eng, with_rows=True)
        eng.lock_update()
        out.append((mid, _snapshot(eng, with_rows=False)))
    return out


@pytest.mark.parametrize("case", list(CASES))
def test_resume_and_rewind_continue_bitwise(case):
    shape, run, setting, k = CASES[case]
    lock = synth.LOCK_SETTINGS[setting]
    W = synth.gen_weights(shape)
    pr = synth.gen_prompts(shape, run)
    steps = min(run.steps, k + 8)

    e1 = _engine(shape, run, lock, W, pr)
    for _ in range(k):
        e1.step()
        e1.lock_update()
    host = e1.save_checkpoint()
    dev = torch.empty(e1.checkpoint_bytes(), dtype=torch.uint8, device="cuda")
    e1.save_checkpoint(dev)
    assert np.array_equal(host, dev.cpu().numpy())
    at_save = _snapshot(e1, with_rows=False)
    ref = _run_to_end(e1, k, steps)
    info_end = e1.last_step_info()

    # a fresh handle resumed from the host image
    e2 = _engine(shape, run, lock, W, pr)
    e2.load_checkpoint(host)
    _assert_same(at_save, _snapshot(e2, with_rows=False), "after load")
    assert e2.last_step_info()[0] == k - 1
    got = _run_to_end(e2, k, steps)
    for i, ((rm, ru), (gm, gu)) in enumerate(zip(ref, got)):
        _assert_same(rm, gm, f"resumed step {k + i} (posterior)")
        _assert_same(ru, gu, f"resumed step {k + i} (update)")
    assert e2.last_step_info() == info_end

    # the first handle rewound from the device image
    e1.load_checkpoint(dev)
    _assert_same(at_save, _snapshot(e1, with_rows=False), "after rewind")
    got = _run_to_end(e1, k, steps)
    for i, ((rm, ru), (gm, gu)) in enumerate(zip(ref, got)):
        _assert_same(rm, gm, f"rewound step {k + i} (posterior)")
        _assert_same(ru, gu, f"rewound step {k + i} (update)")
    e1.close()
    e2.close()


def test_checkpoint_at_step_zero_and_after_the_last_step():
    shape, run = synth.CONFIGS["tiny"]
    lock = synth.LOCK_SETTINGS["scheduled"]
    W = synth.gen_weights(shape)
    pr = synth.gen_prompts(shape, run)
    e1 = _engine(shape, run, lock, W, pr)
    img0 = e1.save_checkpoint()
    ref = _run_to_end(e1, 0, run.steps)
    img_end = e1.save_checkpoint()
    e2 = _engine(shape, run, lock, W, pr)
    e2.load_checkpoint(img0)
    got = _run_to_end(e2, 0, run.steps)
    for i, ((rm, ru), (gm, gu)) in enumerate(zip(ref, got)):
        _assert_same(rm, gm, f"step {i}")
        _assert_same(ru, gu, f"step {i}")
    e3 = _engine(shape, run, lock, W, pr)
    e3.load_checkpoint(img_end)
    with pytest.raises(L.DlmError) as ei:
        e3.step()  # every step was taken
    assert ei.value.status == L.DLM_E_STATE
    for e in (e1, e2, e3):
        e.close()


def test_checkpoint_refusals():
    shape, run = synth.CONFIGS["tiny"]
    lock = synth.LOCK_SETTINGS["natural"]
    W = synth.gen_weights(shape)
    pr = synth.gen_prompts(shape, run)
    e1 = _engine(shape, run, lock, W, pr)
    e1.step()
    with pytest.raises(L.DlmError) as ei:  # a step pending its lock update
        e1.save_checkpoint()
    assert ei.value.status == L.DLM_E_STATE
    e1.lock_update()
    img = e1.save_checkpoint()
    with pytest.raises(L.DlmError) as ei:
        e1.save_checkpoint(np.empty(img.nbytes - 1, dtype=np.uint8))
    assert ei.value.status == L.DLM_E_SIZE
    with pytest.raises(L.DlmError) as ei:
        e1.load_checkpoint(img[:-1].copy())
    assert ei.value.status == L.DLM_E_SIZE
    bad = img.copy()
    bad[0] ^= 0xFF  # magic
    with pytest.raises(L.DlmError) as ei:
        e1.load_checkpoint(bad)
    assert ei.value.status == L.DLM_E_INVALID
    # a handle whose run descriptor differs (another KL threshold)
    other = _engine(shape, run, dict(lock, kl_eps=2e-3), W, pr)
    assert other.checkpoint_bytes() == img.nbytes
    with pytest.raises(L.DlmError) as ei:
        other.load_checkpoint(img)
    assert ei.value.status == L.DLM_E_INVALID
    # a refused load leaves the handle as it was: it still runs its own course
    tok = other.tokens().clone()
    assert other.step() == run.seq_len and torch.equal(other.tokens(), tok)
    other.lock_update()
    for e in (e1, other):
        e.close()


def test_resume_at_the_llada_shape():
    """Full LLaDA-8B shape (32 layers, d = 4096, V = 126464, N = 512; the image
    holds 259 MB of previous logits and 268 MB of K/V): saved after 3 scheduled
    steps into device memory, resumed in a fresh handle; the next 3 steps
    (M from 381 down, on the fused LM-head statistics path) are bitwise those
    of the uninterrupted run."""
    shape, run = synth.CONFIGS["llada8b"]
    lock = synth.LOCK_SETTINGS["scheduled"]
    dw = E.random_device_weights(shape, seed=0)
    pr = torch.from_numpy(synth.gen_prompts(shape, run)).cuda()
    e1 = E.Engine(shape, dw, run, lock, pr)
    for _ in range(3):
        e1.step()
        e1.lock_update()
    img = torch.empty(e1.checkpoint_bytes(), dtype=torch.uint8, device="cuda")
    assert img.numel() > 500_000_000
    e1.save_checkpoint(img)
    ref = _run_to_end(e1, 3, 6)
    e1.close()
    e2 = E.Engine(shape, dw, run, lock, pr)
    e2.load_checkpoint(img)
    got = _run_to_end(e2, 3, 6)
    for i, ((rm, ru), (gm, gu)) in enumerate(zip(ref, got)):
        _assert_same(rm, gm, f"step {3 + i} (posterior)")
        _assert_same(ru, gu, f"step {3 + i} (update)")
    e2.close()
