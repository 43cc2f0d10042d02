"""Step-level parity: the whole denoising step through the C ABI against the
oracle in lockstep (tokens and lock masks bit-exact after replay of near-tie
decisions; logits within 1e-4 (fp32) or 2e-2 of the logit scale (bf16)),
plus properties checked at the full LLaDA-8B shape."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from selective_token_recompute_amd import engine as E
from tests.harness import bits_to_bool, run_lockstep

pytestmark = pytest.mark.gpu


def _report(name, reps):
    n = len(reps)
    rp = sum(r.replayed for r in reps)
    print(f"\n[{name}] steps={n} replays={rp} ({rp / max(n, 1):.0%}) "
          f"max|dz|={max(r.max_dz for r in reps):.3g} scale={max(r.z_scale for r in reps):.3g} "
          f"M={[r.m for r in reps][:8]}...", flush=True)


@pytest.fixture(scope="module")
def tiny():
    shape, run = synth.CONFIGS["tiny"]
    return shape, run, synth.gen_weights(shape), synth.gen_prompts(shape, run)


@pytest.mark.parametrize("setting", ["natural", "kl_only", "scheduled", "vanilla"])
def test_tiny_fp32_all_steps(tiny, setting):
    shape, run, W, pr = tiny
    reps = run_lockstep(shape, W, run, synth.LOCK_SETTINGS[setting], pr)
    _report(f"tiny/{setting}", reps)
    assert len(reps) == run.steps


def test_tiny_fp32_kl_reverse_direction(tiny):
    shape, run, W, pr = tiny
    lock = dict(synth.LOCK_SETTINGS["kl_only"], kl_dir=1)
    _report("tiny/kl_dir1", run_lockstep(shape, W, run, lock, pr))


MID = synth.ModelShape(2, 512, 4, 4, 128, 1024, 4096, bf16=True)
MID_GQA = synth.ModelShape(2, 512, 8, 2, 128, 1024, 4000, bf16=True)
MID_RUN = synth.RunShape(2, 192, 64, 32, 64)   # two sequences, 2 semi-AR blocks
# Dream-7B's head grouping (7 query heads per K/V head) at small width, three
# sequences of different prompt content, two semi-AR blocks
MID_G7 = synth.ModelShape(2, 896, 7, 1, 128, 2368, 4000, bf16=True)
MID_G7_RUN = synth.RunShape(3, 160, 32, 32, 64)
# the long-context schedule (N=4096, 1024 prompt + 3072 generated in 12
# semi-AR blocks of 256, one step per block) at small width
LONG_SMALL = synth.ModelShape(2, 256, 4, 4, 64, 512, 1000, bf16=True)
LONG_SMALL_RUN = synth.RunShape(1, 4096, 1024, 12, 256)


@pytest.mark.parametrize("shape", [MID, MID_GQA], ids=["mha", "gqa"])
@pytest.mark.parametrize("setting", ["scheduled", "kl_only", "natural"])
def test_mid_bf16_mfma_path(shape, setting):
    W = synth.gen_weights(shape)
    pr = synth.gen_prompts(shape, MID_RUN)
    reps = run_lockstep(shape, W, MID_RUN, synth.LOCK_SETTINGS[setting], pr)
    _report(f"mid-{shape.n_kv_heads}/{setting}", reps)


@pytest.mark.parametrize("setting", ["scheduled", "natural"])
def test_mid_bf16_group7_batched(setting):
    W = synth.gen_weights(MID_G7)
    pr = synth.gen_prompts(MID_G7, MID_G7_RUN)
    reps = run_lockstep(MID_G7, W, MID_G7_RUN, synth.LOCK_SETTINGS[setting], pr)
    _report(f"mid-g7/{setting}", reps)


@pytest.mark.parametrize("setting", ["scheduled"])
def test_long_context_blocks(setting):
    reps = run_lockstep(LONG_SMALL, synth.gen_weights(LONG_SMALL), LONG_SMALL_RUN,
                        synth.LOCK_SETTINGS[setting], synth.gen_prompts(LONG_SMALL, LONG_SMALL_RUN))
    _report(f"long-4096/{setting}", reps)
    assert reps[0].m == LONG_SMALL_RUN.seq_len


def test_tiny_bf16_generic_path():
    shape, run = synth.CONFIGS["tiny"]
    shape = dataclasses.replace(shape, bf16=True)
    W = synth.gen_weights(shape)
    pr = synth.gen_prompts(shape, run)
    _report("tiny-bf16/scheduled", run_lockstep(shape, W, run, synth.LOCK_SETTINGS["scheduled"], pr))


@pytest.mark.parametrize("case", ["tiny-fp32", "mid-bf16", "mid-gqa-bf16"])
def test_poisoned_state_is_never_read(tiny, case):
    """Every array a step writes before it reads starts as NaN
    (dlm_debug_poison); the lockstep against the oracle still holds every
    logit and statistic finite and within tolerance, so no step reads a
    value it did not write (K/V of positions not yet computed, previous
    logits of rows without a previous posterior, workspace, activations)."""
    if case == "tiny-fp32":
        shape, run, W, pr = tiny
        steps = run.steps
    else:
        shape = MID if case == "mid-bf16" else MID_GQA
        run, W, pr = MID_RUN, synth.gen_weights(shape), synth.gen_prompts(shape, MID_RUN)
        steps = 10
    reps = run_lockstep(shape, W, run, synth.LOCK_SETTINGS["scheduled"], pr, steps=steps,
                        poison=True)
    assert len(reps) == steps and all(np.isfinite(r.max_dz) for r in reps)


def test_per_step_metrics_record(tiny, tmp_path):
    """The engine's per-step JSON-lines record against the oracle's own
    trajectory: active rows, unmasked count, new locks, FLOPs."""
    import json
    shape, run, W, pr = tiny
    lock = synth.LOCK_SETTINGS["scheduled"]
    dev = torch.device("cuda")
    path = str(tmp_path / "metrics.jsonl")
    eng = E.Engine(shape, E.upload_weights(W, shape, dev), run, lock,
                   torch.from_numpy(pr).to(dev), metrics_path=path)
    orc = oracle.Oracle(shape, W, run, lock, pr)
    want = []
    for t in range(run.steps):
        eng.step()
        orc.step()
        before = orc.locked().copy()
        orc.lock_update()
        eng.lock_update()
        want.append(dict(m=orc.m, commits=len(orc.commits()[0]),
                         new=int((orc.locked() & ~before).sum()), locked=int(orc.locked().sum())))
    eng.close()
    got = [json.loads(line) for line in open(path)]
    assert [g["t"] for g in got] == list(range(run.steps))
    for g, w in zip(got, want):
        assert g["m_tot"] == w["m"] == sum(g["m_b"])
        assert g["commits"] == w["commits"]
        assert g["new_locks"] == w["new"] and g["locked"] == w["locked"]
        assert g["flops"] == pytest.approx(oracle.closed_form_flops(shape, [w["m"]], run.seq_len))


def test_same_run_twice_is_bitwise_identical(llada_weights):
    """Determinism: two engines on the same LLaDA-8B-shaped run (full width,
    32 layers, scheduled locking, the first 6 steps: M = 512, 384, ...) give
    bitwise identical logits, statistics, tokens, lock bits and counters at
    every step (every reduction runs in a fixed order)."""
    shape, run = synth.CONFIGS["llada8b"]
    lock = synth.LOCK_SETTINGS["scheduled"]
    pr = torch.from_numpy(synth.gen_prompts(shape, run)).cuda()
    e1 = E.Engine(shape, llada_weights, run, lock, pr)
    e2 = E.Engine(shape, llada_weights, run, lock, pr)
    for t in range(6):
        m1, m2 = e1.step(), e2.step()
        assert m1 == m2
        rs, rp = (a[:m1].long() for a in e1.rows()[:2])
        assert torch.equal(e1.logits()[rs, rp].view(torch.int32),
                           e2.logits()[rs, rp].view(torch.int32)), f"step {t}: logits"
        s1, s2 = e1.stats(), e2.stats()
        for k in s1:
            assert torch.equal(s1[k][:m1].view(torch.int32), s2[k][:m1].view(torch.int32)), k
        e1.lock_update()
        e2.lock_update()
        assert torch.equal(e1.tokens(), e2.tokens()) and torch.equal(e1.lock_bits(), e2.lock_bits())
        assert torch.equal(e1.counters(), e2.counters())
        kc1, vc1 = e1.kv_cache()
        kc2, vc2 = e2.kv_cache()
        assert torch.equal(kc1.view(torch.int16), kc2.view(torch.int16))
        assert torch.equal(vc1.view(torch.int16), vc2.view(torch.int16))
    e1.close()
    e2.close()


def test_poison_only_before_the_first_step(tiny):
    shape, run, W, pr = tiny
    dev = torch.device("cuda")
    eng = E.Engine(shape, E.upload_weights(W, shape, dev), run, synth.LOCK_SETTINGS["natural"],
                   torch.from_numpy(pr).to(dev))
    eng.debug_poison()
    eng.step()
    from selective_token_recompute_amd._lib import DLM_E_STATE, DlmError
    with pytest.raises(DlmError) as ei:
        eng.debug_poison()
    assert ei.value.status == DLM_E_STATE
    eng.close()


def test_empty_active_set_and_forced_locks(tiny):
    """Every row force-locked: the next step has M = 0 and is a no-op."""
    shape, run, W, pr = tiny
    dev = torch.device("cuda")
    eng = E.Engine(shape, E.upload_weights(W, shape, dev), run, synth.LOCK_SETTINGS["natural"],
                   torch.from_numpy(pr).to(dev))
    assert eng.step() == run.seq_len
    bits = np.full((1, 1), np.uint64(0xFFFFFFFF), dtype=np.uint64)
    eng.lock_update(commits=([], [], []), lock_bits=bits)
    tok_before = eng.tokens().cpu().numpy().copy()
    assert eng.step() == 0
    _, m, flops = eng.last_step_info()
    assert m == 0 and flops == 0.0
    eng.lock_update()
    assert np.array_equal(eng.tokens().cpu().numpy(), tok_before)
    eng.close()


def test_nan_weight_is_latched_and_reported(tiny):
    """A NaN in the LM head makes the log-normaliser non-finite; the device
    latches it, the lock update commits and locks nothing from that step, and
    the next dlm_step returns DLM_E_NUMERIC."""
    shape, run, W, pr = tiny
    dev = torch.device("cuda")
    dw = E.upload_weights(W, shape, dev)
    dw["lm_head"][3, 5] = float("nan")
    eng = E.Engine(shape, dw, run, synth.LOCK_SETTINGS["scheduled"],
                   torch.from_numpy(pr).to(dev))
    eng.step()
    tok0 = eng.tokens().cpu().numpy().copy()
    bits0 = eng.lock_bits().cpu().numpy().copy()
    cnt0 = eng.counters().cpu().numpy().copy()
    eng.lock_update()
    torch.cuda.synchronize()
    assert np.array_equal(eng.tokens().cpu().numpy(), tok0)
    assert np.array_equal(eng.lock_bits().cpu().numpy(), bits0)
    assert np.array_equal(eng.counters().cpu().numpy(), cnt0)
    from selective_token_recompute_amd._lib import DLM_E_NUMERIC, DlmError
    with pytest.raises(DlmError) as ei:
        eng.step()
    assert ei.value.status == DLM_E_NUMERIC
    eng.close()


# --- full LLaDA-8B shape: properties that hold at any size ------------------------

@pytest.fixture(scope="module")
def llada_weights():
    shape, _ = synth.CONFIGS["llada8b"]
    return E.random_device_weights(shape, seed=0)


@pytest.mark.parametrize("setting", ["scheduled", "natural"])
def test_llada_full_run_invariants(llada_weights, setting):
    shape, run = synth.CONFIGS["llada8b"]
    lock = synth.LOCK_SETTINGS[setting]
    pr = torch.from_numpy(synth.gen_prompts(shape, run)).cuda()
    eng = E.Engine(shape, llada_weights, run, lock, pr)
    ks = [oracle.unit_schedule(run, t)["k"] for t in range(run.steps)]
    G = run.seq_len - run.prompt_len
    prev_bits = np.zeros((1, run.seq_len), np.uint8)
    prev_tok = eng.tokens().cpu().numpy().copy()
    ms, total_flops = [], 0.0
    for t in range(run.steps):
        m = eng.step()
        ms.append(m)
        _, _, fl = eng.last_step_info()
        cf = oracle.closed_form_flops(shape, [m], run.seq_len)
        assert abs(fl - cf) <= 1e-9 * cf
        total_flops += fl
        st = eng.stats()
        assert torch.isfinite(st["lse"]).all()
        eng.lock_update()
        tok = eng.tokens().cpu().numpy()
        bits = bits_to_bool(eng.lock_bits().cpu().numpy().view(np.uint64), run.seq_len)
        assert (bits >= prev_bits).all()
        assert np.array_equal(tok[prev_bits == 1], prev_tok[prev_bits == 1])
        dec = prev_tok != shape.mask_id
        assert np.array_equal(tok[dec], prev_tok[dec])
        assert not (bits.astype(bool) & (tok == shape.mask_id)).any()
        assert (prev_tok == shape.mask_id).sum() - (tok == shape.mask_id).sum() == ks[t]
        prev_bits, prev_tok = bits, tok.copy()
    assert (prev_tok != shape.mask_id).all()
    assert all(a >= b for a, b in zip(ms, ms[1:]))
    if setting == "scheduled":
        expect = [run.seq_len] + [G - sum(ks[: max(0, t - 2)]) for t in range(1, run.steps)]
        assert ms == expect
    else:
        # random-init posteriors never pass the 0.9 confidence gate: only the prompt locks
        assert ms == [run.seq_len] + [G] * (run.steps - 1)
    eng.close()
    print(f"\n[llada8b/{setting}] mean M={np.mean(ms):.1f} total TFLOP={total_flops / 1e12:.2f}")


def test_override_path_matches_oracle(tiny):
    """dlm_lock_update with overrides: given commits replace the top-k choice,
    given lock bits (and counters) replace the lock test, on both sides."""
    from tests.harness import bool_to_bits
    shape, run, W, pr = tiny
    lock = synth.LOCK_SETTINGS["natural"]  # the gate never passes: no rule-side near ties
    dev = torch.device("cuda")
    eng = E.Engine(shape, E.upload_weights(W, shape, dev), run, lock, torch.from_numpy(pr).to(dev))
    orc = oracle.Oracle(shape, W, run, lock, pr)
    rng = np.random.default_rng(21)
    N = run.seq_len
    for t in range(run.steps):
        eng.step()
        orc.step()
        x = orc.tokens()
        masked = np.nonzero(x[0] == shape.mask_id)[0]
        pick = rng.choice(masked, size=min(len(masked), int(rng.integers(0, 3))), replace=False)
        commits = (np.zeros(len(pick), np.int32), pick.astype(np.int32),
                   rng.integers(0, shape.vocab - 1, len(pick)).astype(np.int32))
        if t % 2 == 0:
            decoded = (x != shape.mask_id) & (rng.random(x.shape) < 0.2)
            cnt = rng.integers(0, 3, x.shape).astype(np.int32)
            orc.lock_update(commits=commits, locked=decoded.astype(np.uint8), cnt=cnt)
            eng.lock_update(commits=commits, lock_bits=bool_to_bits(decoded.astype(np.uint8)),
                            counters=cnt)
        else:
            orc.lock_update(commits=commits)
            eng.lock_update(commits=commits)
        torch.cuda.synchronize()
        assert np.array_equal(eng.tokens().cpu().numpy(), orc.tokens())
        lk = eng.lock_bits().cpu().numpy().view(np.uint64)
        assert np.array_equal(lk, bool_to_bits(orc.locked()))
        assert np.array_equal(eng.counters().cpu().numpy(), orc.counters())
    eng.close()


@pytest.mark.parametrize("shape", [MID, MID_GQA], ids=["mha", "gqa"])
def test_kv_cache_matches_oracle(shape):
    """The per-layer K cache and the transposed V cache written by the fused
    QKV epilogue (M >= 96) and by the unfused rotary/scatter path (small M)
    equal the oracle's caches within bf16 rounding."""
    run = MID_RUN
    W = synth.gen_weights(shape)
    pr = synth.gen_prompts(shape, run)
    dev = torch.device("cuda")
    lock = synth.LOCK_SETTINGS["scheduled"]
    eng = E.Engine(shape, E.upload_weights(W, shape, dev), run, lock, torch.from_numpy(pr).to(dev))
    orc = oracle.Oracle(shape, W, run, lock, pr)
    ms = []
    for t in range(run.steps):
        ms.append(eng.step())
        orc.step()
        if t in (0, run.steps - 1):
            kg, vg = eng.kv_cache()
            for layer in range(shape.n_layers):
                ko, vo = orc.kv(layer)
                kgl = kg[layer].float().cpu().numpy()
                vgl = vg[layer].float().cpu().numpy().transpose(0, 1, 3, 2)
                for got, want in ((kgl, ko), (vgl, vo)):
                    err = np.abs(got - want)
                    scale = float(np.abs(want).max())
                    # layer 0 sees identical inputs: one bf16 rounding apart; deeper
                    # layers inherit fp32-vs-fp64 differences, so a 1% scale bar
                    tol = (2.0 ** -7 * np.abs(want) + 1e-3 * scale) if layer == 0 else \
                        1e-2 * scale
                    assert (err <= tol).all(), (t, layer, err.max(), scale)
        orc.lock_update()
        # follow the oracle's decisions so both caches see the same inputs
        from tests.harness import bool_to_bits
        cs, cp, ct = orc.commits()
        eng.lock_update(commits=(cs, cp, ct), lock_bits=bool_to_bits(orc.locked()),
                        counters=orc.counters())
    assert max(ms) >= 96 and min(ms) < 96  # both QKV paths ran
    eng.close()
