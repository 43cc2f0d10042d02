"""Pins of the CPU oracle against what the pages and mathematics fix.

Pages: the SureLock explainer ("Stopping Computation for Converged Tokens in
Masked Diffusion-LM Decoding") and the SlowFast explainer ("Accelerating
Diffusion LLMs with SlowFast Sampling").  Each test names the fact it pins.
"""
import dataclasses
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import synth
from oracle import naive

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _run_oracle(shape, W, run, lock, prompts, overrides=None):
    o = oracle.Oracle(shape, W, run, lock, prompts)
    trace = []
    for t in range(run.steps):
        x_in = o.tokens()
        locked_in = o.locked()
        o.step()
        rows = o.rows()
        z = o.logits()[1]
        st = o.stats()
        m, fl = o.m, o.flops
        if overrides and t in overrides:
            o.lock_update(**overrides[t])
        else:
            o.lock_update()
        trace.append(dict(t=t, x_in=x_in, locked_in=locked_in, rows=rows, logits=z, stats=st,
                          m=m, flops=fl, x_out=o.tokens(), locked_out=o.locked(),
                          commits=o.commits()))
    return trace


@pytest.fixture(scope="module")
def tiny():
    shape, run = synth.CONFIGS["tiny"]
    return shape, run, synth.gen_weights(shape), synth.gen_prompts(shape, run)


def _finite_diff(a, b):
    a = np.where(np.isinf(a), 0.0, a)
    b = np.where(np.isinf(b), 0.0, b)
    return float(np.abs(a - b).max())


# --- P1: locking off is exactly vanilla full recompute (SureLock §1) ---------

def test_p1_lock_off_equals_full_recompute(tiny):
    shape, run, W, pr = tiny
    ref = naive.generate(shape, W, run, pr)
    tr = _run_oracle(shape, W, run, synth.LOCK_SETTINGS["vanilla"], pr)
    for t, st in enumerate(tr):
        assert st["m"] == run.seq_len
        assert _finite_diff(st["logits"], ref["logits"][t][0]) <= 1e-10
        assert np.array_equal(st["x_out"], ref["tokens"][t])
        assert np.isinf(st["logits"][:, shape.mask_id]).all()


def test_p1_negative_eps_equals_policy_none(tiny):
    shape, run, W, pr = tiny
    none = _run_oracle(shape, W, run, synth.LOCK_SETTINGS["vanilla"], pr)
    lk = dict(policy="test", kl_eps=-1.0, conf_tau=0.0, n_consec=1,
              lock_prompt_after_first_step=0)
    test = _run_oracle(shape, W, run, lk, pr)
    for a, b in zip(none, test):
        assert np.array_equal(a["logits"], b["logits"])
        assert np.array_equal(a["x_out"], b["x_out"])
        assert not b["locked_out"].any()


def test_p1_bf16_storage_lock_off_matches_naive():
    shape, run = synth.CONFIGS["tiny"]
    shape = dataclasses.replace(shape, bf16=True)
    run = dataclasses.replace(run, steps=4)
    W = synth.gen_weights(shape)
    pr = synth.gen_prompts(shape, run)
    ref = naive.generate(shape, W, run, pr)
    tr = _run_oracle(shape, W, run, synth.LOCK_SETTINGS["vanilla"], pr)
    for t, st in enumerate(tr):
        # same rounding points on both sides; only fp64 summation order differs,
        # which can move a value across a bf16 rounding boundary
        assert _finite_diff(st["logits"], ref["logits"][t][0]) <= 2e-3
        assert np.array_equal(st["x_out"], ref["tokens"][t])


# --- P8: brute force on a tiny model, three implementations -----------------

def test_p8_brute_force_three_ways():
    shape = synth.ModelShape(2, 8, 2, 1, 4, 12, 16, bf16=False)
    run = synth.RunShape(1, 8, 2, 4, 6)
    W = synth.gen_weights(shape)
    pr = synth.gen_prompts(shape, run)
    loops = naive.generate_loops(shape, W, run, pr)
    vec = naive.generate(shape, W, run, pr)
    tr = _run_oracle(shape, W, run, synth.LOCK_SETTINGS["vanilla"], pr)
    for t in range(run.steps):
        assert _finite_diff(loops["logits"][t][0], vec["logits"][t][0]) <= 1e-12
        assert _finite_diff(tr[t]["logits"], loops["logits"][t][0]) <= 1e-12
        assert np.array_equal(loops["tokens"][t], tr[t]["x_out"])
        assert np.array_equal(vec["tokens"][t], tr[t]["x_out"])


# --- P2: fresh cached K/V give exactly the full-recompute rows ---------------

def test_p2_locked_rows_with_fresh_cache_equal_full_recompute():
    """SureLock §2 continued attention: active queries attend to every position
    through the cache.  When no token changed since the cache was written, the
    cached K/V equal fresh ones, so the active rows must equal the matching
    rows of a full recompute."""
    shape = synth.ModelShape(2, 32, 4, 2, 8, 48, 64, bf16=False)
    run = synth.RunShape(1, 16, 4, 12, 12)  # G=12, T=12 -> k=1 each step
    run = dataclasses.replace(run, prompt_len=12, block_len=4)  # G=4 over 12 steps
    assert oracle.unit_schedule(run, 0)["k"] == 0 and oracle.unit_schedule(run, 1)["k"] == 0
    W = synth.gen_weights(shape)
    pr = synth.gen_prompts(shape, run)
    lock = synth.LOCK_SETTINGS["vanilla"]
    o = oracle.Oracle(shape, W, run, dict(lock, policy="test", kl_eps=-1.0), pr)
    o.step()
    _, z0 = o.logits()
    rng = np.random.default_rng(5)
    lk = np.zeros((1, run.seq_len), np.uint8)
    lk[0, rng.choice(run.seq_len, 7, replace=False)] = 1
    o.lock_update(locked=lk)  # k_0 = 0: tokens unchanged
    o.step()
    seq, pos, _ = o.rows()
    assert len(pos) == run.seq_len - 7
    _, z1 = o.logits()
    full = naive.forward_full(shape, W, o.tokens()[0])
    assert _finite_diff(z1, full[pos]) <= 1e-12
    assert _finite_diff(z0, full) <= 1e-12


def test_p2_compacted_attention_rows_equal_dense():
    rng = np.random.default_rng(7)
    N, nq, nkv, hd = 24, 4, 2, 8
    q = rng.standard_normal((N, nq, hd))
    k = rng.standard_normal((1, nkv, N, hd))
    v = rng.standard_normal((1, nkv, N, hd))
    # dense attention of every position (library softmax)
    dense = np.empty_like(q)
    for h in range(nq):
        g = h // (nq // nkv)
        s = q[:, h, :] @ k[0, g].T / math.sqrt(hd)
        dense[:, h, :] = scipy.special.softmax(s, axis=1) @ v[0, g]
    A = np.sort(rng.choice(N, 9, replace=False))
    o = oracle.unit_attention(q[A], np.zeros(len(A), np.int32), k, v)
    assert np.abs(o - dense[A]).max() <= 1e-12


# --- P3: invariants of the lock state (SureLock §2 permanent deactivation) --

def _check_invariants(shape, run, trace):
    prev_m = None
    for st in trace:
        lin, lout = st["locked_in"], st["locked_out"]
        assert (lout >= lin).all(), "a lock was released"
        if prev_m is not None:
            assert st["m"] <= prev_m, "active set grew"
        prev_m = st["m"]
        xin, xout = st["x_in"], st["x_out"]
        assert np.array_equal(xin[lin == 1], xout[lin == 1]), "locked token changed"
        dec = xin != shape.mask_id
        assert np.array_equal(xin[dec], xout[dec]), "decoded token reverted"
        assert not (lout.astype(bool) & (xout == shape.mask_id)).any(), "masked position locked"
        sch = oracle.unit_schedule(run, st["t"])
        for b in range(run.batch):
            cand = int(((xin[b] == shape.mask_id) &
                        (np.arange(run.seq_len) >= sch["lo"]) &
                        (np.arange(run.seq_len) < sch["hi"])).sum())
            dropped = int((xin[b] == shape.mask_id).sum() - (xout[b] == shape.mask_id).sum())
            assert dropped == min(sch["k"], cand)


@pytest.mark.parametrize("setting", ["natural", "kl_only", "scheduled", "vanilla"])
def test_p3_invariants(tiny, setting):
    shape, run, W, pr = tiny
    tr = _run_oracle(shape, W, run, synth.LOCK_SETTINGS[setting], pr)
    _check_invariants(shape, run, tr)
    assert (tr[-1]["x_out"] != shape.mask_id).all(), "all masks decoded after T steps"


def test_p3_invariants_random_lock_overrides(tiny):
    shape, run, W, pr = tiny
    rng = np.random.default_rng(11)
    ov = {}
    for t in range(run.steps):
        lk = (rng.random((1, run.seq_len)) < 0.08).astype(np.uint8)
        lk[0, run.prompt_len:] = 0  # force-lock only prompt positions
        ov[t] = dict(locked=lk)
    tr = _run_oracle(shape, W, run, synth.LOCK_SETTINGS["kl_only"], pr, overrides=ov)
    _check_invariants(shape, run, tr)


# --- P4: FLOP count equals the closed form (SureLock §2 complexity) ---------

def test_p4_flops_closed_form_and_scheduled_trace(tiny):
    shape, run, W, pr = tiny
    tr = _run_oracle(shape, W, run, synth.LOCK_SETTINGS["scheduled"], pr)
    ks = [oracle.unit_schedule(run, t)["k"] for t in range(run.steps)]
    G = run.seq_len - run.prompt_len
    for st in tr:
        t = st["t"]
        assert st["flops"] == pytest.approx(
            oracle.closed_form_flops(shape, [st["m"]], run.seq_len), rel=1e-12)
        # scheduled locking: a position decoded at step s locks at the end of
        # step s+2; the prompt locks after step 0
        expect = run.seq_len if t == 0 else G - sum(ks[: max(0, t - 2)])
        assert st["m"] == expect
    ms = [st["m"] for st in tr]
    assert ms[:6] == [32, 24, 24, 23, 21, 20]
    # MHA closed form 2L(M(4d^2 + 3 d dff) + 2MNd) + 2MdV
    d, dff, L, N, V = shape.d_model, shape.d_ff, shape.n_layers, run.seq_len, shape.vocab
    M = 17
    assert oracle.closed_form_flops(shape, [M], N) == 2 * L * (M * (4 * d * d + 3 * d * dff)
                                                              + 2 * M * N * d) + 2 * M * d * V


def test_p4_llada_scheduled_saving():
    shape, run = synth.CONFIGS["llada8b"]
    ks = [oracle.unit_schedule(run, t)["k"] for t in range(run.steps)]
    assert set(ks) == {3}
    G = run.seq_len - run.prompt_len
    ms = [run.seq_len] + [G - sum(ks[: max(0, t - 2)]) for t in range(1, run.steps)]
    assert ms[:4] == [512, 384, 384, 381] and ms[-1] == 9
    f_lock = sum(oracle.closed_form_flops(shape, [m], run.seq_len) for m in ms)
    f_van = run.steps * oracle.closed_form_flops(shape, [run.seq_len], run.seq_len)
    assert 1 - f_lock / f_van == pytest.approx(0.609, abs=0.002)


# --- schedule (SlowFast §1: semi-autoregressive blocks; top-k per step) -----

def test_schedule_tables():
    shape, run = synth.CONFIGS["tiny"]
    ks = [oracle.unit_schedule(run, t)["k"] for t in range(run.steps)]
    assert ks == [1, 2] * 8 and sum(ks) == 24
    _, run5 = synth.CONFIGS["longctx"]
    per_block = {}
    steps = {}
    for t in range(run5.steps):
        s = oracle.unit_schedule(run5, t)
        per_block[s["beta"]] = per_block.get(s["beta"], 0) + s["k"]
        steps[s["beta"]] = steps.get(s["beta"], 0) + 1
        assert s["hi"] - s["lo"] == 256 and s["lo"] == 1024 + 256 * s["beta"]
    assert len(per_block) == 12 and set(per_block.values()) == {256}
    assert set(steps.values()) == {42, 43} and sum(steps.values()) == 512
    assert oracle.unit_schedule(run5, run5.steps)["beta"] == -1


# --- golden hand-derived transitions ----------------------------------------

def _golden_cases():
    with open(os.path.join(GOLD, "lock_transition_cases.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_lock_transition_golden(case):
    shape = synth.ModelShape(1, 8, 1, 1, 8, 8, case["vocab"], bf16=False)
    run = synth.RunShape(case["batch"], case["seq_len"], case["prompt_len"], case["steps"],
                         case["block_len"])
    lock = {k: case[k] for k in ("policy", "kl_eps", "conf_tau", "n_consec",
                                 "lock_prompt_after_first_step")}
    x0 = np.array(case["x"], np.int32)
    real = np.array([x0[s, p] != shape.mask_id for s, p in zip(case["row_seq"],
                                                                 case["row_pos"])], np.uint8)
    x, locked, cnt = oracle.unit_lock_transition(
        shape, run, lock, case["t"], case["row_seq"], case["row_pos"], real, case["argmax"],
        case["conf"], case["kl"], case["has_kl"], x0, case["locked"], case["cnt"])
    assert x.tolist() == case["expect_x"]
    assert locked.tolist() == case["expect_locked"]
    assert cnt.tolist() == case["expect_cnt"]


# --- P5: softmax / KL / argmax closed forms (SureLock §2 locking condition) -

def test_p5_vocab_stats_closed_forms():
    rng = np.random.default_rng(3)
    V = 50
    mask = V - 1
    z = rng.standard_normal((6, V)) * 3
    z[:, mask] = -np.inf
    st = oracle.unit_vocab_stats(z, mask_id=mask)
    zz = z[:, :mask]
    assert np.allclose(st["lse"], scipy.special.logsumexp(zz, axis=1), atol=1e-13)
    assert np.array_equal(st["argmax"], zz.argmax(axis=1))
    assert np.allclose(st["conf"], scipy.special.softmax(zz, axis=1).max(axis=1), atol=1e-14)
    # KL(p||p) = 0
    st2 = oracle.unit_vocab_stats(z, prev=st["logp"], mask_id=mask)
    assert np.abs(st2["kl"]).max() <= 1e-13
    # KL(p || uniform over V-1) = log(V-1) - H(p)
    uni = np.full((6, V), -math.log(V - 1))
    uni[:, mask] = -np.inf
    st3 = oracle.unit_vocab_stats(z, prev=uni, mask_id=mask)
    p = scipy.special.softmax(zz, axis=1)
    H = -(p * np.log(p)).sum(axis=1)
    assert np.allclose(st3["kl"], math.log(V - 1) - H, atol=1e-12)
    # against the library relative entropy, both directions
    z2 = rng.standard_normal((6, V)) * 2
    z2[:, mask] = -np.inf
    q_log = oracle.unit_vocab_stats(z2, mask_id=mask)["logp"]
    q = scipy.special.softmax(z2[:, :mask], axis=1)
    fwd = oracle.unit_vocab_stats(z, prev=q_log, mask_id=mask, kl_dir=0)["kl"]
    bwd = oracle.unit_vocab_stats(z, prev=q_log, mask_id=mask, kl_dir=1)["kl"]
    assert np.allclose(fwd, scipy.special.rel_entr(p, q).sum(axis=1), atol=1e-12)
    assert np.allclose(bwd, scipy.special.rel_entr(q, p).sum(axis=1), atol=1e-12)
    # no previous posterior -> KL undefined
    assert np.isnan(st["kl"]).all()


def test_p5_special_logits():
    V = 40
    mask = V - 1
    const = np.zeros((1, V))
    const[0, mask] = -np.inf
    st = oracle.unit_vocab_stats(const, mask_id=mask)
    assert st["argmax"][0] == 0 and st["conf"][0] == pytest.approx(1 / (V - 1), rel=1e-14)
    dom = np.zeros((1, V))
    dom[0, 7] = 50.0
    dom[0, mask] = 1e9  # the mask column never counts, whatever its value
    st = oracle.unit_vocab_stats(dom, mask_id=mask)
    assert st["argmax"][0] == 7
    assert st["conf"][0] == pytest.approx(1 / (1 + (V - 2) * math.exp(-50)), rel=1e-15)
    tie = np.zeros((1, V))
    tie[0, [5, 9, 30]] = 2.0
    assert oracle.unit_vocab_stats(tie, mask_id=mask)["argmax"][0] == 5


# --- P6: attention special cases --------------------------------------------

def test_p6_attention_special_cases():
    rng = np.random.default_rng(9)
    hd, N = 8, 10
    q = rng.standard_normal((3, 2, hd))
    kk = np.tile(rng.standard_normal(hd), (1, 1, N, 1))
    v = rng.standard_normal((1, 1, N, hd))
    o = oracle.unit_attention(q, np.zeros(3, np.int32), kk, v)
    assert np.allclose(o, v[0, 0].mean(axis=0), atol=1e-14)  # equal keys -> mean of V
    o1 = oracle.unit_attention(q, np.zeros(3, np.int32), kk[:, :, :1], v[:, :, :1])
    assert np.allclose(o1, v[0, 0, 0], atol=1e-15)  # one key -> its value
    k = rng.standard_normal((1, 1, N, hd))
    k[0, 0, 4] = q[0, 0] * 1e3  # one dominant score for head 0 of row 0
    o2 = oracle.unit_attention(q[:1, :1], np.zeros(1, np.int32), k, v)
    assert np.allclose(o2[0, 0], v[0, 0, 4], atol=1e-12)
    perm = rng.permutation(N)
    a = oracle.unit_attention(q, np.zeros(3, np.int32), k, v)
    b = oracle.unit_attention(q, np.zeros(3, np.int32), k[:, :, perm], v[:, :, perm])
    assert np.allclose(a, b, atol=1e-13)
    # batch rows attend only to their own sequence's cache
    k2 = rng.standard_normal((2, 1, N, hd))
    v2 = rng.standard_normal((2, 1, N, hd))
    o3 = oracle.unit_attention(q, np.array([1, 0, 1], np.int32), k2, v2)
    o4 = oracle.unit_attention(q[[0, 2]], np.zeros(2, np.int32), k2[1:], v2[1:])
    assert np.array_equal(o3[[0, 2]], o4)


# --- P7: RMSNorm and RoPE ----------------------------------------------------

def test_p7_rmsnorm_and_rope():
    rng = np.random.default_rng(13)
    d = 16
    g = rng.standard_normal(d).astype(np.float32)
    c = 3.0
    y = oracle.unit_rmsnorm(np.full((1, d), c), g, 1e-5)
    assert np.allclose(y[0], g.astype(np.float64) * c / math.sqrt(c * c + 1e-5), atol=1e-15)
    x = rng.standard_normal((4, d))
    y = oracle.unit_rmsnorm(x, np.ones(d, np.float32), 0.0)
    assert np.allclose(np.mean(y * y, axis=1), 1.0, atol=1e-13)
    hd = 16
    u = rng.standard_normal((5, 3, hd))
    assert np.array_equal(oracle.unit_rope(u, np.zeros(5, np.int32), 10000.0), u)
    pos = np.array([0, 3, 17, 100, 511], np.int32)
    r = oracle.unit_rope(u, pos, 10000.0)
    assert np.allclose(np.linalg.norm(r, axis=2), np.linalg.norm(u, axis=2), atol=1e-12)
    # rotation by pos*theta_j of pair (j, j + hd/2): a plain 2x2 rotation check
    j, p = 3, 17
    ang = p * 10000.0 ** (-2.0 * j / hd)
    a0, a1 = u[2, 1, j], u[2, 1, j + hd // 2]
    assert r[2, 1, j] == pytest.approx(a0 * math.cos(ang) - a1 * math.sin(ang), abs=1e-14)
    assert r[2, 1, j + hd // 2] == pytest.approx(a0 * math.sin(ang) + a1 * math.cos(ang), abs=1e-14)
    # relative position: <R_m q, R_n k> depends only on m - n
    q = rng.standard_normal((1, 1, hd))
    k = rng.standard_normal((1, 1, hd))
    dots = []
    for m_, n_ in [(5, 2), (105, 102), (40, 37)]:
        rq = oracle.unit_rope(q, np.array([m_], np.int32), 10000.0)
        rk = oracle.unit_rope(k, np.array([n_], np.int32), 10000.0)
        dots.append(float((rq * rk).sum()))
    assert np.allclose(dots, dots[0], atol=1e-12)


# --- the remaining primitives -------------------------------------------------

def test_bf16_rounding_matches_library():
    rng = np.random.default_rng(17)
    x = (rng.standard_normal(2000) * 10.0 ** rng.integers(-6, 6, 2000)).astype(np.float32)
    lib = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    ours = np.array([oracle.bf16_round(float(v)) for v in x])
    assert np.array_equal(ours, lib)
    assert oracle.bf16_round(1.0 + 2.0 ** -8) == 1.0  # tie -> even
    assert oracle.bf16_round(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    assert np.array_equal(naive._bf16(x.astype(np.float64)), lib)


def test_linear_and_compact_primitives():
    rng = np.random.default_rng(19)
    x = rng.standard_normal((7, 33))
    W = rng.standard_normal((5, 33)).astype(np.float32)
    assert np.allclose(oracle.unit_linear(x, W), x @ W.astype(np.float64).T, atol=1e-12)
    for p in (0.0, 1.0, 0.3, 0.9):
        bits = synth.gen_lock_bits(3, 130, p, seed=int(p * 10))
        seq, pos, mb = oracle.unit_compact(bits, 130)
        dense = np.zeros((3, 130), bool)
        for b in range(3):
            for i in range(130):
                dense[b, i] = (int(bits[b, i // 64]) >> (i % 64)) & 1
        bb, ii = np.nonzero(~dense)
        assert np.array_equal(seq, bb) and np.array_equal(pos, ii)
        assert np.array_equal(mb, (~dense).sum(axis=1))


# --- SlowFast sampler ([SF] §2 two-stage pipeline) ------------------------------
# Hand-worked cycles: each expected commit, span and state below follows from
# the page's description (exploratory top-k in a window while the end point's
# variance is tracked, accelerated in-span threshold commits with a top-k
# fallback, out-of-span positions frozen until the span is decoded).

SF_MASK = 99


def _sf_run(N=16, window=4):
    return synth.RunShape(1, N, 4, 16, window)


def _sf_lock(**kw):
    d = dict(synth.LOCK_SETTINGS["scheduled"], sampler="slowfast", sf_k=1, sf_kmax=8,
             sf_whist=2, sf_tau_conv=0.5, sf_tau_high=0.8, sf_var=1.0)
    d.update(kw)
    return d


def _sf_step(run, lock, x, frozen, hp, st, conf_of):
    """Rows = every non-frozen position (ascending); argmax of position p is
    1000 + p; conf from conf_of (default 0.1)."""
    pos = np.array([p for p in range(len(x)) if not frozen[p]], np.int32)
    conf = np.array([conf_of.get(int(p), 0.1) for p in pos])
    (cp, ct), x, frozen, hp, st = oracle.unit_slowfast(run, lock, SF_MASK, pos, 1000 + pos, conf,
                                                       x, frozen, hp, st)
    assert np.array_equal(ct, 1000 + cp)
    return sorted(cp.tolist()), x, frozen, hp, st


def test_slowfast_cycle_hand_worked():
    run, lock = _sf_run(), _sf_lock()
    x = np.array([1, 2, 3, 4] + [SF_MASK] * 12, np.int32)
    frozen = np.zeros(16, np.uint8)
    hp = np.ones(16, np.uint8)
    st = np.zeros(13, np.int32)
    # exploratory: frontier 4, end point 8 (positions 5 and 8 reach 0.5), one
    # end point recorded; top-1 of the window [4, 8) is position 5
    c, x, frozen, hp, st = _sf_step(run, lock, x, frozen, hp, st,
                                    {4: 0.3, 5: 0.6, 6: 0.2, 8: 0.55})
    assert c == [5] and list(st[:5]) == [0, 0, 0, 1, 1] and st[5] == 8
    # end point 9: variance of (8, 9) = 0.25 < 1 -> span [4, 10); position 4
    # alone is above 0.8 and k = 1 -> it commits; 10..15 freeze
    c, x, frozen, hp, st = _sf_step(run, lock, x, frozen, hp, st, {4: 0.85, 9: 0.7})
    assert c == [4] and list(st[:5]) == [1, 4, 10, 2, 2] and list(st[5:7]) == [8, 9]
    assert frozen.tolist() == [0] * 10 + [1] * 6
    # accelerated: 6 and 7 above 0.8 both commit; 8, 9 left
    c, x, frozen, hp, st = _sf_step(run, lock, x, frozen, hp, st,
                                    {6: 0.9, 7: 0.95, 8: 0.3, 9: 0.1})
    assert c == [6, 7] and st[0] == 1
    # none above 0.8: top-1 fallback (position 9, 0.45)
    c, x, frozen, hp, st = _sf_step(run, lock, x, frozen, hp, st, {8: 0.4, 9: 0.45})
    assert c == [9] and st[0] == 1 and frozen[10:].all()
    # last in-span mask: the cycle ends, the frozen positions return without a
    # previous posterior, the state resets
    c, x, frozen, hp, st = _sf_step(run, lock, x, frozen, hp, st, {8: 0.2})
    assert c == [8] and not st.any() and not frozen.any()
    assert hp.tolist() == [1] * 10 + [0] * 6
    # a new cycle from frontier 10: nothing reaches 0.5 -> no end point
    # recorded; top-1 of [10, 14) is 12
    c, x, frozen, hp, st = _sf_step(run, lock, x, frozen, hp, st, {12: 0.45, 15: 0.49})
    assert c == [12] and list(st[:5]) == [0, 0, 0, 1, 0]
    assert (x[:10] != SF_MASK).all() and x[12] == 1012


def test_slowfast_kmax_and_empty_span():
    """End points too scattered for the variance test: the stage ends after
    sf_kmax exploratory steps; with no converged position the span is the
    frontier alone."""
    run, lock = _sf_run(N=24, window=8), _sf_lock(sf_kmax=3, sf_k=2)
    x = np.array([1, 2, 3, 4] + [SF_MASK] * 20, np.int32)
    frozen, hp, st = np.zeros(24, np.uint8), np.ones(24, np.uint8), np.zeros(13, np.int32)
    c, x, frozen, hp, st = _sf_step(run, lock, x, frozen, hp, st, {20: 0.6, 6: 0.4, 7: 0.3})
    assert c == [6, 7] and st[0] == 0 and st[5] == 20
    # the window [4, 12) holds position 10 (0.6) and 5 (0.3): top-2
    c, x, frozen, hp, st = _sf_step(run, lock, x, frozen, hp, st, {10: 0.6, 4: 0.2, 5: 0.3})
    assert c == [5, 10] and st[0] == 0 and list(st[5:7]) == [20, 10]  # variance 25
    # third exploratory step: no position reaches 0.5 -> nothing recorded;
    # sf_kmax reached -> span [4, 11) up to the last end point (10); no
    # in-span position above 0.8 -> top-2 of the span: 9 (0.45) and 4 (0.1,
    # smallest position among the rest); 11.. freeze
    c, x, frozen, hp, st = _sf_step(run, lock, x, frozen, hp, st, {9: 0.45})
    assert c == [4, 9] and list(st[:5]) == [1, 4, 11, 3, 2]
    assert frozen.tolist() == [0] * 11 + [1] * 13


def test_slowfast_kmax_without_end_point():
    """No position ever reaches the convergence threshold: the stage ends by
    sf_kmax with the frontier alone as the span, decoded at once."""
    run, lock = _sf_run(N=12, window=2), _sf_lock(sf_kmax=2)
    x = np.array([1, 2, 3, 4] + [SF_MASK] * 8, np.int32)
    frozen, hp, st = np.zeros(12, np.uint8), np.ones(12, np.uint8), np.zeros(13, np.int32)
    c, x, frozen, hp, st = _sf_step(run, lock, x, frozen, hp, st, {5: 0.3})
    assert c == [5] and list(st[:5]) == [0, 0, 0, 1, 0]
    c, x, frozen, hp, st = _sf_step(run, lock, x, frozen, hp, st, {7: 0.3})
    assert c == [4] and not st.any() and not frozen.any()


def test_slowfast_variance_test_against_numpy():
    """The stage-end test against numpy's population variance of the last
    sf_whist end points, on random end-point sequences (W = 1..4)."""
    rng = np.random.default_rng(5)
    for W in (1, 2, 3, 4):
        for trial in range(40):
            var_thr = float(rng.choice([0.5, 1.0, 2.0, 6.25]))
            lock = _sf_lock(sf_whist=W, sf_kmax=100, sf_var=var_thr)
            N = 64
            run = _sf_run(N=N, window=1)
            x = np.array([1, 2, 3, 4] + [SF_MASK] * (N - 4), np.int32)
            frozen, hp, st = np.zeros(N, np.uint8), np.ones(N, np.uint8), np.zeros(13, np.int32)
            ends = []
            for step in range(6):
                s = int(np.argmax(x == SF_MASK))
                e = int(rng.integers(s, min(N, s + 6)))
                ends.append(e)
                # only position e reaches tau_conv, below tau_high; the window of
                # one position commits the frontier while exploring
                c, x, frozen, hp, st = _sf_step(run, lock, x, frozen, hp, st, {e: 0.6})
                last = ends[-W:]
                stable = len(ends) >= W and np.var(np.array(last, np.float64)) < var_thr
                if stable:
                    assert st[0] == 1 or (not st.any()), (W, ends)
                    break
                assert st[0] == 0 and c == [s], (W, ends, st)


def test_slowfast_ties_prefer_smaller_position():
    run, lock = _sf_run(), _sf_lock(sf_k=2)
    x = np.array([1, 2, 3, 4] + [SF_MASK] * 12, np.int32)
    frozen, hp, st = np.zeros(16, np.uint8), np.ones(16, np.uint8), np.zeros(13, np.int32)
    c, *_ = _sf_step(run, lock, x, frozen, hp, st, {4: 0.3, 5: 0.4, 6: 0.4, 7: 0.4})
    assert c == [5, 6]
