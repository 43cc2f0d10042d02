"""Kernel-level parity: each stage of the step on the GPU (through the op-level
C ABI) against the CPU oracle on identical seeded inputs."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from selective_token_recompute_amd import _lib as L
from selective_token_recompute_amd import ops
from tests.harness import top2_gap

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def _bf16_np(a: np.ndarray) -> np.ndarray:
    return synth.round_to_bf16(a.astype(np.float32))


def _dev(a: np.ndarray, dtype=torch.bfloat16) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV).to(dtype)


# --- compaction (bit exact) ----------------------------------------------------

@pytest.mark.parametrize("B,N,p", [(1, 1, 0.0), (3, 130, 0.0), (3, 130, 0.3), (3, 130, 1.0),
                                   (2, 64, 0.5), (1, 512, 0.25), (8, 1024, 0.9),
                                   (4, 4096, 0.7), (1, 65, 0.99)])
def test_compact_bit_exact(B, N, p):
    bits = synth.gen_lock_bits(B, N, p, seed=B * 1000 + N)
    rs, rp, mb, rst, M = ops.compact(torch.from_numpy(bits.view(np.int64)).to(DEV), B, N)
    seq, pos, mb_o = oracle.unit_compact(bits, N)
    assert M == len(seq)
    assert np.array_equal(rs.cpu().numpy(), seq) and np.array_equal(rp.cpu().numpy(), pos)
    assert np.array_equal(mb.cpu().numpy(), mb_o)
    assert np.array_equal(rst.cpu().numpy(), np.concatenate([[0], np.cumsum(mb_o)]))


# --- GEMM ----------------------------------------------------------------------

def _gemm_inputs(M, N, K, seed, bf16=True):
    A = synth.gen_normal((M, K), seed, 1.0, bf16=bf16)
    W = synth.gen_normal((N, K), seed + 1, 0.02, bf16=bf16)
    W2 = synth.gen_normal((N, K), seed + 2, 0.02, bf16=bf16)
    return A, W, W2


GEMM_M = [1, 15, 16, 17, 20, 33, 64, 65, 102, 128, 256, 384, 512, 1024]


@pytest.mark.parametrize("M", GEMM_M)
def test_gemm_store_bf16_ragged_m(M):
    N, K = 384, 512
    A, W, _ = _gemm_inputs(M, N, K, seed=M)
    C = ops.gemm(L.DLM_EPI_STORE_F32, _dev(A), _dev(W))
    ref = oracle.unit_linear(A, W)
    err = np.abs(_f64(C) - ref).max()
    assert err <= 1e-5 * max(1.0, np.abs(ref).max()) + 1e-5, err


@pytest.mark.parametrize("M,N,K", [(7, 200, 128), (130, 72, 256), (512, 4096, 4096),
                                   (384, 12288, 128), (9, 4096, 12288),
                                   # Dream-7B width at large M: the plan trades the
                                   # 256x256 tile for 256x192 to fill the last round
                                   (2500, 3584, 256)])
def test_gemm_resid_add_bf16(M, N, K):
    A, W, _ = _gemm_inputs(M, N, K, seed=N + K)
    h0 = synth.gen_normal((M, N), 99, 1.0)
    H = torch.from_numpy(h0).to(DEV)
    ops.gemm(L.DLM_EPI_RESID_ADD, _dev(A), _dev(W), C=H)
    ref = h0.astype(np.float64) + oracle.unit_linear(A, W)
    err = np.abs(_f64(H) - ref).max()
    assert err <= 2e-5 * max(1.0, np.abs(ref).max()), err


@pytest.mark.parametrize("M,N,K", [(1, 320, 512), (16, 320, 512), (33, 320, 512),
                                   (100, 320, 512), (384, 320, 512),
                                   # the 12-wave 256x192 tile of 384 < M <= 1536 at the
                                   # model's K: ragged M, several k-slices
                                   (385, 384, 4096), (700, 384, 4096), (1536, 384, 4096),
                                   # the fill-per-byte choice above M = 384: the 12-wave
                                   # 192x192 tile at d_ff 12288, 256x256 at d_ff 18944
                                   (640, 12288, 256), (640, 18944, 128)])
def test_gemm_swiglu_bf16(M, N, K):
    A, Wg, Wu = _gemm_inputs(M, N, K, seed=7 * M)
    U = ops.gemm(L.DLM_EPI_SWIGLU, _dev(A), _dev(Wg), W2=_dev(Wu))
    g = oracle.unit_linear(A, Wg)
    u = oracle.unit_linear(A, Wu)
    ref = g / (1.0 + np.exp(-g)) * u
    got = _f64(U)
    # output is stored in bf16: one rounding of a value with a tiny fp32 error
    err = np.abs(got - ref)
    assert (err <= 2.0 ** -8 * np.abs(ref) + 1e-5).all(), err.max()


@pytest.mark.parametrize("M", [1, 5, 64, 300])
def test_gemm_logits_scatter_bf16(M):
    B, N, V, K = 2, 160, 1000, 256
    rng = np.random.default_rng(M)
    flat = np.sort(rng.choice(B * N, M, replace=False))
    rs, rp = (flat // N).astype(np.int32), (flat % N).astype(np.int32)
    A, W, _ = _gemm_inputs(M, V, K, seed=3 * M)
    Z = torch.full((B, N, V), 7.0, device=DEV)
    ops.gemm(L.DLM_EPI_LOGITS, _dev(A), _dev(W), C=Z, row_seq=torch.from_numpy(rs).to(DEV),
             row_pos=torch.from_numpy(rp).to(DEV), seq_len=N, mask_id=V - 1)
    z = Z.cpu().numpy()
    ref = oracle.unit_linear(A, W)
    got = z[rs, rp]
    assert np.isneginf(got[:, V - 1]).all()
    assert np.abs(got[:, :-1] - ref[:, :-1]).max() <= 1e-5 * max(1, np.abs(ref).max())
    untouched = np.ones((B, N), bool)
    untouched[rs, rp] = False
    assert (z[untouched] == 7.0).all()


@pytest.mark.parametrize("epi", [L.DLM_EPI_STORE_F32, L.DLM_EPI_SWIGLU])
def test_gemm_fp32_generic(epi):
    M, N, K = 37, 172, 64
    A, W, W2 = _gemm_inputs(M, N, K, seed=5, bf16=False)
    C = ops.gemm(epi, _dev(A, torch.float32), _dev(W, torch.float32),
                 W2=_dev(W2, torch.float32) if epi == L.DLM_EPI_SWIGLU else None)
    g = oracle.unit_linear(A, W)
    if epi == L.DLM_EPI_SWIGLU:
        u = oracle.unit_linear(A, W2)
        ref = g / (1 + np.exp(-g)) * u
    else:
        ref = g
    assert np.abs(_f64(C) - ref).max() <= 1e-5 * max(1, np.abs(ref).max())


# --- attention -------------------------------------------------------------------

def _attn_case(B, N, nq, nkv, hd, rows_per_seq, seed, bf16=True):
    rng = np.random.default_rng(seed)
    kc = synth.gen_normal((B, nkv, N, hd), seed, 1.0, bf16=bf16)
    vc = synth.gen_normal((B, nkv, N, hd), seed + 1, 1.0, bf16=bf16)
    seqs = []
    for b in range(B):
        m = min(rows_per_seq[b], N)
        seqs.append(np.full(m, b, np.int32))
    row_seq = np.concatenate(seqs) if seqs else np.zeros(0, np.int32)
    M = len(row_seq)
    q = synth.gen_normal((M, nq, hd), seed + 2, 1.0, bf16=bf16)
    row_start = np.concatenate([[0], np.cumsum([len(s) for s in seqs])]).astype(np.int32)
    return q, kc, vc, row_seq, row_start


@pytest.mark.parametrize("B,N,nq,nkv,hd,rows", [
    (1, 32, 4, 4, 128, [32]),
    (1, 100, 4, 4, 128, [37]),        # ragged key tail
    (1, 512, 8, 8, 128, [384]),
    (1, 512, 8, 8, 128, [1]),         # split-KV at tiny M
    (3, 1024, 8, 2, 128, [5, 300, 77]),  # GQA, several sequences
    (2, 4096, 4, 4, 128, [9, 3]),
    (1, 256, 4, 1, 64, [100]),        # hd 64, MQA
    (1, 1024, 32, 32, 128, [256]),    # default plan: four key groups on 128-key tiles
    (1, 2048, 16, 16, 128, [256]),    # the same over two key splits
])
def test_attention_bf16_mfma(B, N, nq, nkv, hd, rows):
    q, kc, vc, rs, rst = _attn_case(B, N, nq, nkv, hd, rows, seed=N + nq)
    # the engine caches V transposed: [B][nkv][hd][N]
    o = ops.attention(_dev(q.reshape(len(rs), nq * hd)), torch.from_numpy(rst).to(DEV),
                      _dev(kc), _dev(vc.transpose(0, 1, 3, 2)), nq, nkv, hd)
    ref = oracle.unit_attention(q, rs, kc, vc).reshape(len(rs), nq * hd)
    err = np.abs(_f64(o) - ref)
    # P is rounded to bf16 before the PV product and o is stored in bf16
    assert (err <= 1e-2 + 2.0 ** -7 * np.abs(ref)).all(), err.max()


ATTN_LAYOUTS = [(1, 1), (2, 1), (4, 1), (2, 2), (4, 2)]  # (key groups, query blocks per wave)


@pytest.mark.parametrize("N", [320, 384])
@pytest.mark.parametrize("splits", [0, 1, 2, 3, 8, 64])
@pytest.mark.parametrize("stages", [2, 4])
@pytest.mark.parametrize("layout", ATTN_LAYOUTS)
def test_attention_forced_plans(splits, stages, layout, N):
    """Every split-KV count (including more splits than key tiles, which the
    plan clamps, and a count that leaves a short last range), LDS depth and
    wave layout, with two sequences of ragged row counts and GQA, against the
    oracle; N = 320 runs 64-key tiles, N = 384 the 128-key tiles."""
    B, nq, nkv, hd = 2, 8, 2, 128
    q, kc, vc, rs, rst = _attn_case(B, N, nq, nkv, hd, [37, 70], seed=11)
    o = ops.attention_config(_dev(q.reshape(len(rs), nq * hd)), torch.from_numpy(rst).to(DEV),
                             _dev(kc), _dev(vc.transpose(0, 1, 3, 2)), nq, nkv, hd,
                             splits=splits, stages=stages, key_halves=layout[0],
                             qblocks=layout[1])
    ref = oracle.unit_attention(q, rs, kc, vc).reshape(len(rs), nq * hd)
    err = np.abs(_f64(o) - ref)
    assert (err <= 1e-2 + 2.0 ** -7 * np.abs(ref)).all(), err.max()


@pytest.mark.parametrize("key_tile", [64, 128])
@pytest.mark.parametrize("layout", ATTN_LAYOUTS)
@pytest.mark.parametrize("B,N,nq,nkv,hd,rows", [
    (1, 1024, 4, 4, 128, [200]),   # 16 or 8 key tiles, 4 query tiles (one partly filled)
    (2, 256, 4, 1, 64, [100, 29]),  # hd 64, MQA: 4 queries per row share a wave
])
def test_attention_wave_layouts(layout, key_tile, B, N, nq, nkv, hd, rows):
    """Each wave layout and key tile without a forced split, at hd 64 and
    128, against the oracle."""
    q, kc, vc, rs, rst = _attn_case(B, N, nq, nkv, hd, rows, seed=N + hd + layout[0])
    o = ops.attention_config(_dev(q.reshape(len(rs), nq * hd)), torch.from_numpy(rst).to(DEV),
                             _dev(kc), _dev(vc.transpose(0, 1, 3, 2)), nq, nkv, hd, splits=1,
                             key_halves=layout[0], qblocks=layout[1], key_tile=key_tile)
    ref = oracle.unit_attention(q, rs, kc, vc).reshape(len(rs), nq * hd)
    err = np.abs(_f64(o) - ref)
    assert (err <= 1e-2 + 2.0 ** -7 * np.abs(ref)).all(), err.max()


@pytest.mark.parametrize("layout", list(range(ops.attention_num_layouts())))
@pytest.mark.parametrize("splits", [0, 1, 2, 3, 64])
@pytest.mark.parametrize("hd", [128, 64])
def test_attention_32x32_layouts(layout, splits, hd):
    """Every layout of the 32x32-MFMA kernel with each split count (the plan's,
    none, two, a count that leaves a short last range, more than there are
    key tiles), at both head sizes, with three sequences of ragged row counts
    (one empty, one longer than a workgroup's query tile) and GQA, against
    the oracle."""
    B, N, nq, nkv = 3, 384, 8, 2
    q, kc, vc, rs, rst = _attn_case(B, N, nq, nkv, hd, [37, 0, 140], seed=17 + layout + hd)
    o = ops.attention_layout(_dev(q.reshape(len(rs), nq * hd)), torch.from_numpy(rst).to(DEV),
                             _dev(kc), _dev(vc.transpose(0, 1, 3, 2)), nq, nkv, hd,
                             layout=layout, splits=splits)
    ref = oracle.unit_attention(q, rs, kc, vc).reshape(len(rs), nq * hd)
    err = np.abs(_f64(o) - ref)
    assert (err <= 1e-2 + 2.0 ** -7 * np.abs(ref)).all(), err.max()


@pytest.mark.parametrize("B,N,nq,nkv,rows", [
    (1, 512, 32, 32, [384]),    # the LLaDA-8B step at M = 384
    (1, 1024, 32, 32, [20]),    # one layer over a 1024-key cache at M = 20 (key splits)
    (1, 512, 32, 32, [9]),      # the end of a scheduled-lock run
    (1, 512, 32, 32, [288]),    # 64-query tiles: 32-query ones would need two rounds of CUs
    (1, 1024, 32, 32, [640]),   # 128-query tiles, for the same reason
    (2, 1024, 28, 4, [700, 1]),  # Dream-7B grouping, uneven sequences
])
def test_attention_32x32_default_plan(B, N, nq, nkv, rows):
    """The default plan at the benchmark's shapes (layout and split count of
    its own choosing), against the oracle."""
    hd = 128
    q, kc, vc, rs, rst = _attn_case(B, N, nq, nkv, hd, rows, seed=N + nq + rows[0])
    o = ops.attention(_dev(q.reshape(len(rs), nq * hd)), torch.from_numpy(rst).to(DEV),
                      _dev(kc), _dev(vc.transpose(0, 1, 3, 2)), nq, nkv, hd)
    ref = oracle.unit_attention(q, rs, kc, vc).reshape(len(rs), nq * hd)
    err = np.abs(_f64(o) - ref)
    assert (err <= 1e-2 + 2.0 ** -7 * np.abs(ref)).all(), err.max()


def test_attention_fp32_generic():
    B, N, nq, nkv, hd = 2, 32, 4, 2, 16
    q, kc, vc, rs, rst = _attn_case(B, N, nq, nkv, hd, [20, 7], seed=3, bf16=False)
    o = ops.attention(_dev(q.reshape(len(rs), nq * hd), torch.float32),
                      torch.from_numpy(rst).to(DEV), _dev(kc, torch.float32),
                      _dev(vc.transpose(0, 1, 3, 2), torch.float32), nq, nkv, hd)
    ref = oracle.unit_attention(q, rs, kc, vc).reshape(len(rs), nq * hd)
    assert np.abs(_f64(o) - ref).max() <= 1e-5


# --- vocabulary statistics -----------------------------------------------------------

def _vocab_run(z_cur, z_prev, has_prev_rows, kl_dir):
    """z_cur, z_prev: float32 [M][V]; rows placed at seq 0, positions 0..M-1."""
    M, V = z_cur.shape
    zc = torch.from_numpy(z_cur[None]).to(DEV)
    zp = torch.from_numpy(z_prev[None]).to(DEV)
    # previous log-normaliser from the oracle definition of the previous posterior
    prev_stats = oracle.unit_vocab_stats(z_prev.astype(np.float64), mask_id=V - 1)
    lse_prev = torch.from_numpy(prev_stats["lse"].astype(np.float32)[None]).to(DEV)
    hp = torch.from_numpy(np.asarray(has_prev_rows, np.int32)[None]).to(DEV)
    lse_cur = torch.zeros((1, M), device=DEV)
    rs = torch.zeros(M, dtype=torch.int32, device=DEV)
    rp = torch.arange(M, dtype=torch.int32, device=DEV)
    out = ops.vocab_stats(rs, rp, zc, zp, lse_prev, hp, lse_cur, mask_id=V - 1, kl_dir=kl_dir)
    # oracle: previous log-probabilities from the same fp32 logits and fp32 lse
    prev_logp = z_prev.astype(np.float64) - lse_prev.cpu().numpy()[0][:, None].astype(np.float64)
    ref = oracle.unit_vocab_stats(z_cur, prev_logp, np.asarray(has_prev_rows, np.uint8),
                                  mask_id=V - 1, kl_dir=kl_dir)
    return {k: v.cpu().numpy() for k, v in out.items()}, ref, hp.cpu().numpy(), lse_cur


@pytest.mark.parametrize("V", [126464, 1000, 1001, 152064])
@pytest.mark.parametrize("kl_dir", [0, 1])
def test_vocab_stats_random(V, kl_dir):
    rng = np.random.default_rng(V + kl_dir)
    M = 37
    z = (rng.standard_normal((M, V)) * 1.3).astype(np.float32)
    zp = (z + rng.standard_normal((M, V)).astype(np.float32) * 0.05).astype(np.float32)
    z[:, V - 1] = -np.inf
    zp[:, V - 1] = -np.inf
    hp = (np.arange(M) % 3 != 0).astype(np.int32)
    g, r, hp_after, lse_cur = _vocab_run(z, zp, hp, kl_dir)
    assert np.array_equal(g["argmax"], r["argmax"])
    assert np.allclose(g["conf"], r["conf"], rtol=1e-5, atol=0)
    assert np.allclose(g["lse"], r["lse"], rtol=0, atol=2e-5)
    hk = hp.astype(bool)
    assert np.array_equal(g["has_kl"], hp)
    assert np.isnan(g["kl"][~hk]).all()
    assert np.allclose(g["kl"][hk], r["kl"][hk], rtol=1e-3, atol=2e-6), \
        np.abs(g["kl"][hk] - r["kl"][hk]).max()
    assert (hp_after == 1).all() and np.allclose(lse_cur.cpu().numpy()[0], r["lse"], atol=2e-5)
    assert g["err"][0] == 0


def test_vocab_stats_adversarial():
    V = 4096
    M = 6
    z = np.zeros((M, V), np.float32)
    z[0, [5, 9, 3000]] = 2.0            # ties -> smallest index
    z[1, :] = 0.0                       # constant -> conf 1/(V-1), argmax 0
    z[2, 17] = 60.0                     # dominant logit
    z[3, :] = np.linspace(-80, 80, V)   # huge range
    z[4, 100:2000] = -np.inf            # -inf columns
    z[4, 2500] = 1.0
    z[5] = np.random.default_rng(1).standard_normal(V).astype(np.float32)
    z[:, V - 1] = 1e6                   # the mask column never counts
    zp = z.copy()                       # prev == cur -> KL 0
    g, r, _, _ = _vocab_run(z, zp, np.ones(M, np.int32), 0)
    assert g["argmax"].tolist() == [5, 0, 17, V - 2, 2500, int(np.argmax(z[5, :-1]))]
    assert np.array_equal(g["argmax"], r["argmax"])
    assert np.allclose(g["conf"], r["conf"], rtol=2e-5)
    assert np.abs(g["kl"]).max() <= 2e-6


# --- LM head with the statistics in its epilogue ------------------------------------------

LMSTATS_CFGS = [1, 5, 6, 7, 8, 9, 10, 12, 13, 14, 24, 25, 28]  # tiles the fused epilogue is built for


def _lm_head_stats_case(M, V, K, kl_dir, cfg=-1, seed=0, A=None, W=None):
    """Runs the fused LM head on M rows scattered over B=2 sequences of 96
    positions; returns (GPU outputs, the GPU's stored logits of the rows, the
    oracle's logits, the oracle's statistics of its own logits, context)."""
    B, N = 2, 96
    rng = np.random.default_rng(seed)
    flat = np.sort(rng.choice(B * N, M, replace=False))
    rs, rp = (flat // N).astype(np.int32), (flat % N).astype(np.int32)
    if A is None:
        A, W, _ = _gemm_inputs(M, V, K, seed=seed + 11)
    zref = oracle.unit_linear(A, W)
    zprev = (rng.standard_normal((B, N, V)) * 0.3).astype(np.float32)
    zprev[rs, rp] = (zref + rng.standard_normal((M, V)) * 0.05).astype(np.float32)
    zprev[..., V - 1] = -np.inf
    lse_prev = oracle.unit_vocab_stats(zprev.reshape(-1, V), mask_id=V - 1)["lse"]
    lse_prev = lse_prev.astype(np.float32).reshape(B, N)
    hp = (rng.random((B, N)) < 0.7).astype(np.int32)
    Z = torch.full((B, N, V), 7.0, device=DEV)
    hp_d = torch.from_numpy(hp.copy()).to(DEV)
    lse_cur = torch.full((B, N), -5.0, device=DEV)
    out = ops.lm_head_stats(_dev(A), _dev(W), Z, torch.from_numpy(rs).to(DEV),
                            torch.from_numpy(rp).to(DEV), torch.from_numpy(zprev).to(DEV),
                            torch.from_numpy(lse_prev).to(DEV), hp_d, lse_cur, mask_id=V - 1,
                            kl_dir=kl_dir, cfg=cfg)
    g = {k: v.cpu().numpy() for k, v in out.items()}
    z = Z.cpu().numpy()
    got = z[rs, rp]
    prev_logp = zprev[rs, rp].astype(np.float64) - lse_prev[rs, rp].astype(np.float64)[:, None]
    zo = zref.copy()
    zo[:, V - 1] = -np.inf
    ref = oracle.unit_vocab_stats(zo, prev_logp, hp[rs, rp].astype(np.uint8), mask_id=V - 1,
                                  kl_dir=kl_dir)
    ctx = dict(rs=rs, rp=rp, z=z, hp=hp, hp_after=hp_d.cpu().numpy(),
               lse_cur=lse_cur.cpu().numpy(), zprev=zprev, lse_prev=lse_prev)
    return g, got, zref, ref, ctx


def _check_lm_head_stats(g, got, zref, ref, ctx, V):
    rs, rp = ctx["rs"], ctx["rp"]
    # the logits: stored at each row's slot, mask column -inf, other slots untouched
    assert np.isneginf(got[:, V - 1]).all()
    assert np.abs(got[:, :-1] - zref[:, :-1]).max() <= 1e-5 * max(1, np.abs(zref).max())
    untouched = np.ones(ctx["z"].shape[:2], bool)
    untouched[rs, rp] = False
    assert (ctx["z"][untouched] == 7.0).all()
    # the statistics against the oracle's statistics of its own (fp64) logits:
    # with every logit within dz of the oracle's, lse moves by at most dz, the
    # confidence by a factor within e^(+-2 dz), KL by at most 4 dz (plus fp32
    # accumulation); argmax may differ only where the oracle's top two logits
    # are within 2 dz
    dz = float(np.abs(got[:, :-1] - zref[:, :-1]).max())
    hk = ctx["hp"][rs, rp].astype(bool)
    gap = top2_gap(zref, V - 1)
    bad = g["argmax"] != ref["argmax"]
    assert not (bad & (gap > 2.0 * dz + 1e-12)).any(), (int(bad.sum()), dz)
    assert (np.abs(g["conf"] - ref["conf"]) <= ref["conf"] * (2.5 * dz + 1e-5) + 1e-7).all()
    assert (np.abs(g["lse"] - ref["lse"]) <= dz + 2e-5).all()
    assert np.array_equal(g["has_kl"].astype(bool), hk)
    assert np.isnan(g["kl"][~hk]).all()
    if hk.any():
        err = np.abs(g["kl"][hk] - ref["kl"][hk])
        assert (err <= 1e-3 * np.abs(ref["kl"][hk]) + 4.0 * dz + 2e-6).all(), err.max()
    # per-position state: has_prev set and lse recorded at the active slots only
    after = ctx["hp"].copy()
    after[rs, rp] = 1
    assert np.array_equal(ctx["hp_after"], after)
    assert (np.abs(ctx["lse_cur"][rs, rp] - ref["lse"]) <= dz + 2e-5).all()
    assert (ctx["lse_cur"][untouched] == -5.0).all()
    assert g["err"][0] == 0


@pytest.mark.parametrize("M,V,K", [(1, 1000, 256), (37, 1001, 256), (150, 9001, 128),
                                   (192, 40000, 128), (100, 126464, 64)])
@pytest.mark.parametrize("kl_dir", [0, 1])
def test_lm_head_stats_vs_oracle(M, V, K, kl_dir):
    g, got, zref, ref, ctx = _lm_head_stats_case(M, V, K, kl_dir, seed=M + V + kl_dir)
    _check_lm_head_stats(g, got, zref, ref, ctx, V)


@pytest.mark.parametrize("cfg", LMSTATS_CFGS)
def test_lm_head_stats_every_tile(cfg):
    g, got, zref, ref, ctx = _lm_head_stats_case(70, 1001, 128, cfg % 2, cfg=cfg, seed=cfg)
    _check_lm_head_stats(g, got, zref, ref, ctx, 1001)


@pytest.mark.parametrize("cfg", [1, 12, 13])
def test_lm_head_stats_matches_unfused_path(cfg):
    """On one tile configuration, the same logits (bit for bit) and statistics
    as the LM-head GEMM with the plain logits epilogue followed by the
    separate vocabulary-statistics kernel."""
    M, V, K = 120, 5000, 256
    g, got, zref, ref, ctx = _lm_head_stats_case(M, V, K, 0, cfg=cfg, seed=5)
    rs, rp = (torch.from_numpy(ctx[k]).to(DEV) for k in ("rs", "rp"))
    A, W, _ = _gemm_inputs(M, V, K, seed=5 + 11)
    Z = torch.full((2, 96, V), 7.0, device=DEV)
    ops.gemm_config(L.DLM_EPI_LOGITS, _dev(A), _dev(W), cfg, splits=1, C=Z, row_seq=rs,
                    row_pos=rp, seq_len=96, mask_id=V - 1)
    assert np.array_equal(Z.cpu().numpy(), ctx["z"])  # identical logits, bit for bit
    zprev = torch.from_numpy(ctx["zprev"]).to(DEV)
    lse_prev = torch.from_numpy(ctx["lse_prev"]).to(DEV)
    u = ops.vocab_stats(rs, rp, Z, zprev, lse_prev,
                        torch.from_numpy(ctx["hp"].copy()).to(DEV), torch.zeros((2, 96), device=DEV),
                        mask_id=V - 1, kl_dir=0)
    u = {k: v.cpu().numpy() for k, v in u.items()}
    assert np.array_equal(u["argmax"], g["argmax"])
    assert np.allclose(u["conf"], g["conf"], rtol=1e-5)
    assert np.allclose(u["lse"], g["lse"], atol=1e-5)
    hk = u["has_kl"].astype(bool)
    assert np.array_equal(hk, g["has_kl"].astype(bool))
    assert np.allclose(u["kl"][hk], g["kl"][hk], rtol=1e-3, atol=2e-6)


def test_lm_head_stats_ties_and_mask_column():
    """Equal maxima in different column tiles go to the smaller index; a
    mask-token column with the largest logit never counts."""
    M, V, K = 40, 3000, 128
    A, W, _ = _gemm_inputs(M, V, K, seed=77)
    # integer activations and winner rows 4 e_0: every winner logit is exactly
    # 4.0 whatever order a tile sums its k-slices in (the other logits stay
    # well below that: |z| of a few tenths)
    A = np.random.default_rng(77).integers(-2, 3, size=A.shape).astype(A.dtype)
    A[:, 0] = 1.0
    row = np.zeros_like(W[5])
    row[0] = 4.0
    W[5] = row      # three equal winners in different column tiles
    W[700] = row
    W[2998] = row
    W[V - 1, 0] = 40.0  # the mask column: largest, excluded
    g, got, zref, ref, ctx = _lm_head_stats_case(M, V, K, 0, seed=3, A=A, W=W)
    assert (got[:, 5] == got[:, 700]).all() and (got[:, 5] == got[:, 2998]).all()
    assert (g["argmax"] == 5).all()
    _check_lm_head_stats(g, got, zref, ref, ctx, V)


# --- commit + lock (bit exact) ----------------------------------------------------

def _golden():
    with open(os.path.join(os.path.dirname(__file__), "golden",
                           "lock_transition_cases.json")) as f:
        return json.load(f)["cases"]


def _commit_lock_gpu(case_like, t, rows_seq, rows_pos, real, argmax, conf, kl, has_kl, x,
                     locked, cnt, lock, run, mask_id):
    from tests.harness import bool_to_bits, bits_to_bool
    B, N = run.batch, run.seq_len
    sch = oracle.unit_schedule(run, t)
    rs = np.asarray(rows_seq, np.int32)
    counts = np.bincount(rs, minlength=B)
    rst = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    dv = lambda a, dt=torch.int32: torch.from_numpy(np.ascontiguousarray(a)).to(DEV).to(dt)
    tok = dv(np.asarray(x, np.int32))
    bits = dv(bool_to_bits(np.asarray(locked, np.uint8)).view(np.int64), torch.int64)
    cn = dv(np.asarray(cnt, np.int32))
    ops.commit_lock(batch=B, seq_len=N, prompt_len=run.prompt_len, mask_id=mask_id,
                    blk_lo=sch["lo"], blk_hi=sch["hi"], k=max(sch["k"], 0) if sch["beta"] >= 0 else 0,
                    do_commit=1, do_lock=1, policy=1 if lock["policy"] == "test" else 0,
                    kl_eps=lock["kl_eps"], conf_tau=lock["conf_tau"], n_consec=lock["n_consec"],
                    lock_prompt=int(t == 0 and lock["lock_prompt_after_first_step"]),
                    row_seq=dv(rs), row_pos=dv(np.asarray(rows_pos, np.int32)),
                    row_start=dv(rst), row_real=dv(np.asarray(real, np.int32)),
                    argmax=dv(np.asarray(argmax, np.int32)),
                    conf=dv(np.asarray(conf, np.float32), torch.float32),
                    kl=dv(np.asarray(kl, np.float32), torch.float32),
                    has_kl=dv(np.asarray(has_kl, np.int32)), tokens=tok, bits=bits, counters=cn)
    return (tok.cpu().numpy(), bits_to_bool(bits.cpu().numpy().view(np.uint64), N),
            cn.cpu().numpy())


@pytest.mark.parametrize("case", _golden(), ids=lambda c: c["name"])
def test_commit_lock_golden(case):
    run = synth.RunShape(case["batch"], case["seq_len"], case["prompt_len"], case["steps"],
                         case["block_len"])
    lock = {k: case[k] for k in ("policy", "kl_eps", "conf_tau", "n_consec",
                                 "lock_prompt_after_first_step")}
    x0 = np.array(case["x"], np.int32)
    mask_id = case["vocab"] - 1
    real = [int(x0[s, p] != mask_id) for s, p in zip(case["row_seq"], case["row_pos"])]
    x, lk, cnt = _commit_lock_gpu(case, case["t"], case["row_seq"], case["row_pos"], real,
                                  case["argmax"], case["conf"], case["kl"], case["has_kl"], x0,
                                  case["locked"], case["cnt"], lock, run, mask_id)
    assert x.tolist() == case["expect_x"]
    assert lk.tolist() == case["expect_locked"]
    assert cnt.tolist() == case["expect_cnt"]


# (batch, seq_len, prompt_len, steps, block_len): blocks of 130 (one gather
# pass per sequence); blocks of 1250 with more than 1024 rows per sequence
# (several gather passes) and k of about 60 or 400 per step
COMMIT_RUNS = [(3, 300, 40, 20, 130)] * 6 + [(2, 2600, 100, 40, 1250)] * 2 + \
    [(2, 2600, 100, 6, 1250)] * 2


@pytest.mark.parametrize("seed", range(len(COMMIT_RUNS)))
def test_commit_lock_random_vs_oracle(seed):
    rng = np.random.default_rng(100 + seed)
    B, N, P, T, blk = COMMIT_RUNS[seed]
    run = synth.RunShape(B, N, P, T, blk)
    V = 50
    lock = dict(policy="test", kl_eps=1e-3, conf_tau=0.3, n_consec=2,
                lock_prompt_after_first_step=1)
    shape = synth.ModelShape(1, 8, 1, 1, 8, 8, V, bf16=False)
    t = int(rng.integers(0, run.steps))
    x = np.where(rng.random((B, N)) < 0.5, V - 1, rng.integers(0, V - 1, (B, N))).astype(np.int32)
    x[:, :P] = rng.integers(0, V - 1, (B, P))
    locked = (rng.random((B, N)) < 0.3) & (x != V - 1)
    cnt = rng.integers(0, 2, (B, N)).astype(np.int32)
    rows = [(b, i) for b in range(B) for i in range(N) if not locked[b, i]]
    rs = np.array([r[0] for r in rows], np.int32)
    rp = np.array([r[1] for r in rows], np.int32)
    M = len(rows)
    real = (x[rs, rp] != V - 1).astype(np.uint8)
    conf = np.round(rng.random(M), 2).astype(np.float32)  # many exact ties
    kl = (rng.random(M) * 2e-3).astype(np.float32)
    has_kl = (rng.random(M) < 0.8).astype(np.uint8)
    am = rng.integers(0, V - 1, M).astype(np.int32)
    xo, lo, co = oracle.unit_lock_transition(shape, run, lock, t, rs, rp, real, am,
                                             conf.astype(np.float64), kl.astype(np.float64),
                                             has_kl, x, locked.astype(np.uint8), cnt)
    lock32 = dict(lock, kl_eps=float(np.float32(lock["kl_eps"])))
    xg, lg, cg = _commit_lock_gpu(None, t, rs, rp, real, am, conf, kl, has_kl, x,
                                  locked.astype(np.uint8), cnt, lock32, run, V - 1)
    assert np.array_equal(xg, xo) and np.array_equal(lg, lo) and np.array_equal(cg, co)


# --- norms and rotary scatter ---------------------------------------------------------

@pytest.mark.parametrize("bf16", [False, True])
def test_embed_rmsnorm_and_rmsnorm(bf16):
    V, d, N = 300, 512, 40
    dt = torch.bfloat16 if bf16 else torch.float32
    emb = synth.gen_normal((V, d), 1, 0.5, bf16=bf16)
    g = synth.gen_normal((d,), 2, 1.0, bf16=bf16)
    rng = np.random.default_rng(0)
    tokens = rng.integers(0, V, (2, N)).astype(np.int32)
    tokens[0, 3] = V - 1
    rs = np.array([0, 0, 1, 1, 1], np.int32)
    rp = np.array([3, 9, 0, 17, 39], np.int32)
    h, y, real = ops.embed_rmsnorm(torch.from_numpy(tokens).to(DEV), torch.from_numpy(rs).to(DEV),
                                   torch.from_numpy(rp).to(DEV), _dev(emb, dt), _dev(g, dt),
                                   1e-5, V - 1)
    x = emb[tokens[rs, rp]].astype(np.float64)
    assert np.array_equal(_f64(h), x)
    ref = oracle.unit_rmsnorm(x, g, 1e-5)
    tol = (2.0 ** -8 * np.abs(ref) + 1e-6) if bf16 else 1e-5 * (1 + np.abs(ref))
    assert (np.abs(_f64(y) - ref) <= tol).all()
    assert real.cpu().numpy().tolist() == [0, 1, 1, 1, 1]
    y2 = ops.rmsnorm(h, _dev(g, dt), 1e-5)
    assert (np.abs(_f64(y2) - ref) <= tol).all()


@pytest.mark.parametrize("bf16", [False, True])
def test_rope_scatter(bf16):
    B, N, nq, nkv, hd = 2, 600, 4, 2, 128
    dt = torch.bfloat16 if bf16 else torch.float32
    rng = np.random.default_rng(4)
    rs = np.array([0, 0, 1, 1], np.int32)
    rp = np.array([0, 599, 5, 300], np.int32)
    M = len(rs)
    qkv = synth.gen_normal((M, (nq + 2 * nkv) * hd), 8, 1.0)
    table = ops.rope_table(N, hd, 10000.0)
    q = torch.zeros((M, nq * hd), dtype=dt, device=DEV)
    kc = torch.full((B, nkv, N, hd), 3.0, dtype=dt, device=DEV)
    vc = torch.full((B, nkv, hd, N), 3.0, dtype=dt, device=DEV)  # transposed V cache
    ops.rope_scatter(torch.from_numpy(qkv).to(DEV), torch.from_numpy(rs).to(DEV),
                     torch.from_numpy(rp).to(DEV), table, q, kc, vc, nq, nkv, hd)
    x = qkv.astype(np.float64).reshape(M, nq + 2 * nkv, hd)
    rot = oracle.unit_rope(x[:, : nq + nkv], rp, 10000.0)
    tol = lambda ref: (2.0 ** -8 * np.abs(ref) + 2e-6) if bf16 else 2e-5 * (1 + np.abs(ref))
    qr = rot[:, :nq].reshape(M, nq * hd)
    assert (np.abs(_f64(q) - qr) <= tol(qr)).all()
    kcn, vcn = _f64(kc), _f64(vc)
    for i in range(M):
        kr = rot[i, nq:]
        assert (np.abs(kcn[rs[i], :, rp[i]] - kr) <= tol(kr)).all()
        vr = x[i, nq + nkv:]
        assert (np.abs(vcn[rs[i], :, :, rp[i]] - vr) <= tol(vr)).all()
    touched = np.zeros((B, N), bool)
    touched[rs, rp] = True
    assert (kcn[np.broadcast_to(~touched[:, None, :], kcn.shape[:3])] == 3.0).all()
    assert (np.moveaxis(vcn, 3, 2)[np.broadcast_to(~touched[:, None, :], kcn.shape[:3])] == 3.0).all()


@pytest.mark.parametrize("cfg", [35, 36, 37, 38, 39, 40, 41, 42, 43, 45, 47, 48, 49])
@pytest.mark.parametrize("epi", [L.DLM_EPI_STORE_F32, L.DLM_EPI_SWIGLU])
def test_gemm_prefetch_tiles_long_k(cfg, epi):
    """The fragment-prefetch tiles over a long K (64 k-slices: the steady
    two-step loop and every tail length), ragged M and N, against the oracle."""
    if epi == L.DLM_EPI_SWIGLU and cfg == 42:
        pytest.skip("48-column wave tiles cannot pair gate and up")
    for M, N, K in [(200, 300, 4096), (77, 130, 64 * 7), (5, 40, 64 * 5)]:
        A, W, W2 = _gemm_inputs(M, N, K, seed=cfg + K)
        g = oracle.unit_linear(A, W)
        if epi == L.DLM_EPI_SWIGLU:
            u = oracle.unit_linear(A, W2)
            want = g / (1 + np.exp(-g)) * u
            C = ops.gemm_config(epi, _dev(A), _dev(W), cfg, 1, W2=_dev(W2))
            tol = 2.0 ** -8 * np.abs(want) + 1e-5
        else:
            want = g
            C = ops.gemm_config(epi, _dev(A), _dev(W), cfg, 1)
            tol = 2e-5 * max(1.0, np.abs(want).max())
        got = _f64(C)
        assert (np.abs(got - want) <= tol).all(), (M, N, K, np.abs(got - want).max())


# every tile configuration but 13 (256x256 with a 2-slice ring: one wave row
# of fp32 results does not fit its LDS, so the op refuses it); tiles of 64,
# 192 and 256 columns split or straddle heads
QKV_CFGS = [c for c in range(ops.num_gemm_configs()) if c != 13]


def test_gemm_qkv_refuses_oversized_tile():
    with pytest.raises(L.DlmError) as e:
        _qkv_fused_case(8, 16, 13, seed=1)
    assert e.value.status == L.DLM_E_UNSUPPORTED


def _qkv_fused_case(M, N, cfg, seed):
    """Fused QKV (projection + rotary + cache scatter) on M rows of B=2
    sequences of N positions, GQA 4/2 heads of 128; returns the GPU outputs
    and the oracle's (fp64 linear, rotary)."""
    B, nq, nkv, hd, K = 2, 4, 2, 128, 256
    rng = np.random.default_rng(seed)
    flat = np.sort(rng.choice(B * N, M, replace=False))
    rs, rp = (flat // N).astype(np.int32), (flat % N).astype(np.int32)
    A, W, _ = _gemm_inputs(M, (nq + 2 * nkv) * hd, K, seed=seed + 1)
    table = ops.rope_table(N, hd, 10000.0)
    q = torch.zeros((M, nq * hd), dtype=torch.bfloat16, device=DEV)
    kc = torch.full((B, nkv, N, hd), 3.0, dtype=torch.bfloat16, device=DEV)
    vc = torch.full((B, nkv, hd, N), 3.0, dtype=torch.bfloat16, device=DEV)
    ops.gemm_qkv(_dev(A), _dev(W), torch.from_numpy(rs).to(DEV), torch.from_numpy(rp).to(DEV),
                 table, q, kc, vc, nq, nkv, cfg=cfg)
    x = oracle.unit_linear(A, W).reshape(M, nq + 2 * nkv, hd)
    rot = oracle.unit_rope(x[:, : nq + nkv], rp, 10000.0)
    return dict(rs=rs, rp=rp, q=_f64(q), kc=_f64(kc), vc=_f64(vc), x=x, rot=rot, nq=nq, nkv=nkv)


def _check_qkv_fused(c, B=2):
    tol = lambda ref: 2.0 ** -8 * np.abs(ref) + 1e-5
    nq, nkv, rs, rp = c["nq"], c["nkv"], c["rs"], c["rp"]
    M = len(rs)
    qr = c["rot"][:, :nq].reshape(M, -1)
    assert (np.abs(c["q"] - qr) <= tol(qr)).all(), np.abs(c["q"] - qr).max()
    kr = c["rot"][:, nq:]                      # [M][nkv][hd]
    kg = c["kc"][rs, :, rp]                    # [M][nkv][hd]
    assert (np.abs(kg - kr) <= tol(kr)).all(), np.abs(kg - kr).max()
    vr = c["x"][:, nq + nkv:]
    vg = np.moveaxis(c["vc"], 3, 2)[rs, :, rp]  # [M][nkv][hd]
    assert (np.abs(vg - vr) <= tol(vr)).all(), np.abs(vg - vr).max()
    N = c["kc"].shape[2]
    untouched = np.ones((B, N), bool)
    untouched[rs, rp] = False
    assert (np.moveaxis(c["kc"], 2, 1)[untouched] == 3.0).all()
    assert (np.moveaxis(c["vc"], 3, 1)[untouched] == 3.0).all()


@pytest.mark.parametrize("cfg", QKV_CFGS)
def test_gemm_qkv_fused_every_tile(cfg):
    # dense active rows (runs of consecutive positions: packed V stores) and
    # a ragged row count
    _check_qkv_fused(_qkv_fused_case(203, 128, cfg, seed=cfg))


@pytest.mark.parametrize("M,N", [(1, 600), (37, 602), (96, 130), (384, 512), (500, 4096)])
def test_gemm_qkv_fused_default_plan(M, N):
    # N % 4 != 0 takes the unpacked V stores; sparse rows break position runs
    _check_qkv_fused(_qkv_fused_case(M, N, -1, seed=M + N))


@pytest.mark.parametrize("splits", [1, 3])
@pytest.mark.parametrize("epi", [L.DLM_EPI_STORE_F32, L.DLM_EPI_RESID_ADD, L.DLM_EPI_SWIGLU,
                                 L.DLM_EPI_LOGITS])
def test_gemm_every_tile_config(epi, splits):
    """Every MFMA tile configuration the plan may choose, with and without
    split-K (the last workgroup of a tile reduces), called twice on the same
    workspace, against the oracle; ragged M and N exercise the guards."""
    M, N, K = 77, 200, 384
    A, W, W2 = _gemm_inputs(M, N, K, seed=31)
    g = oracle.unit_linear(A, W)
    if epi == L.DLM_EPI_SWIGLU:
        u = oracle.unit_linear(A, W2)
        ref = g / (1 + np.exp(-g)) * u
    else:
        ref = g
    rs = torch.zeros(M, dtype=torch.int32, device=DEV)
    rp = torch.arange(M, dtype=torch.int32, device=DEV)
    for cfg in range(ops.num_gemm_configs()):
        if epi == L.DLM_EPI_SWIGLU and cfg in (7, 27, 42):
            continue  # an odd number of 16-column wave tiles cannot pair gate and up
        for call in range(2):
            if epi == L.DLM_EPI_RESID_ADD:
                h0 = synth.gen_normal((M, N), 5 + call, 1.0)
                C = torch.from_numpy(h0).to(DEV)
                ops.gemm_config(epi, _dev(A), _dev(W), cfg, splits, C=C)
                got, want = _f64(C), h0.astype(np.float64) + ref
            elif epi == L.DLM_EPI_LOGITS:
                C = torch.zeros((1, 96, N), device=DEV)
                ops.gemm_config(epi, _dev(A), _dev(W), cfg, splits, C=C, row_seq=rs, row_pos=rp,
                                seq_len=96, mask_id=N - 1)
                got = C.cpu().numpy()[0, :M].astype(np.float64)
                assert np.isneginf(got[:, N - 1]).all()
                got, want = got[:, :-1], ref[:, :-1]
            else:
                C = ops.gemm_config(epi, _dev(A), _dev(W), cfg, splits,
                                    W2=_dev(W2) if epi == L.DLM_EPI_SWIGLU else None)
                got, want = _f64(C), ref
            tol = (2.0 ** -8 * np.abs(want) + 1e-5) if epi == L.DLM_EPI_SWIGLU else \
                (2e-5 * max(1.0, np.abs(want).max()))
            assert (np.abs(got - want) <= tol).all(), (cfg, call, np.abs(got - want).max())
