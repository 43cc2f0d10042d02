"""Op-level calls (include/dlm_ops.h) on torch device tensors: one stage of the
step per call, with the same kernels and launch plans the engine uses.
Argument marshalling only."""
from __future__ import annotations

from typing import Optional

import torch

from . import _lib as L


def _s(stream=None) -> int:
    return (stream if stream is not None else torch.cuda.current_stream()).cuda_stream


def _p(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _dt(t: torch.Tensor) -> int:
    return L.DLM_BF16 if t.dtype == torch.bfloat16 else L.DLM_FP32


def compact(bits: torch.Tensor, batch: int, seq_len: int):
    """bits int64 [B][W] (uint64 bit patterns) -> row_seq, row_pos, m_b, row_start, M."""
    dev = bits.device
    n = batch * seq_len
    row_seq = torch.empty(n, dtype=torch.int32, device=dev)
    row_pos = torch.empty(n, dtype=torch.int32, device=dev)
    m_b = torch.empty(batch, dtype=torch.int32, device=dev)
    row_start = torch.empty(batch + 1, dtype=torch.int32, device=dev)
    ctl = torch.zeros(4, dtype=torch.int32, device=dev)
    L.check(L.lib().dlm_op_compact(_p(bits), batch, seq_len, _p(row_seq), _p(row_pos), _p(m_b),
                                   _p(row_start), _p(ctl), _s()), "dlm_op_compact")
    M = int(ctl[0].item())
    return row_seq[:M], row_pos[:M], m_b, row_start, M


def embed_rmsnorm(tokens, row_seq, row_pos, emb, g, eps, mask_id):
    M, d = row_seq.numel(), emb.shape[1]
    h = torch.empty((M, d), dtype=torch.float32, device=emb.device)
    y = torch.empty((M, d), dtype=emb.dtype, device=emb.device)
    real = torch.empty(M, dtype=torch.int32, device=emb.device)
    L.check(L.lib().dlm_op_embed_rmsnorm(_dt(emb), M, d, tokens.shape[1], float(eps), mask_id,
                                         _p(tokens), _p(row_seq), _p(row_pos), _p(emb), _p(g),
                                         _p(h), _p(y), _p(real), _s()), "dlm_op_embed_rmsnorm")
    return h, y, real


def rmsnorm(x: torch.Tensor, g: torch.Tensor, eps: float) -> torch.Tensor:
    M, d = x.shape
    y = torch.empty((M, d), dtype=g.dtype, device=x.device)
    L.check(L.lib().dlm_op_rmsnorm(_dt(g), M, d, float(eps), _p(x), _p(g), _p(y), _s()),
            "dlm_op_rmsnorm")
    return y


def gemm_ws_bytes(dtype: int, epi: int, M: int, N: int, K: int) -> int:
    return int(L.lib().dlm_op_gemm_ws_bytes(dtype, epi, M, N, K))


def gemm(epi: int, A: torch.Tensor, W: torch.Tensor, W2=None, C=None, row_seq=None,
         row_pos=None, seq_len: int = 0, mask_id: int = 0, ws=None):
    """Runs one GEMM plan; C is allocated for STORE_F32 / SWIGLU if not given."""
    M, K = A.shape
    N = W.shape[0]
    dt = _dt(A)
    if C is None:
        if epi == L.DLM_EPI_STORE_F32:
            C = torch.empty((M, N), dtype=torch.float32, device=A.device)
        elif epi == L.DLM_EPI_SWIGLU:
            C = torch.empty((M, N), dtype=A.dtype, device=A.device)
        else:
            raise ValueError("C required for this epilogue")
    need = gemm_ws_bytes(dt, epi, M, N, K)
    if ws is None and need > 0:
        ws = torch.zeros(need, dtype=torch.uint8, device=A.device)  # split counters start at 0
    L.check(L.lib().dlm_op_gemm(dt, epi, M, N, K, _p(A), _p(W), _p(W2), _p(C), _p(row_seq),
                                _p(row_pos), seq_len, mask_id, _p(ws),
                                0 if ws is None else ws.numel(), _s()), "dlm_op_gemm")
    return C


def gemm_noalloc_max_bytes() -> int:
    return int(L.lib().dlm_op_gemm_noalloc_max_bytes())


def gemm_noalloc(epi: int, A: torch.Tensor, W: torch.Tensor, C: torch.Tensor, W2=None,
                 row_seq=None, row_pos=None, seq_len: int = 0, mask_id: int = 0) -> torch.Tensor:
    """dlm_op_gemm_noalloc: the GEMM with its split-K partials in the
    library's device scratch array; C must be given (nothing is allocated)."""
    M, K = A.shape
    N = W.shape[0]
    L.check(L.lib().dlm_op_gemm_noalloc(_dt(A), epi, M, N, K, _p(A), _p(W), _p(W2), _p(C),
                                        _p(row_seq), _p(row_pos), seq_len, mask_id, _s()),
            "dlm_op_gemm_noalloc")
    return C


def gemm_config(epi: int, A, W, cfg: int, splits: int = 0, W2=None, C=None, row_seq=None,
                row_pos=None, seq_len: int = 0, mask_id: int = 0):
    """GEMM with a forced tile configuration (cfg) and split-K factor."""
    M, K = A.shape
    N = W.shape[0]
    if C is None:
        C = torch.empty((M, N), dtype=torch.float32 if epi != L.DLM_EPI_SWIGLU else A.dtype,
                        device=A.device)
    need = max(splits, 1) * M * N * (8 if epi == L.DLM_EPI_SWIGLU else 4)
    ws = _ws_cache(need, A.device)
    L.check(L.lib().dlm_op_gemm_config(_dt(A), epi, M, N, K, _p(A), _p(W), _p(W2), _p(C),
                                       _p(row_seq), _p(row_pos), seq_len, mask_id, cfg, splits,
                                       _p(ws), ws.numel(), _s()), "dlm_op_gemm_config")
    return C


_WS = {}


def _ws_cache(nbytes, device):
    """A zeroed workspace reused across calls (split counters are left zero)."""
    t = _WS.get(device)
    if t is None or t.numel() < nbytes:
        t = torch.zeros(nbytes, dtype=torch.uint8, device=device)
        _WS[device] = t
    return t


def num_gemm_configs() -> int:
    return int(L.lib().dlm_op_gemm_num_configs())


def gemm_qkv(A, W, row_seq, row_pos, table, q, kc, vc, nq, nkv, cfg=-1):
    """QKV projection with rotary embedding and cache scatter fused (bf16,
    head_dim 128): q [M][nq*128], kc [B][nkv][N][128], vc [B][nkv][128][N]."""
    M, K = A.shape
    L.check(L.lib().dlm_op_gemm_qkv(M, K, nq, nkv, kc.shape[2], _p(A), _p(W), _p(row_seq),
                                    _p(row_pos), _p(table), _p(q), _p(kc), _p(vc), cfg, _s()),
            "dlm_op_gemm_qkv")


def rope_table(seq_len: int, head_dim: int, base: float, device="cuda") -> torch.Tensor:
    t = torch.empty((seq_len, head_dim // 2, 2), dtype=torch.float32, device=device)
    L.check(L.lib().dlm_op_rope_table(seq_len, head_dim, float(base), _p(t), _s()),
            "dlm_op_rope_table")
    return t


def rope_scatter(qkv, row_seq, row_pos, table, q, kc, vc, nq, nkv, hd):
    M = qkv.shape[0]
    L.check(L.lib().dlm_op_rope_scatter(_dt(q), M, nq, nkv, hd, kc.shape[2], _p(qkv), _p(row_seq),
                                        _p(row_pos), _p(table), _p(q), _p(kc), _p(vc), _s()),
            "dlm_op_rope_scatter")


def attention(q, row_start, kc, vc, nq, nkv, hd, o=None, ws=None):
    """q [M][nq*hd]; kc/vc [B][nkv][N][hd]; returns o [M][nq*hd]."""
    M = q.shape[0]
    B, _, N, _ = kc.shape
    dt = _dt(q)
    if o is None:
        o = torch.empty_like(q)
    need = int(L.lib().dlm_op_attention_ws_bytes(dt, M, B, N, nq, nkv, hd))
    if ws is None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    L.check(L.lib().dlm_op_attention(dt, M, B, N, nq, nkv, hd, _p(q), _p(row_start), _p(kc),
                                     _p(vc), _p(o), _p(ws), 0 if ws is None else ws.numel(),
                                     _s()), "dlm_op_attention")
    return o


def attention_config(q, row_start, kc, vc, nq, nkv, hd, splits=0, stages=0, key_halves=0,
                     qblocks=0, key_tile=0, o=None):
    """attention() with a forced split-KV count, LDS stage count, key groups
    (waves per 16-query block), 16-query blocks per wave and keys per LDS
    tile (0: the plan's)."""
    M = q.shape[0]
    B, _, N, _ = kc.shape
    dt = _dt(q)
    if o is None:
        o = torch.empty_like(q)
    need = int(L.lib().dlm_op_attention_config_ws_bytes(dt, M, B, N, nq, nkv, hd, splits))
    ws = _ws_cache(max(need, 256), q.device)
    L.check(L.lib().dlm_op_attention_config(dt, M, B, N, nq, nkv, hd, _p(q), _p(row_start), _p(kc),
                                            _p(vc), _p(o), splits, stages, key_halves, qblocks,
                                            key_tile, _p(ws),
                                            ws.numel(),
                                            _s()), "dlm_op_attention_config")
    return o


def attention_num_layouts() -> int:
    return int(L.lib().dlm_op_attention_num_layouts())


def attention_layout(q, row_start, kc, vc, nq, nkv, hd, layout=-1, splits=0, o=None):
    """attention() on the 32x32-MFMA kernel with a forced layout (-1: the
    plan's) and split count (0: the plan's)."""
    M = q.shape[0]
    B, _, N, _ = kc.shape
    dt = _dt(q)
    if o is None:
        o = torch.empty_like(q)
    need = int(L.lib().dlm_op_attention_layout_ws_bytes(dt, M, B, N, nq, nkv, hd, splits, layout))
    ws = _ws_cache(max(need, 256), q.device)
    L.check(L.lib().dlm_op_attention_layout(dt, M, B, N, nq, nkv, hd, _p(q), _p(row_start),
                                            _p(kc), _p(vc), _p(o), splits, layout, _p(ws),
                                            ws.numel(), _s()), "dlm_op_attention_layout")
    return o


def vocab_stats(row_seq, row_pos, z_cur, z_prev, lse_prev, has_prev, lse_cur, mask_id,
                kl_dir=0, ws=None):
    """z_cur/z_prev float [B][N][V]; has_prev int32 [B][N] (read, then set)."""
    M = row_seq.numel()
    B, N, V = z_cur.shape
    dev = z_cur.device
    out = dict(argmax=torch.empty(M, dtype=torch.int32, device=dev),
               conf=torch.empty(M, dtype=torch.float32, device=dev),
               kl=torch.empty(M, dtype=torch.float32, device=dev),
               has_kl=torch.empty(M, dtype=torch.int32, device=dev),
               lse=torch.empty(M, dtype=torch.float32, device=dev),
               err=torch.zeros(1, dtype=torch.int32, device=dev))
    need = int(L.lib().dlm_op_vocab_ws_bytes(M, V))
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    L.check(L.lib().dlm_op_vocab_stats(M, V, mask_id, kl_dir, N, _p(row_seq), _p(row_pos),
                                       _p(z_cur), _p(z_prev), _p(lse_prev), _p(has_prev),
                                       _p(lse_cur), _p(out["argmax"]), _p(out["conf"]),
                                       _p(out["kl"]), _p(out["has_kl"]), _p(out["lse"]),
                                       _p(out["err"]), _p(ws), ws.numel(), _s()),
            "dlm_op_vocab_stats")
    return out


def lm_head_stats(A, W, z_cur, row_seq, row_pos, z_prev, lse_prev, has_prev, lse_cur, mask_id,
                  kl_dir=0, cfg=-1):
    """LM head (bf16 A [M][K] x W [V][K]) storing logits into z_cur [B][N][V]
    at each row's (seq, pos) slot, with the vocabulary statistics computed in
    its epilogue; returns the same dict as vocab_stats()."""
    M, K = A.shape
    V = W.shape[0]
    B, N, _ = z_cur.shape
    dev = A.device
    out = dict(argmax=torch.empty(M, dtype=torch.int32, device=dev),
               conf=torch.empty(M, dtype=torch.float32, device=dev),
               kl=torch.empty(M, dtype=torch.float32, device=dev),
               has_kl=torch.empty(M, dtype=torch.int32, device=dev),
               lse=torch.empty(M, dtype=torch.float32, device=dev),
               err=torch.zeros(1, dtype=torch.int32, device=dev))
    need = int(L.lib().dlm_op_lm_head_stats_ws_bytes(M, V, K, cfg))
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    L.check(L.lib().dlm_op_lm_head_stats(M, V, K, _p(A), _p(W), _p(z_cur), _p(row_seq),
                                         _p(row_pos), N, mask_id, kl_dir, _p(z_prev),
                                         _p(lse_prev), _p(has_prev), _p(lse_cur),
                                         _p(out["argmax"]), _p(out["conf"]), _p(out["kl"]),
                                         _p(out["has_kl"]), _p(out["lse"]), _p(out["err"]), cfg,
                                         _p(ws), ws.numel(), _s()), "dlm_op_lm_head_stats")
    return out


def commit_lock(*, batch, seq_len, prompt_len, mask_id, blk_lo, blk_hi, k, do_commit, do_lock,
                policy, kl_eps, conf_tau, n_consec, lock_prompt, row_seq, row_pos, row_start,
                row_real, argmax, conf, kl, has_kl, tokens, bits, counters):
    L.check(L.lib().dlm_op_commit_lock(batch, seq_len, prompt_len, mask_id, blk_lo, blk_hi, k,
                                       do_commit, do_lock, policy, float(kl_eps), float(conf_tau),
                                       n_consec, lock_prompt, _p(row_seq), _p(row_pos),
                                       _p(row_start), _p(row_real), _p(argmax), _p(conf), _p(kl),
                                       _p(has_kl), _p(tokens), _p(bits), _p(counters), _s()),
            "dlm_op_commit_lock")


def slowfast_commit(*, batch, seq_len, mask_id, window, sf_k, sf_kmax, sf_whist, sf_tau_conv,
                    sf_tau_high, sf_var, row_pos, row_start, argmax, conf, tokens, frozen,
                    has_prev, sf_state):
    """One SlowFast commit decision per sequence on device arrays; tokens,
    frozen (int64 view of the uint64 bits), has_prev and sf_state are
    updated in place."""
    L.check(L.lib().dlm_op_slowfast_commit(batch, seq_len, mask_id, window, sf_k, sf_kmax,
                                           sf_whist, float(sf_tau_conv), float(sf_tau_high),
                                           float(sf_var), _p(row_pos), _p(row_start),
                                           _p(argmax), _p(conf), _p(tokens), _p(frozen),
                                           _p(has_prev), _p(sf_state), _s()),
            "dlm_op_slowfast_commit")
