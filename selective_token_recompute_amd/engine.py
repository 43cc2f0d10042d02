"""Python face of the engine: the C-ABI calls under their own names, plus a
small ``Engine`` that owns the torch buffers (weights, prompts, state block)
and the stream.  PyTorch is used only for device memory and streams; every
step of the computation runs in the library's kernels.
"""
from __future__ import annotations

import ctypes
from typing import Dict, List, Optional

import numpy as np
import torch

from . import _lib as L

_DT = {L.DLM_FP32: torch.float32, L.DLM_BF16: torch.bfloat16}


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


# ---- descriptors -------------------------------------------------------------

def model_desc(shape) -> L.dlm_model_desc:
    return L.dlm_model_desc(shape.n_layers, shape.d_model, shape.n_heads, shape.n_kv_heads,
                            shape.head_dim, shape.d_ff, shape.vocab, shape.mask_id,
                            float(shape.rope_base), float(shape.rms_eps),
                            L.DLM_BF16 if shape.bf16 else L.DLM_FP32)


# SlowFast sampler settings when the lock dict names none ([SF] §4 ablation:
# at most 8 exploratory steps, history window 2, variance threshold 1.0)
SF_DEFAULTS = dict(sf_k=1, sf_kmax=8, sf_whist=2, sf_tau_conv=0.9, sf_tau_high=0.9, sf_var=1.0)


def run_desc(run, lock: Dict) -> L.dlm_run_desc:
    pol = L.DLM_LOCK_TEST if lock["policy"] == "test" else L.DLM_LOCK_NONE
    smp = L.DLM_SAMPLER_SLOWFAST if lock.get("sampler") == "slowfast" else L.DLM_SAMPLER_SEMI_AR
    sf = {k: lock.get(k, v) for k, v in SF_DEFAULTS.items()}
    return L.dlm_run_desc(run.batch, run.seq_len, run.prompt_len, run.steps, run.block_len,
                          float(lock["kl_eps"]), float(lock["conf_tau"]), int(lock["n_consec"]),
                          int(lock.get("kl_dir", 0)), int(lock["lock_prompt_after_first_step"]),
                          pol, smp, int(sf["sf_k"]), int(sf["sf_kmax"]), int(sf["sf_whist"]),
                          float(sf["sf_tau_conv"]), float(sf["sf_tau_high"]), float(sf["sf_var"]),
                          int(lock.get("refresh_budget", 0)),
                          float(lock.get("refresh_eps", lock["kl_eps"])))


# ---- the C ABI under its own names ---------------------------------------------

def dlm_state_bytes(model: L.dlm_model_desc, run: L.dlm_run_desc) -> int:
    return int(L.lib().dlm_state_bytes(ctypes.byref(model), ctypes.byref(run)))


def dlm_step_init(model, weights: L.dlm_weights, run, prompt_ptr: int, state_ptr: int,
                  state_bytes: int, stream: int) -> ctypes.c_void_p:
    h = ctypes.c_void_p()
    L.check(L.lib().dlm_step_init(ctypes.byref(model), ctypes.byref(weights), ctypes.byref(run),
                                  prompt_ptr, state_ptr, state_bytes, stream, ctypes.byref(h)),
            "dlm_step_init")
    return h


def dlm_step(h) -> int:
    m = ctypes.c_int32(0)
    L.check(L.lib().dlm_step(h, ctypes.byref(m)), "dlm_step")
    return int(m.value)


def dlm_lock_update(h, ov: Optional[L.dlm_override] = None) -> None:
    L.check(L.lib().dlm_lock_update(h, ctypes.byref(ov) if ov is not None else None),
            "dlm_lock_update")


def dlm_get(h, what: int):
    p = ctypes.c_void_p()
    n = ctypes.c_int64()
    L.check(L.lib().dlm_get(h, what, ctypes.byref(p), ctypes.byref(n)), "dlm_get")
    return int(p.value or 0), int(n.value)


def dlm_checkpoint_bytes(h) -> int:
    return int(L.lib().dlm_checkpoint_bytes(h))


def dlm_checkpoint_save(h, dst_ptr: int, dst_bytes: int) -> None:
    L.check(L.lib().dlm_checkpoint_save(h, ctypes.c_void_p(dst_ptr), dst_bytes),
            "dlm_checkpoint_save")


def dlm_checkpoint_load(h, src_ptr: int, src_bytes: int) -> None:
    L.check(L.lib().dlm_checkpoint_load(h, ctypes.c_void_p(src_ptr), src_bytes),
            "dlm_checkpoint_load")


def _buffer(buf):
    """(address, bytes) of a C-contiguous numpy array or torch tensor."""
    if isinstance(buf, np.ndarray):
        if not buf.flags["C_CONTIGUOUS"]:
            raise ValueError("checkpoint buffer must be contiguous")
        return buf.ctypes.data, buf.nbytes
    if not buf.is_contiguous():
        raise ValueError("checkpoint buffer must be contiguous")
    return buf.data_ptr(), buf.numel() * buf.element_size()


def dlm_destroy(h) -> None:
    L.check(L.lib().dlm_destroy(h), "dlm_destroy")


def dlm_error_string(status: int) -> str:
    return L.error_string(status)


# ---- weights on the device -------------------------------------------------------

LAYER_KEYS = ["attn_norm", "w_qkv", "w_o", "ffn_norm", "w_gate", "w_up", "w_down"]


def upload_weights(W: Dict, shape, device="cuda") -> Dict:
    """Copies host float32 weights (bf16-representable for bf16 models) to
    device tensors of the model's storage type."""
    dt = torch.bfloat16 if shape.bf16 else torch.float32

    def up(a):
        return torch.from_numpy(a).to(device=device).to(dt).contiguous()

    return dict(tok_emb=up(W["tok_emb"]), final_norm=up(W["final_norm"]),
                lm_head=up(W["lm_head"]),
                layers=[{k: up(lay[k]) for k in LAYER_KEYS} for lay in W["layers"]])


def random_device_weights(shape, seed: int = 0, gain_std: float = 0.1, device="cuda") -> Dict:
    """Random-init weights drawn directly on the device (torch's generator,
    N(0, 0.02) matrices, gains 1 + gain_std N(0,1)); for timing runs at full
    size where a host copy would be wasteful."""
    dt = torch.bfloat16 if shape.bf16 else torch.float32
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    d, dff, V = shape.d_model, shape.d_ff, shape.vocab

    def mat(r, c):
        out = torch.empty((r, c), dtype=dt, device=device)
        step = max(1, (1 << 26) // c)
        for i in range(0, r, step):
            blk = torch.randn((min(step, r - i), c), generator=g, device=device) * 0.02
            out[i:i + blk.shape[0]] = blk.to(dt)
        return out

    def gain():
        return (1.0 + gain_std * torch.randn(d, generator=g, device=device)).to(dt)

    layers = []
    for _ in range(shape.n_layers):
        layers.append(dict(attn_norm=gain(), w_qkv=mat(shape.qkv_out, d),
                           w_o=mat(d, shape.n_heads * shape.head_dim), ffn_norm=gain(),
                           w_gate=mat(dff, d), w_up=mat(dff, d), w_down=mat(d, dff)))
    return dict(tok_emb=mat(V, d), final_norm=gain(), lm_head=mat(V, d), layers=layers)


def weights_desc(dw: Dict):
    """dlm_weights pointing at device tensors; returns (struct, keepalive)."""
    n = len(dw["layers"])
    arrs = {k: (ctypes.c_void_p * n)(*[lay[k].data_ptr() for lay in dw["layers"]])
            for k in LAYER_KEYS}
    P = ctypes.POINTER(ctypes.c_void_p)
    w = L.dlm_weights(dw["tok_emb"].data_ptr(), dw["final_norm"].data_ptr(),
                      dw["lm_head"].data_ptr(), *[ctypes.cast(arrs[k], P) for k in LAYER_KEYS])
    return w, arrs


class Engine:
    """One decoding run on the GPU through the C ABI."""

    def __init__(self, shape, dev_weights: Dict, run, lock: Dict, prompts: torch.Tensor,
                 stream: Optional[torch.cuda.Stream] = None, metrics_path: Optional[str] = None):
        """metrics_path: if given, every lock_update appends one JSON line
        {t, m_tot, m_b, commits, new_locks, locked, flops} to that file (the
        step's active rows per sequence, positions unmasked and locked by the
        update, locked positions in all, the step's algorithmic FLOPs); this
        reads small arrays back to the host each step."""
        self.shape, self.run, self.lock = shape, run, lock
        self.metrics_path = metrics_path
        self.device = prompts.device
        self.stream = stream
        self.dw = dev_weights
        self._m = model_desc(shape)
        self._r = run_desc(run, lock)
        self.state_bytes = dlm_state_bytes(self._m, self._r)
        if self.state_bytes == 0:
            raise ValueError("engine rejected the model/run descriptors")
        self.state = torch.empty(self.state_bytes, dtype=torch.uint8, device=self.device)
        self.prompts = prompts.to(torch.int32).contiguous()
        self._w, self._keep = weights_desc(dev_weights)
        self.h = dlm_step_init(self._m, self._w, self._r, self.prompts.data_ptr(),
                               self.state.data_ptr(), self.state_bytes, _stream(stream))
        self.t = 0
        self.m = None

    def close(self):
        if getattr(self, "h", None) is not None:
            dlm_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def step(self) -> int:
        self.m = dlm_step(self.h)
        return self.m

    def debug_poison(self) -> None:
        """dlm_debug_poison: NaN in every array a step writes before it reads
        (only before the first step)."""
        L.check(L.lib().dlm_debug_poison(self.h), "dlm_debug_poison")

    def checkpoint_bytes(self) -> int:
        return dlm_checkpoint_bytes(self.h)

    def save_checkpoint(self, out=None):
        """dlm_checkpoint_save at a step boundary into `out` (a contiguous
        numpy array or torch tensor, host or device, of at least
        checkpoint_bytes()); without `out` a new host uint8 array is
        returned."""
        if out is None:
            out = np.empty(self.checkpoint_bytes(), dtype=np.uint8)
        dlm_checkpoint_save(self.h, *_buffer(out))
        return out

    def load_checkpoint(self, buf) -> None:
        """dlm_checkpoint_load from an image written by save_checkpoint of a
        handle with the same model and run descriptors."""
        dlm_checkpoint_load(self.h, *_buffer(buf))

    def lock_update(self, commits=None, lock_bits=None, counters=None) -> None:
        """commits: (seq, pos, tok) int sequences replacing the top-k choice;
        lock_bits: uint64 numpy [B][W] ORed in instead of the lock test;
        counters: int32 numpy [B][N] (with lock_bits)."""
        if self.metrics_path:
            tok0 = self.tokens().clone()
            bits0 = self.lock_bits().clone()
        if commits is None and lock_bits is None:
            dlm_lock_update(self.h, None)
        else:
            import numpy as np
            keep = []

            def arr(a, dt):
                a = np.ascontiguousarray(a, dtype=dt)
                keep.append(a)
                return a.ctypes.data

            ov = L.dlm_override(None, None, None, -1, None, None)
            if commits is not None:
                ov.commit_seq = arr(commits[0], np.int32)
                ov.commit_pos = arr(commits[1], np.int32)
                ov.commit_tok = arr(commits[2], np.int32)
                ov.n_commit = len(commits[0])
            if lock_bits is not None:
                ov.lock_bits = arr(lock_bits, np.uint64)
                if counters is not None:
                    ov.counters = arr(counters, np.int32)
            dlm_lock_update(self.h, ov)
        if self.metrics_path:
            self._write_metrics(tok0, bits0)
        self.t += 1

    def _write_metrics(self, tok0: torch.Tensor, bits0: torch.Tensor) -> None:
        import json

        import numpy as np

        def nbits(b: torch.Tensor) -> int:
            return int(np.unpackbits(b.cpu().numpy().view(np.uint8)).sum())

        step, m, flops = self.last_step_info()
        rs = self.rows()[0][:m].cpu().numpy() if m else np.zeros(0, np.int32)
        bits1 = self.lock_bits()
        rec = dict(t=step, m_tot=m, m_b=np.bincount(rs, minlength=self.run.batch).tolist(),
                   commits=int((self.tokens() != tok0).sum().item()),
                   new_locks=nbits(bits1 & ~bits0), locked=nbits(bits1), flops=flops)
        with open(self.metrics_path, "a") as f:
            f.write(json.dumps(rec) + "\n")

    def _view(self, what: int, dtype: torch.dtype, shape=None) -> torch.Tensor:
        p, n = dlm_get(self.h, what)
        off = p - self.state.data_ptr()
        nbytes = n * torch.tensor([], dtype=dtype).element_size()
        t = self.state[off:off + nbytes].view(dtype)
        return t.view(*shape) if shape is not None else t

    def tokens(self) -> torch.Tensor:
        return self._view(L.DLM_GET_TOKENS, torch.int32, (self.run.batch, self.run.seq_len))

    def lock_bits(self) -> torch.Tensor:
        return self._view(L.DLM_GET_LOCK_BITS, torch.int64,
                          (self.run.batch, (self.run.seq_len + 63) // 64))

    def counters(self) -> torch.Tensor:
        return self._view(L.DLM_GET_COUNTERS, torch.int32, (self.run.batch, self.run.seq_len))

    def frozen_bits(self) -> torch.Tensor:
        return self._view(L.DLM_GET_FROZEN, torch.int64,
                          (self.run.batch, (self.run.seq_len + 63) // 64))

    def sf_state(self) -> torch.Tensor:
        return self._view(L.DLM_GET_SF_STATE, torch.int32, (self.run.batch, L.SF_STATE_INTS))

    def has_prev(self) -> torch.Tensor:
        return self._view(L.DLM_GET_HAS_PREV, torch.int32, (self.run.batch, self.run.seq_len))

    def drift(self) -> torch.Tensor:
        return self._view(L.DLM_GET_DRIFT, torch.float32, (self.run.batch, self.run.seq_len))

    def refresh_bits(self) -> torch.Tensor:
        return self._view(L.DLM_GET_REFRESH, torch.int64,
                          (self.run.batch, (self.run.seq_len + 63) // 64))

    def rows(self):
        return (self._view(L.DLM_GET_ROW_SEQ, torch.int32),
                self._view(L.DLM_GET_ROW_POS, torch.int32),
                self._view(L.DLM_GET_ROW_REAL, torch.int32))

    def stats(self) -> Dict[str, torch.Tensor]:
        return dict(argmax=self._view(L.DLM_GET_ARGMAX, torch.int32),
                    conf=self._view(L.DLM_GET_CONF, torch.float32),
                    kl=self._view(L.DLM_GET_KL, torch.float32),
                    has_kl=self._view(L.DLM_GET_HAS_KL, torch.int32),
                    lse=self._view(L.DLM_GET_LSE, torch.float32))

    def logits(self) -> torch.Tensor:
        """float [B][N][V]; rows of the last step's active positions are valid."""
        return self._view(L.DLM_GET_LOGITS, torch.float32,
                          (self.run.batch, self.run.seq_len, self.shape.vocab))

    def kv_cache(self):
        """K [L][B][nkv][N][hd] and V transposed [L][B][nkv][hd][N]."""
        sh = (self.shape.n_layers, self.run.batch, self.shape.n_kv_heads, self.run.seq_len,
              self.shape.head_dim)
        sht = sh[:3] + (sh[4], sh[3])
        dt = torch.bfloat16 if self.shape.bf16 else torch.float32
        return self._view(L.DLM_GET_KCACHE, dt, sh), self._view(L.DLM_GET_VCACHE, dt, sht)

    def last_step_info(self):
        s = ctypes.c_int32()
        m = ctypes.c_int32()
        f = ctypes.c_double()
        L.check(L.lib().dlm_last_step_info(self.h, ctypes.byref(s), ctypes.byref(m),
                                           ctypes.byref(f)), "dlm_last_step_info")
        return int(s.value), int(m.value), float(f.value)

    def set_timing(self, on: bool) -> None:
        L.check(L.lib().dlm_set_timing(self.h, 1 if on else 0), "dlm_set_timing")

    def read_timing(self) -> Dict[str, Dict[str, float]]:
        out = {}
        for c, name in enumerate(L.KCLASSES):
            ms = ctypes.c_double()
            n = ctypes.c_int64()
            by = ctypes.c_double()
            fl = ctypes.c_double()
            L.check(L.lib().dlm_read_timing(self.h, c, ctypes.byref(ms), ctypes.byref(n),
                                            ctypes.byref(by), ctypes.byref(fl)),
                    "dlm_read_timing")
            out[name] = dict(ms=ms.value, launches=n.value, bytes=by.value, flops=fl.value)
        return out
