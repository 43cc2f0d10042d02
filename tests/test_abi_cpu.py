"""C-ABI checks that need no GPU: the library loads, exports every function
the headers declare, sizes its state, and rejects invalid arguments on the
host before any launch."""
import ctypes
import os
import re

import pytest

import synth
from selective_token_recompute_amd import _lib as L
from selective_token_recompute_amd import engine as E

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for h in ("dlm.h", "dlm_ops.h"):
        src = open(os.path.join(ROOT, "include", h)).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names |= set(re.findall(r"\b(dlm_[a-z_]+)\s*\(", src))
    return names


def test_library_exports_every_declared_symbol():
    lib = L.lib()
    declared = _declared()
    assert len(declared) >= 20
    missing = [n for n in sorted(declared) if not hasattr(lib, n)]
    assert not missing, missing
    assert set(L.EXPORTS) == declared


def test_error_strings():
    for s in (0, -1, -2, -3, -4, -5, -6):
        assert L.error_string(s)
    assert L.error_string(-99) == "unknown status"


def _descs(cfg="llada8b", setting="natural"):
    shape, run = synth.CONFIGS[cfg]
    return E.model_desc(shape), E.run_desc(run, synth.LOCK_SETTINGS[setting])


def test_state_bytes_sizes():
    m, r = _descs()
    n = E.dlm_state_bytes(m, r)
    shape, run = synth.CONFIGS["llada8b"]
    BN = run.batch * run.seq_len
    kv = 2 * shape.n_layers * BN * shape.n_kv_heads * shape.head_dim * 2
    z = 2 * BN * shape.vocab * 4
    assert n >= kv + z and n % 256 == 0
    m, r = _descs("tiny")
    assert 0 < E.dlm_state_bytes(m, r) < (64 << 20) + (8 << 20)


@pytest.mark.parametrize("field,value", [
    ("n_layers", 0), ("head_dim", 7), ("head_dim", 512), ("n_kv_heads", 3), ("vocab", 1),
    ("mask_id", 126464), ("mask_id", -1), ("dtype", 5)])
def test_invalid_model_rejected(field, value):
    m, r = _descs()
    setattr(m, field, value)
    assert E.dlm_state_bytes(m, r) == 0


@pytest.mark.parametrize("field,value", [
    ("batch", 0), ("batch", 2000), ("seq_len", 0), ("prompt_len", 600), ("steps", 0),
    ("block_len", 0), ("n_consec", 0), ("kl_dir", 2), ("lock_policy", 3),
    ("kl_eps", float("nan"))])
def test_invalid_run_rejected(field, value):
    m, r = _descs()
    setattr(r, field, value)
    assert E.dlm_state_bytes(m, r) == 0


@pytest.mark.parametrize("field,value", [
    ("sampler", 2), ("sf_k", 0), ("sf_kmax", 0), ("sf_whist", 0), ("sf_whist", 9),
    ("sf_tau_conv", float("nan")), ("sf_tau_high", float("nan")), ("sf_var", float("nan"))])
def test_invalid_slowfast_run_rejected(field, value):
    shape, run = synth.CONFIGS["llada8b"]
    m, r = E.model_desc(shape), E.run_desc(run, synth.LOCK_SETTINGS["slowfast"])
    assert E.dlm_state_bytes(m, r) > 0
    setattr(r, field, value)
    assert E.dlm_state_bytes(m, r) == 0


def test_slowfast_sequence_limit():
    # the commit kernel stages a sequence's candidates in LDS: seq_len <= 4096
    import dataclasses
    shape, run = synth.CONFIGS["longctx"]
    lock = synth.LOCK_SETTINGS["slowfast"]
    assert E.dlm_state_bytes(E.model_desc(shape), E.run_desc(run, lock)) > 0
    big = dataclasses.replace(run, seq_len=4160)
    assert E.dlm_state_bytes(E.model_desc(shape), E.run_desc(big, lock)) == 0
    # the semi-autoregressive sampler has no such limit
    assert E.dlm_state_bytes(E.model_desc(shape),
                             E.run_desc(big, synth.LOCK_SETTINGS["natural"])) > 0


def test_steps_fewer_than_blocks_rejected():
    shape, run = synth.CONFIGS["longctx"]
    import dataclasses
    bad = dataclasses.replace(run, steps=11)  # 12 blocks need >= 12 steps
    assert E.dlm_state_bytes(E.model_desc(shape), E.run_desc(bad, synth.LOCK_SETTINGS["natural"])) == 0


def test_step_init_rejects_bad_arguments_without_launching():
    m, r = _descs("tiny")
    lib = L.lib()
    h = ctypes.c_void_p()
    w = L.dlm_weights()  # all NULL
    buf = (ctypes.c_uint8 * 512)()
    st = lib.dlm_step_init(ctypes.byref(m), ctypes.byref(w), ctypes.byref(r), None,
                           ctypes.addressof(buf), 512, None, ctypes.byref(h))
    assert st == L.DLM_E_INVALID and not h.value
    assert lib.dlm_step_init(None, None, None, None, None, 0, None, None) == L.DLM_E_INVALID


def test_null_handle_calls():
    lib = L.lib()
    assert lib.dlm_step(None, None) == L.DLM_E_INVALID
    assert lib.dlm_lock_update(None, None) == L.DLM_E_INVALID
    p = ctypes.c_void_p()
    n = ctypes.c_int64()
    assert lib.dlm_get(None, 0, ctypes.byref(p), ctypes.byref(n)) == L.DLM_E_INVALID
    assert lib.dlm_destroy(None) == L.DLM_E_INVALID
    assert lib.dlm_set_timing(None, 1) == L.DLM_E_INVALID
    assert lib.dlm_checkpoint_bytes(None) == 0
    buf = ctypes.create_string_buffer(64)
    assert lib.dlm_checkpoint_save(None, buf, 64) == L.DLM_E_INVALID
    assert lib.dlm_checkpoint_load(None, buf, 64) == L.DLM_E_INVALID


def test_op_argument_validation():
    lib = L.lib()
    assert lib.dlm_op_gemm(7, 0, 4, 4, 4, None, None, None, None, None, None, 0, 0, None, 0,
                           None) == L.DLM_E_INVALID
    assert lib.dlm_op_gemm(1, 0, -1, 4, 4, None, None, None, None, None, None, 0, 0, None, 0,
                           None) == L.DLM_E_INVALID
    assert lib.dlm_op_gemm(1, 9, 4, 4, 4, None, None, None, None, None, None, 0, 0, None, 0,
                           None) == L.DLM_E_INVALID
    # M = 0 is a no-op that never touches the device
    assert lib.dlm_op_gemm(1, 0, 0, 4, 4, None, None, None, None, None, None, 0, 0, None, 0,
                           None) == L.DLM_OK
    assert lib.dlm_op_attention(1, 4, 1, 8, 4, 3, 128, None, None, None, None, None, None, 0,
                                None) == L.DLM_E_INVALID
    assert lib.dlm_op_compact(None, 1, 8, None, None, None, None, None, None) == L.DLM_E_INVALID
    assert lib.dlm_op_commit_lock(1, 8, 2, 15, 6, 2, 1, 1, 1, 1, 0.0, 0.0, 1, 0,
                                  *([None] * 11), None) == L.DLM_E_INVALID
    # slowfast_commit: null arrays, then bad sizes with (dummy) non-null arrays
    assert lib.dlm_op_slowfast_commit(1, 8, 7, 4, 1, 8, 2, 0.5, 0.9, 1.0,
                                      *([None] * 8), None) == L.DLM_E_INVALID
    buf = (ctypes.c_uint8 * 64)()
    p = ctypes.addressof(buf)
    for args in [(1, 5000, 7, 4, 1, 8, 2), (1, 8, 7, 0, 1, 8, 2), (1, 8, 7, 4, 0, 8, 2),
                 (1, 8, 7, 4, 1, 8, 9), (0, 8, 7, 4, 1, 8, 2)]:
        assert lib.dlm_op_slowfast_commit(*args, 0.5, 0.9, 1.0, *([p] * 8),
                                          None) == L.DLM_E_INVALID


def test_workspace_queries():
    # small M splits K (weight streaming), large M does not
    assert L.lib().dlm_op_gemm_ws_bytes(1, 0, 8, 4096, 4096) > 0
    assert L.lib().dlm_op_gemm_ws_bytes(1, 0, 1024, 12288, 4096) == 0
    assert L.lib().dlm_op_gemm_ws_bytes(0, 0, 8, 4096, 4096) == 0  # fp32 path: no split
    assert L.lib().dlm_op_vocab_ws_bytes(384, 126464) > 0
    # attention splits the keys (combine pass) only from N = 1024 at small M
    assert L.lib().dlm_op_attention_ws_bytes(1, 20, 1, 1024, 32, 32, 128) > 0
    assert L.lib().dlm_op_attention_ws_bytes(1, 1, 1, 512, 32, 32, 128) == 0
    assert L.lib().dlm_op_attention_ws_bytes(1, 1024, 1, 1024, 32, 32, 128) == 0


@pytest.mark.parametrize("field,value", [
    ("refresh_budget", -1), ("refresh_budget", 513), ("refresh_eps", float("nan")),
    ("sampler", 1)])
def test_invalid_refresh_run_rejected(field, value):
    # the drift-aware refresh needs the semi-AR sampler, 0 <= budget <= seq_len
    shape, run = synth.CONFIGS["llada8b"]
    m, r = E.model_desc(shape), E.run_desc(run, synth.LOCK_SETTINGS["refresh"])
    assert r.refresh_budget == 8 and E.dlm_state_bytes(m, r) > 0
    setattr(r, field, value)
    assert E.dlm_state_bytes(m, r) == 0


def test_refresh_sequence_limit():
    # the selection stages a sequence's locked positions in LDS: seq_len <= 4096
    import dataclasses
    shape, run = synth.CONFIGS["longctx"]
    lock = synth.LOCK_SETTINGS["refresh"]
    assert E.dlm_state_bytes(E.model_desc(shape), E.run_desc(run, lock)) > 0
    big = dataclasses.replace(run, seq_len=4160)
    assert E.dlm_state_bytes(E.model_desc(shape), E.run_desc(big, lock)) == 0
    assert E.dlm_state_bytes(E.model_desc(shape),
                             E.run_desc(big, dict(lock, refresh_budget=0))) > 0
