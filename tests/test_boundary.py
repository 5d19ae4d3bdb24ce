"""CPU tests of the C-ABI boundary: the library loads, exports every function
include/gptmi.h declares, and rejects invalid arguments with the documented
status before any GPU work (so these run without a GPU)."""
import ctypes
import os
import subprocess

import pytest

from decoder_only_gpt_bf16_amd import binding as B
from decoder_only_gpt_bf16_amd import synth


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(B.LIB_PATH):
        from decoder_only_gpt_bf16_amd.build import build
        build(verbose=False)
    return B.lib()


def test_exports_every_declared_symbol(L):
    names = B.header_functions()
    assert {"gpt_block_fwd", "gpt_block_bwd", "lm_head_xent_fwd_bwd", "val_bpb_reduce"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        assert hasattr(L, n)


def test_status_strings(L):
    assert L.gpt_status_string(0) == b"ok"
    assert L.gpt_status_string(3) == b"workspace too small"
    assert L.gpt_status_string(99) == b"unknown status"


FAKE = 0x10000   # 16-byte aligned, never dereferenced: validation fails first


def _weights(cfg, ptr=FAKE):
    d = {f: ptr for f in B.BLOCK_FIELDS}
    if not cfg.bias:
        for f in ("ln1_b", "b_qkv", "b_o", "ln2_b", "b_fc", "b_proj"):
            d[f] = None
    if cfg.norm != "layernorm":
        d["ln1_w"] = d["ln2_w"] = d["ln1_b"] = d["ln2_b"] = None
    return B.BlockWeightsC(*[d[f] for f in B.BLOCK_FIELDS])


def _fwd(L, c, Bsz, T, w, x=FAKE, y=FAKE, saved=FAKE, ws=FAKE, nbytes=1 << 40):
    return L.gpt_block_fwd(ctypes.byref(c) if c is not None else None, Bsz, T, x, ctypes.byref(w), y, saved, ws,
                           nbytes, None)


def test_block_fwd_validation(L):
    cfg = synth.D20_BLOCK.cfg
    c = B.make_config(cfg)
    w = _weights(cfg)
    assert _fwd(L, None, 1, 1, w) == B.GPT_ERR_INVALID
    assert b"cfg" in L.gpt_last_error()
    assert _fwd(L, c, 0, 16, w) == B.GPT_ERR_INVALID
    assert _fwd(L, c, 1, 0, w) == B.GPT_ERR_INVALID
    assert _fwd(L, c, 1, 4096, w) == B.GPT_ERR_INVALID          # T > block_size
    assert b"block_size" in L.gpt_last_error()
    assert _fwd(L, c, 1, 16, w, x=None) == B.GPT_ERR_INVALID
    assert _fwd(L, c, 1, 16, w, x=FAKE + 4) == B.GPT_ERR_INVALID  # misaligned
    assert _fwd(L, c, 1, 16, w, saved=None, nbytes=1) == B.GPT_ERR_WORKSPACE  # inference keeps intermediates there
    bad = _weights(cfg)
    bad.w_fc = None
    assert _fwd(L, c, 1, 16, bad) == B.GPT_ERR_INVALID


def test_config_validation(L):
    base = synth.D20_BLOCK.cfg
    import dataclasses
    w = _weights(base)
    for changes, code in [(dict(n_head=3), B.GPT_ERR_INVALID),          # 1280 % 3
                          (dict(n_head=1), B.GPT_ERR_UNSUPPORTED),      # head_dim 1280
                          (dict(n_embd=1280 + 10, n_head=10), B.GPT_ERR_INVALID),  # odd head_dim 129 with rope
                          (dict(n_embd=30, n_head=1), B.GPT_ERR_UNSUPPORTED)]:
        c = B.make_config(dataclasses.replace(base, **changes))
        assert _fwd(L, c, 1, 16, w) == code, changes
    c = B.make_config(base)
    c.dtype = 7
    assert _fwd(L, c, 1, 16, w) == B.GPT_ERR_UNSUPPORTED
    c = B.make_config(base)
    c.norm = 5
    assert _fwd(L, c, 1, 16, w) == B.GPT_ERR_INVALID
    c = B.make_config(dataclasses.replace(base, n_embd=1280 + 20, n_head=10))   # head_dim 130: not multiple of 8
    assert _fwd(L, c, 1, 16, w) == B.GPT_ERR_UNSUPPORTED


def test_gpt2_form_needs_biases_and_gains(L):
    cfg = synth.GPT2_BLOCK.cfg
    c = B.make_config(cfg)
    w = _weights(cfg)
    w.b_o = None
    assert _fwd(L, c, 1, 16, w) == B.GPT_ERR_INVALID
    w = _weights(cfg)
    w.ln2_w = None
    assert _fwd(L, c, 1, 16, w) == B.GPT_ERR_INVALID


def test_block_bwd_validation(L):
    cfg = synth.GPT2_BLOCK.cfg
    c = B.make_config(cfg)
    w = _weights(cfg)
    g = B.BlockGradsC(*[FAKE] * 12)
    args = lambda **k: [ctypes.byref(c), k.get("B", 1), k.get("T", 16), k.get("x", FAKE), k.get("dy", FAKE),  # noqa
                        ctypes.byref(w), k.get("saved", FAKE), k.get("dx", FAKE), ctypes.byref(k.get("g", g)), 0,
                        FAKE, k.get("nb", 1 << 40), None]
    assert L.gpt_block_bwd(*args(saved=None)) == B.GPT_ERR_INVALID
    assert L.gpt_block_bwd(*args(dy=None)) == B.GPT_ERR_INVALID
    assert L.gpt_block_bwd(*args(nb=10)) == B.GPT_ERR_WORKSPACE
    g2 = B.BlockGradsC(*[FAKE] * 12)
    g2.b_fc = None
    assert L.gpt_block_bwd(*args(g=g2)) == B.GPT_ERR_INVALID


def test_lm_head_and_bpb_validation(L):
    c = B.make_config(synth.GPT2_STEP.cfg)
    f = L.lm_head_xent_fwd_bwd
    assert f(ctypes.byref(c), 0, FAKE, FAKE, FAKE, 1.0, FAKE, None, None, None, 0, FAKE, 1 << 40, None) == \
        B.GPT_ERR_INVALID
    assert f(ctypes.byref(c), 16, None, FAKE, FAKE, 1.0, FAKE, None, None, None, 0, FAKE, 1 << 40, None) == \
        B.GPT_ERR_INVALID
    assert f(ctypes.byref(c), 16, FAKE, FAKE, FAKE, 1.0, FAKE, None, None, None, 0, FAKE, 100, None) == \
        B.GPT_ERR_WORKSPACE
    assert L.val_bpb_reduce(0, FAKE, FAKE, FAKE, 10, FAKE, FAKE, None) == B.GPT_ERR_INVALID
    assert L.val_bpb_reduce(10, FAKE, FAKE, None, 10, FAKE, FAKE, None) == B.GPT_ERR_INVALID
    assert L.val_bpb_reduce(10, FAKE, FAKE, FAKE, 0, FAKE, FAKE, None) == B.GPT_ERR_INVALID


def test_embed_and_norm_validation(L):
    c = B.make_config(synth.GPT2_STEP.cfg)
    assert L.gpt_embed_fwd(ctypes.byref(c), 1, 16, FAKE, FAKE, None, FAKE, None) == B.GPT_ERR_INVALID  # no wpe
    assert L.gpt_embed_bwd(ctypes.byref(c), 1, 16, FAKE, FAKE, FAKE, None, 0, FAKE, 8, None) == B.GPT_ERR_WORKSPACE
    assert L.gpt_norm_fwd(ctypes.byref(c), 16, FAKE, None, None, FAKE, None, None) == B.GPT_ERR_INVALID  # LN gain
    assert L.gpt_norm_bwd(ctypes.byref(c), 0, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, 0, FAKE, 1 << 30, None) == \
        B.GPT_ERR_INVALID


def test_sizes(L):
    for w in synth.WORKLOADS:
        c = B.make_config(w.cfg)
        sb = B.gpt_block_saved_bytes(c, w.B, w.T)
        ws = B.gpt_workspace_bytes(c, w.B, w.T)
        N, C, es = w.B * w.T, w.cfg.n_embd, 2 if w.cfg.dtype == "bf16" else 4
        # a1, qkv, o, x1, a2, u, g: 14 C values per token in storage type
        assert sb >= 14 * N * C * es
        assert ws > 0 and ws % 256 == 0
    c = B.make_config(synth.D20_BLOCK.cfg)
    assert B.gpt_block_saved_bytes(c, 1, 4096) == 0
    assert B.gpt_workspace_bytes(c, 0, 16) == 0


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(B, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        B.lib()


def test_adamw_validation_without_gpu():
    """Argument checks run before any launch, so fake aligned addresses do."""
    import ctypes
    L = B.lib()
    t = (B.AdamwTensorC * 2)()
    t[0] = B.AdamwTensorC(16, 32, 48, 64, None, 100, 1)
    t[1] = B.AdamwTensorC(80, 96, 112, 128, 144, 5, 0)
    need = L.gpt_adamw_workspace_bytes(t, 2)
    assert need >= 2 * 8
    ok = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=1, max_norm=1.0)

    def call(cfg=None, count=2, ws=256, nbytes=None, tensors=t):
        c = B.AdamwConfigC(**{**ok, **(cfg or {})})
        return L.gpt_adamw_step(ctypes.byref(c), tensors, count, None, ws, need if nbytes is None else nbytes, None)

    assert call({"step": 0}) == B.GPT_ERR_INVALID
    assert call({"beta1": 1.0}) == B.GPT_ERR_INVALID
    assert call({"lr": float("nan")}) == B.GPT_ERR_INVALID
    assert call({"eps": -1.0}) == B.GPT_ERR_INVALID
    assert call(count=0) == B.GPT_ERR_INVALID
    assert call(nbytes=need - 1) == B.GPT_ERR_WORKSPACE
    assert call(ws=0) == B.GPT_ERR_WORKSPACE
    bad = (B.AdamwTensorC * 1)()
    bad[0] = B.AdamwTensorC(17, 32, 48, 64, None, 100, 1)
    assert call(count=1, tensors=bad) == B.GPT_ERR_INVALID
    bad[0] = B.AdamwTensorC(16, 32, 48, 64, None, 0, 1)
    assert call(count=1, tensors=bad) == B.GPT_ERR_INVALID
    bad[0] = B.AdamwTensorC(16, None, 48, 64, None, 4, 1)
    assert call(count=1, tensors=bad) == B.GPT_ERR_INVALID


def test_operand_limit_refused_before_launch(L):
    """The largest block operand, [B*T, 4C], must stay below 2 GiB (31-bit
    buffer offsets).  A batch beyond it is refused as UNSUPPORTED by the
    validation that runs before any launch (here without a GPU, so any launch
    would have failed with a HIP error instead), and the sizing queries
    return 0 for it."""
    cfg = synth.D20_BLOCK.cfg   # C = 1280, block_size 2048: the limit falls between B = 102 and 103
    c = B.make_config(cfg)
    w = _weights(cfg)
    assert 102 * 2048 * 4 * 1280 * 2 < 2 ** 31 <= 103 * 2048 * 4 * 1280 * 2
    assert B.gpt_block_saved_bytes(c, 102, 2048) > 0
    assert B.gpt_block_saved_bytes(c, 103, 2048) == 0
    assert B.gpt_workspace_bytes(c, 103, 2048) == 0
    assert _fwd(L, c, 103, 2048, w) == B.GPT_ERR_UNSUPPORTED
    assert b"2 GiB" in L.gpt_last_error()
    g = B.BlockGradsC(*[FAKE] * 12)
    for f in ("ln1_w", "ln1_b", "b_qkv", "b_o", "ln2_w", "ln2_b", "b_fc", "b_proj"):
        setattr(g, f, None)
    assert L.gpt_block_bwd(ctypes.byref(c), 103, 2048, FAKE, FAKE, ctypes.byref(w), FAKE, FAKE, ctypes.byref(g), 0,
                           FAKE, 1 << 40, None) == B.GPT_ERR_UNSUPPORTED
    assert L.gpt_embed_fwd(ctypes.byref(c), 103, 2048, FAKE, FAKE, None, FAKE, None) == B.GPT_ERR_UNSUPPORTED
    # the LM head: a logit chunk [N, 8192] bf16 reaches 2 GiB at N = 131072
    f = L.lm_head_xent_fwd_bwd
    assert f(ctypes.byref(c), 131072, FAKE, FAKE, FAKE, 1.0, FAKE, None, None, None, 0, FAKE, 1 << 40, None) == \
        B.GPT_ERR_UNSUPPORTED
    assert f(ctypes.byref(c), 131071, FAKE, FAKE, FAKE, 1.0, FAKE, None, None, None, 0, FAKE, 100, None) == \
        B.GPT_ERR_WORKSPACE
