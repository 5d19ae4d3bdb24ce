"""Whole-model training step and val-bpb evaluation assembled from C-ABI calls.

Torch allocates device memory; every arithmetic step is one of the library's
entry points (embedding, blocks, final norm, LM head + cross-entropy,
bits-per-byte).  Layout of one step ("nanoGPT — Karpathy's minimal GPT
pretraining repo", model.py: wte (+ wpe) -> n_layer blocks -> final norm ->
lm_head, tied to wte; train.py: loss = mean cross-entropy on shifted
targets, then backward).
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding as B
from .synth import bf16_bits

_TORCH_DTYPE = {"bf16": torch.bfloat16, "fp32": torch.float32}


def upload(a, dtype: str, device="cuda"):
    """float64 array of storage-representable values -> device tensor (exact)."""
    if a is None:
        return None
    if dtype == "bf16":
        bits = bf16_bits(np.asarray(a))
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.asarray(a, dtype=np.float32)).to(device)


def upload_i32(a, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


def to_f64(t) -> np.ndarray:
    return t.detach().float().cpu().double().numpy()


def workspace(cfg_c, Bsz, T, device="cuda"):
    n = B.gpt_workspace_bytes(cfg_c, Bsz, T)
    if n == 0:
        raise B.GptError(B.GPT_ERR_INVALID, B.lib().gpt_last_error().decode())
    return torch.empty(n, dtype=torch.uint8, device=device)


class BlockRunner:
    """One block fwd+bwd on device buffers (the single-block workloads)."""

    def __init__(self, cfg, Bsz, T, x, dy, params: dict, device="cuda"):
        self.cfg, self.B, self.T = cfg, Bsz, T
        self.c = B.make_config(cfg)
        dt = cfg.dtype
        self.x = upload(x.reshape(Bsz * T, -1), dt, device)
        self.dy = upload(dy.reshape(Bsz * T, -1), dt, device)
        self.w = {k: upload(v, dt, device) for k, v in params.items()}
        self.y = torch.empty_like(self.x)
        self.dx = torch.empty_like(self.x)
        self.saved = torch.empty(B.gpt_block_saved_bytes(self.c, Bsz, T), dtype=torch.uint8, device=device)
        self.ws = workspace(self.c, Bsz, T, device)
        self.g = {k: (None if v is None else torch.zeros(v.shape, dtype=torch.float32, device=device))
                  for k, v in params.items()}

    def forward(self, saved=True):
        B.gpt_block_fwd(self.c, self.B, self.T, self.x, self.w, self.y, self.saved if saved else None, self.ws)

    def backward(self, accumulate=0):
        B.gpt_block_bwd(self.c, self.B, self.T, self.x, self.dy, self.w, self.saved, self.dx, self.g, accumulate,
                        self.ws)

    def step(self):
        self.forward()
        self.backward()


class ModelRunner:
    """Full model: training step (fwd + bwd) or forward-only nats for val bpb."""

    def __init__(self, cfg, Bsz, T, P: dict, token_bytes=None, device="cuda", train=True):
        self.cfg, self.B, self.T, self.N = cfg, Bsz, T, Bsz * T
        self.c = B.make_config(cfg)
        dt = cfg.dtype
        up = lambda a: upload(a, dt, device)  # noqa: E731
        self.wte = up(P["wte"])
        self.wpe = up(P.get("wpe"))
        self.blocks = [{k: up(v) for k, v in bp.items()} for bp in P["blocks"]]
        self.lnf_w, self.lnf_b = up(P.get("lnf_w")), up(P.get("lnf_b"))
        self.lm_head = up(P.get("lm_head"))
        L, C, N = len(self.blocks), cfg.n_embd, self.N
        tdt = _TORCH_DTYPE[dt]
        self.xs = [torch.empty((N, C), dtype=tdt, device=device) for _ in range(L + 1)]
        self.hf = torch.empty((N, C), dtype=tdt, device=device)
        self.ws = workspace(self.c, Bsz, T, device)
        self.loss = torch.zeros(1, dtype=torch.float32, device=device)
        self.nats = torch.zeros(N, dtype=torch.float32, device=device)
        self.token_bytes = None if token_bytes is None else upload_i32(token_bytes, device)
        self.sum_nats = torch.zeros(1, dtype=torch.float64, device=device)
        self.sum_bytes = torch.zeros(1, dtype=torch.int64, device=device)
        self.train = train
        if train:
            sb = B.gpt_block_saved_bytes(self.c, Bsz, T)
            self.saved = [torch.empty(sb, dtype=torch.uint8, device=device) for _ in range(L)]
            f32 = lambda a: None if a is None else torch.zeros(a.shape, dtype=torch.float32, device=device)  # noqa
            self.g_blocks = [{k: f32(v) for k, v in bp.items()} for bp in P["blocks"]]
            self.g_wte = f32(P["wte"])
            self.g_wpe = f32(P.get("wpe"))
            self.g_lnf_w, self.g_lnf_b = f32(P.get("lnf_w")), f32(P.get("lnf_b"))
            self.g_lm_head = f32(P.get("lm_head"))
            self.dh = torch.empty((N, C), dtype=tdt, device=device)
            self.dxa = torch.empty((N, C), dtype=tdt, device=device)
            self.dxb = torch.empty((N, C), dtype=tdt, device=device)

    def set_batch(self, ids, targets):
        self.ids = upload_i32(ids.reshape(-1))
        self.tgt = upload_i32(targets.reshape(-1))

    def _head_weight(self):
        return self.lm_head if self.lm_head is not None else self.wte

    def train_step(self):
        c, Bsz, T, N = self.c, self.B, self.T, self.N
        B.gpt_embed_fwd(c, Bsz, T, self.ids, self.wte, self.wpe, self.xs[0])
        for l, bp in enumerate(self.blocks):
            B.gpt_block_fwd(c, Bsz, T, self.xs[l], bp, self.xs[l + 1], self.saved[l], self.ws)
        B.gpt_norm_fwd(c, N, self.xs[-1], self.lnf_w, self.lnf_b, self.hf, None)
        tied = self.lm_head is None
        B.lm_head_xent_fwd_bwd(c, N, self.hf, self._head_weight(), self.tgt, 1.0 / N, self.loss, self.nats,
                               self.dh, self.g_wte if tied else self.g_lm_head, 0, self.ws)
        B.gpt_norm_bwd(c, N, self.xs[-1], self.lnf_w, self.dh, None, self.dxa, self.g_lnf_w, self.g_lnf_b, 0,
                       self.ws)
        cur, nxt = self.dxa, self.dxb
        for l in range(len(self.blocks) - 1, -1, -1):
            B.gpt_block_bwd(c, Bsz, T, self.xs[l], cur, self.blocks[l], self.saved[l], nxt, self.g_blocks[l], 0,
                            self.ws)
            cur, nxt = nxt, cur
        self.dx0 = cur
        B.gpt_embed_bwd(c, Bsz, T, self.ids, cur, self.g_wte, self.g_wpe, 1 if tied else 0, self.ws)

    def eval_step(self):
        """Forward only; adds this batch's bpb sums into sum_nats / sum_bytes."""
        c, Bsz, T, N = self.c, self.B, self.T, self.N
        B.gpt_embed_fwd(c, Bsz, T, self.ids, self.wte, self.wpe, self.xs[0])
        for l, bp in enumerate(self.blocks):
            B.gpt_block_fwd(c, Bsz, T, self.xs[l], bp, self.xs[l + 1], None, self.ws)
        B.gpt_norm_fwd(c, N, self.xs[-1], self.lnf_w, self.lnf_b, self.hf, None)
        B.lm_head_xent_fwd_bwd(c, N, self.hf, self._head_weight(), self.tgt, 1.0 / N, self.loss, self.nats,
                               None, None, 0, self.ws)
        B.val_bpb_reduce(N, self.nats, self.tgt, self.token_bytes, self.cfg.vocab_size, self.sum_nats,
                         self.sum_bytes)
