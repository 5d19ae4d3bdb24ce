"""GPU parity of whole-model workloads assembled from the C entry points:
the tiny fp32 GPT step, the GPT-2 124M step and the d20 val-bpb evaluation,
at reduced sizes and at the full sizes, each against the complete oracle."""
import math

import numpy as np
import pytest
import torch

import oracle as O
from decoder_only_gpt_bf16_amd import synth
from decoder_only_gpt_bf16_amd.model import ModelRunner, to_f64
from tests import _oracle_par as OP
from tests._parity import REL_ACT, REL_LOSS, assert_rel, print_case

pytestmark = pytest.mark.gpu


def _grads_check(G, r, rep):
    for li, gb in enumerate(G["blocks"]):
        for k, v in gb.items():
            if v is not None:
                assert_rel(f"L{li}.d{k}", to_f64(r.g_blocks[li][k]), v, REL_ACT, rep)
    assert_rel("dwte", to_f64(r.g_wte), G["wte"], REL_ACT, rep)
    if G.get("wpe") is not None:
        assert_rel("dwpe", to_f64(r.g_wpe), G["wpe"], REL_ACT, rep)
    if G.get("lnf_w") is not None:
        assert_rel("dlnf_w", to_f64(r.g_lnf_w), G["lnf_w"], REL_ACT, rep)
    if G.get("lnf_b") is not None:
        assert_rel("dlnf_b", to_f64(r.g_lnf_b), G["lnf_b"], REL_ACT, rep)
    if G.get("lm_head") is not None:
        assert_rel("dlm_head", to_f64(r.g_lm_head), G["lm_head"], REL_ACT, rep)


STEP_CASES = [
    ("tiny_gpt_fp32", {}, False),
    ("tiny_gpt_fp32", {}, True),
    ("gpt2_124m_step", dict(B=2, T=128, n_layer=2), False),
    ("gpt2_124m_step", dict(B=1, T=77, n_layer=1), True),
]


@pytest.mark.parametrize("case", STEP_CASES, ids=[f"{c[0]}-{c[1]}-{c[2]}" for c in STEP_CASES])
def test_train_step_parity(case):
    name, sz, aff = case
    w = synth.scaled(synth.BY_NAME[name], **sz)
    print_case("step", name, sz, aff)
    ids, y, P, tb = synth.make_model_inputs(w, random_affine=aff)
    r = ModelRunner(w.cfg, w.B, w.T, P, tb)
    r.set_batch(ids, y)
    r.train_step()
    torch.cuda.synchronize()
    cfg = synth.oracle_cfg(w.cfg)
    loss, nats, G = O.model_fwd_bwd(cfg, ids, y, P)
    rep = {}
    assert_rel("loss", r.loss.item(), loss, REL_LOSS, rep)
    assert_rel("nats", to_f64(r.nats), nats, REL_ACT, rep)
    _grads_check(G, r, rep)
    if name == "tiny_gpt_fp32":
        # every byte length is 1: bpb = loss / ln 2
        s_n, s_b, bpb = O.val_bpb(to_f64(r.nats), y, tb)
        assert abs(bpb - r.loss.item() / math.log(2)) < 1e-5 * bpb
    print(name, {k: f"{v:.2e}" for k, v in rep.items()})


@pytest.mark.timeout(1200)
def test_gpt2_step_full_size():
    """Full GPT-2 124M step (B=16, T=1024, 12 layers, V=50304, Zipf ids)
    against the complete oracle: the loss, every token's nats and every
    parameter gradient.  The oracle runs one sequence per call on a thread
    pool; the mean loss's gradients are the mean of the per-sequence ones
    ("nanoGPT — Karpathy's minimal GPT pretraining repo", train.py section:
    mean cross-entropy over all targets of the batch)."""
    w = synth.GPT2_STEP
    print_case("step-full", w.name)
    ids, y, P, tb = synth.make_model_inputs(w)
    r = ModelRunner(w.cfg, w.B, w.T, P, tb)
    r.set_batch(ids, y)
    r.train_step()
    torch.cuda.synchronize()
    gpu_nats = to_f64(r.nats)
    # the loss is the mean of the per-token nats (the GPU sums them itself)
    assert abs(r.loss.item() - gpu_nats.mean()) <= 1e-5 * gpu_nats.mean()
    cfg = synth.oracle_cfg(w.cfg)
    loss, nats, G = OP.train_step(cfg, ids, y, P)
    rep = {}
    assert_rel("loss", r.loss.item(), loss, REL_LOSS, rep)
    assert_rel("nats", gpu_nats, nats, REL_ACT, rep)
    _grads_check(G, r, rep)
    print("gpt2 full", {k: f"{v:.2e}" for k, v in rep.items()})


EVAL_CASES = [dict(B=2, T=256, n_layer=2), dict(B=1, T=100, n_layer=1)]


@pytest.mark.parametrize("sz", EVAL_CASES, ids=[str(s) for s in EVAL_CASES])
def test_val_bpb_parity(sz):
    w = synth.scaled(synth.D20_EVAL, **sz)
    print_case("eval", sz)
    ids, y, P, tb = synth.make_model_inputs(w)
    r = ModelRunner(w.cfg, w.B, w.T, P, tb, train=False)
    r.set_batch(ids, y)
    r.eval_step()
    torch.cuda.synchronize()
    cfg = synth.oracle_cfg(w.cfg)
    nats = O.model_eval_nats(cfg, ids, y, P)
    s_n, s_b, bpb = O.val_bpb(nats, y, tb)
    rep = {}
    assert_rel("nats", to_f64(r.nats), nats, REL_ACT, rep)
    assert int(r.sum_bytes.item()) == s_b
    assert_rel("sum_nats", r.sum_nats.item(), s_n, REL_LOSS, rep)
    gpu_bpb = r.sum_nats.item() / (math.log(2) * r.sum_bytes.item())
    assert_rel("bpb", gpu_bpb, bpb, REL_LOSS, rep)
    print("eval", sz, {k: f"{v:.2e}" for k, v in rep.items()}, "bpb", gpu_bpb, bpb)


@pytest.mark.timeout(1200)
def test_val_bpb_full_size():
    """Full d20 evaluation (20 layers, B=8, T=2048, V=32768, byte lengths
    1..12) against the complete oracle ("Train your own ChatGPT", 6.2,
    loss_eval.py paragraph): every token's nats, the byte sum exactly, the
    nats sum and bits per byte.  The oracle runs one sequence per call on a
    thread pool."""
    w = synth.D20_EVAL
    print_case("eval-full", w.name)
    ids, y, P, tb = synth.make_model_inputs(w)
    r = ModelRunner(w.cfg, w.B, w.T, P, tb, train=False)
    r.set_batch(ids, y)
    r.eval_step()
    torch.cuda.synchronize()
    cfg = synth.oracle_cfg(w.cfg)
    nats = OP.eval_nats(cfg, ids, y, P)
    s_n, s_b, bpb = O.val_bpb(nats, y, tb)
    rep = {}
    assert_rel("nats", to_f64(r.nats), nats, REL_ACT, rep)
    assert int(r.sum_bytes.item()) == s_b
    assert_rel("sum_nats", r.sum_nats.item(), s_n, REL_LOSS, rep)
    gpu_bpb = r.sum_nats.item() / (math.log(2) * r.sum_bytes.item())
    assert_rel("bpb", gpu_bpb, bpb, REL_LOSS, rep)
    print("eval full", {k: f"{v:.2e}" for k, v in rep.items()}, "bpb", gpu_bpb, bpb)
