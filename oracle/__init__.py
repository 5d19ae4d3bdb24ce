"""Float64 CPU oracle for one decoder-only GPT training step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package; only the tests, the smoke check and the
CPU-baseline leg of the benchmark use it.  It shares no code with the HIP
path: it receives the same seeded inputs (bf16-representable values upcast to
float64) and computes every step from its plain definition in NumPy float64.

Sources (pages, by title):
  * "nanoGPT — Karpathy's minimal GPT pretraining repo": model.py section
    (GPTConfig, Block, CausalSelfAttention, MLP, LayerNorm, weight tying,
    scaled residual init, configure_optimizers: AdamW with decay on 2-D
    tensors only) and train.py section (shifted targets, mean loss, gradient
    clipping to a global norm of 1.0).  AdamW's own steps follow Loshchilov &
    Hutter, "Decoupled Weight Decay Regularization", Algorithm 2.
  * "Train your own ChatGPT" (nanochat lab): 6.2, the loss_eval.py paragraph
    (bits per byte, zero-byte special tokens excluded); 6.3 (masked loss).
  * "nanochat-d20-chat — a chat model trained from scratch": Architecture row
    (RoPE + QK-norm, width 1280, 10 heads, 2048 context).

Every function is pinned by a test under tests/ (finite differences,
PyTorch float64 autograd, closed forms and invariants).  No function here is
"parity unpinned".
"""
from .gpt_oracle import *  # noqa: F401,F403
