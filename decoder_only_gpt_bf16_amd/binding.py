"""ctypes binding of libgptmi.so: the C entry points under the same names.

Argument marshalling only: torch tensors become device pointers, the current
torch stream becomes the hipStream_t argument, status codes become
exceptions.  Every computation runs in the library's HIP kernels.  Loading
fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgptmi.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "gptmi.h")

GPT_OK, GPT_ERR_INVALID, GPT_ERR_UNSUPPORTED, GPT_ERR_WORKSPACE, GPT_ERR_HIP = range(5)
BLOCK_FIELDS = ("ln1_w", "ln1_b", "w_qkv", "b_qkv", "w_o", "b_o",
                "ln2_w", "ln2_b", "w_fc", "b_fc", "w_proj", "b_proj")


class GptError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"gptmi status {status}: {msg}")
        self.status = status


class GptConfigC(ctypes.Structure):
    _fields_ = [("n_layer", ctypes.c_int32), ("n_head", ctypes.c_int32), ("n_embd", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("vocab_size", ctypes.c_int32), ("bias", ctypes.c_int32),
                ("norm", ctypes.c_int32), ("rope", ctypes.c_int32), ("qk_norm", ctypes.c_int32),
                ("rope_base", ctypes.c_float), ("norm_eps", ctypes.c_float), ("dtype", ctypes.c_int32),
                ("attn_window", ctypes.c_int32), ("fp8", ctypes.c_int32)]


class BlockWeightsC(ctypes.Structure):
    _fields_ = [(f, ctypes.c_void_p) for f in BLOCK_FIELDS]


class BlockGradsC(ctypes.Structure):
    _fields_ = [(f, ctypes.c_void_p) for f in BLOCK_FIELDS]


class AdamwTensorC(ctypes.Structure):
    _fields_ = [("param", ctypes.c_void_p), ("grad", ctypes.c_void_p), ("m", ctypes.c_void_p),
                ("v", ctypes.c_void_p), ("param_bf16", ctypes.c_void_p), ("n", ctypes.c_int64),
                ("decay", ctypes.c_int32)]


class AdamwConfigC(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float), ("step", ctypes.c_int32),
                ("max_norm", ctypes.c_float)]


_lib = None
_VP, _I, _SZ, _F = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float
_CFG = ctypes.POINTER(GptConfigC)
_ATP = ctypes.POINTER(AdamwTensorC)

_SIGS = {
    "gpt_block_saved_bytes": (_SZ, [_CFG, _I, _I]),
    "gpt_workspace_bytes": (_SZ, [_CFG, _I, _I]),
    "gpt_block_fwd": (_I, [_CFG, _I, _I, _VP, ctypes.POINTER(BlockWeightsC), _VP, _VP, _VP, _SZ, _VP]),
    "gpt_block_bwd": (_I, [_CFG, _I, _I, _VP, _VP, ctypes.POINTER(BlockWeightsC), _VP, _VP,
                           ctypes.POINTER(BlockGradsC), _I, _VP, _SZ, _VP]),
    "lm_head_xent_fwd_bwd": (_I, [_CFG, _I, _VP, _VP, _VP, _F, _VP, _VP, _VP, _VP, _I, _VP, _SZ, _VP]),
    "lm_head_xent_weighted_fwd_bwd": (_I, [_CFG, _I, _VP, _VP, _VP, _VP, _F, _VP, _VP, _VP, _VP, _I, _VP, _SZ,
                                           _VP]),
    "val_bpb_reduce": (_I, [_I, _VP, _VP, _VP, _I, _VP, _VP, _VP]),
    "gpt_embed_fwd": (_I, [_CFG, _I, _I, _VP, _VP, _VP, _VP, _VP]),
    "gpt_embed_bwd": (_I, [_CFG, _I, _I, _VP, _VP, _VP, _VP, _I, _VP, _SZ, _VP]),
    "gpt_norm_fwd": (_I, [_CFG, _I, _VP, _VP, _VP, _VP, _VP, _VP]),
    "gpt_norm_bwd": (_I, [_CFG, _I, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _I, _VP, _SZ, _VP]),
    "gpt_adamw_step": (_I, [ctypes.POINTER(AdamwConfigC), _ATP, _I, _VP, _VP, _SZ, _VP]),
    "gpt_adamw_workspace_bytes": (_SZ, [_ATP, _I]),
    "gpt_adamw_step_noalloc": (_I, [ctypes.POINTER(AdamwConfigC), _ATP, _I, _VP, _VP]),
    "gpt_fp8_quantize": (_I, [ctypes.c_int64, _VP, _I, _VP, _VP, _VP, _SZ, _VP]),
    "gpt_fp8_workspace_bytes": (_SZ, [ctypes.c_int64]),
    "gpt_fp8_gemm": (_I, [_I, _I, _I, _VP, ctypes.c_int64, _I, _VP, _VP, ctypes.c_int64, _I, _VP, _VP,
                          ctypes.c_int64, _VP]),
    "gpt_trace_begin": (_I, [_I]),
    "gpt_trace_end": (_I, [ctypes.c_char_p, _SZ]),
    "gpt_status_string": (ctypes.c_char_p, [_I]),
    "gpt_last_error": (ctypes.c_char_p, []),
}


def header_functions() -> list:
    """Names of the functions include/gptmi.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"defined", "sizeof"})


def lib() -> ctypes.CDLL:
    """Load libgptmi.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m decoder_only_gpt_bf16_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


# ----------------------------------------------------------------------------
# marshalling helpers
# ----------------------------------------------------------------------------

def make_config(cfg) -> GptConfigC:
    """From a synth.GPTConfig-like object."""
    return GptConfigC(cfg.n_layer, cfg.n_head, cfg.n_embd, cfg.block_size, cfg.vocab_size, int(cfg.bias),
                      0 if cfg.norm == "layernorm" else 1, int(cfg.rope), int(cfg.qk_norm),
                      float(cfg.rope_base), float(cfg.eps), 1 if cfg.dtype == "bf16" else 0,
                      int(getattr(cfg, "window", 0)), int(getattr(cfg, "fp8", False)))


def _p(t, want=None) -> Optional[int]:
    """Device pointer of a contiguous tensor (None passes through).  `want`
    names the element type the C side reads or writes: "f32", "f64", "i32",
    "i64", or a GptConfigC for the configuration's storage type."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensors passed to gptmi must be contiguous")
    if want is not None:
        import torch
        if isinstance(want, GptConfigC):
            exp = torch.bfloat16 if want.dtype == 1 else torch.float32
        else:
            exp = {"f32": torch.float32, "f64": torch.float64, "i32": torch.int32, "i64": torch.int64}[want]
        if t.dtype != exp:
            raise TypeError(f"gptmi expects a {exp} tensor here, got {t.dtype}")
    return t.data_ptr()


def _stream(stream=None) -> Optional[int]:
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _nbytes(t) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def _check(status: int):
    if status != GPT_OK:
        raise GptError(status, lib().gpt_last_error().decode())


def _block_struct(cls, d: dict, want=None):
    return cls(*[_p(d.get(f), want) for f in BLOCK_FIELDS])


# ----------------------------------------------------------------------------
# entry points
# ----------------------------------------------------------------------------

def gpt_block_saved_bytes(cfg: GptConfigC, B: int, T: int) -> int:
    return lib().gpt_block_saved_bytes(ctypes.byref(cfg), B, T)


def gpt_workspace_bytes(cfg: GptConfigC, B: int, T: int) -> int:
    return lib().gpt_workspace_bytes(ctypes.byref(cfg), B, T)


def gpt_block_fwd(cfg, B, T, x, w: dict, y, saved, ws, stream=None):
    W = _block_struct(BlockWeightsC, w, cfg)
    _check(lib().gpt_block_fwd(ctypes.byref(cfg), B, T, _p(x, cfg), ctypes.byref(W), _p(y, cfg), _p(saved), _p(ws),
                               _nbytes(ws), _stream(stream)))


def gpt_block_bwd(cfg, B, T, x, dy, w: dict, saved, dx, grads: dict, accumulate, ws, stream=None):
    W = _block_struct(BlockWeightsC, w, cfg)
    G = _block_struct(BlockGradsC, grads, "f32")
    _check(lib().gpt_block_bwd(ctypes.byref(cfg), B, T, _p(x, cfg), _p(dy, cfg), ctypes.byref(W), _p(saved),
                               _p(dx, cfg),
                               ctypes.byref(G), int(accumulate), _p(ws), _nbytes(ws), _stream(stream)))


def lm_head_xent_fwd_bwd(cfg, N, h, W, targets, loss_scale, loss, nats, dh, dW, accumulate, ws, stream=None):
    _check(lib().lm_head_xent_fwd_bwd(ctypes.byref(cfg), N, _p(h, cfg), _p(W, cfg), _p(targets, "i32"),
                                      float(loss_scale), _p(loss, "f32"), _p(nats, "f32"), _p(dh, cfg),
                                      _p(dW, "f32"), int(accumulate), _p(ws), _nbytes(ws),
                                      _stream(stream)))


def lm_head_xent_weighted_fwd_bwd(cfg, N, h, W, targets, token_weight, loss_scale, loss, nats, dh, dW, accumulate,
                                  ws, stream=None):
    _check(lib().lm_head_xent_weighted_fwd_bwd(ctypes.byref(cfg), N, _p(h, cfg), _p(W, cfg), _p(targets, "i32"),
                                               _p(token_weight, "f32"), float(loss_scale), _p(loss, "f32"),
                                               _p(nats, "f32"), _p(dh, cfg), _p(dW, "f32"), int(accumulate),
                                               _p(ws), _nbytes(ws), _stream(stream)))


def val_bpb_reduce(N, nats, targets, token_bytes, V, sum_nats, sum_bytes, stream=None):
    _check(lib().val_bpb_reduce(N, _p(nats, "f32"), _p(targets, "i32"), _p(token_bytes, "i32"), V,
                                _p(sum_nats, "f64"), _p(sum_bytes, "i64"),
                                _stream(stream)))


def gpt_embed_fwd(cfg, B, T, ids, wte, wpe, x0, stream=None):
    _check(lib().gpt_embed_fwd(ctypes.byref(cfg), B, T, _p(ids, "i32"), _p(wte, cfg), _p(wpe, cfg), _p(x0, cfg),
                               _stream(stream)))


def gpt_embed_bwd(cfg, B, T, ids, dx0, dwte, dwpe, accumulate, ws, stream=None):
    _check(lib().gpt_embed_bwd(ctypes.byref(cfg), B, T, _p(ids, "i32"), _p(dx0, cfg), _p(dwte, "f32"),
                               _p(dwpe, "f32"), int(accumulate),
                               _p(ws), _nbytes(ws), _stream(stream)))


def gpt_trace_begin(capacity: int):
    _check(lib().gpt_trace_begin(capacity))


def gpt_trace_end() -> dict:
    """{call-site name: (launches, total microseconds)}."""
    buf = ctypes.create_string_buffer(1 << 16)
    _check(lib().gpt_trace_end(buf, len(buf)))
    out = {}
    for line in buf.value.decode().splitlines():
        name, n, us = line.split()
        out[name] = (int(n), float(us))
    return out


def gpt_norm_fwd(cfg, N, x, w, b, y, stats, stream=None):
    _check(lib().gpt_norm_fwd(ctypes.byref(cfg), N, _p(x, cfg), _p(w, cfg), _p(b, cfg), _p(y, cfg), _p(stats, "f32"),
                              _stream(stream)))


def gpt_norm_bwd(cfg, N, x, w, dy, resid, dx, dw, db, accumulate, ws, stream=None):
    _check(lib().gpt_norm_bwd(ctypes.byref(cfg), N, _p(x, cfg), _p(w, cfg), _p(dy, cfg), _p(resid, cfg), _p(dx, cfg),
                              _p(dw, "f32"), _p(db, "f32"),
                              int(accumulate), _p(ws), _nbytes(ws), _stream(stream)))


def _adamw_table(tensors):
    """tensors: iterable of dicts with param, grad, m, v (fp32), optional
    param_bf16 (bf16) and decay (bool)."""
    tensors = list(tensors)
    arr = (AdamwTensorC * len(tensors))()
    for i, t in enumerate(tensors):
        n = t["param"].numel()
        for k in ("grad", "m", "v"):
            if t[k].numel() != n:
                raise ValueError(f"tensor {i}: {k} has {t[k].numel()} elements, param has {n}")
        p16 = t.get("param_bf16")
        if p16 is not None:
            import torch
            if p16.dtype != torch.bfloat16 or p16.numel() != n:
                raise TypeError(f"tensor {i}: param_bf16 must be a bf16 tensor of {n} elements")
        arr[i] = AdamwTensorC(_p(t["param"], "f32"), _p(t["grad"], "f32"), _p(t["m"], "f32"), _p(t["v"], "f32"),
                              _p(p16), n, int(bool(t.get("decay", True))))
    return arr


def gpt_adamw_workspace_bytes(tensors) -> int:
    arr = _adamw_table(tensors)
    return lib().gpt_adamw_workspace_bytes(arr, len(arr))


def gpt_adamw_step(tensors, lr, beta1, beta2, eps, weight_decay, step, max_norm, grad_norm, ws, stream=None):
    arr = _adamw_table(tensors)
    cfg = AdamwConfigC(lr, beta1, beta2, eps, weight_decay, int(step), max_norm)
    _check(lib().gpt_adamw_step(ctypes.byref(cfg), arr, len(arr), _p(grad_norm, "f32"), _p(ws), _nbytes(ws),
                                _stream(stream)))


def gpt_adamw_step_noalloc(tensors, lr, beta1, beta2, eps, weight_decay, step, max_norm, grad_norm, stream=None):
    """gpt_adamw_step with the library's own per-GPU scratch (no workspace)."""
    arr = _adamw_table(tensors)
    cfg = AdamwConfigC(lr, beta1, beta2, eps, weight_decay, int(step), max_norm)
    _check(lib().gpt_adamw_step_noalloc(ctypes.byref(cfg), arr, len(arr), _p(grad_norm, "f32"), _stream(stream)))


ADAMW_NOALLOC_MAX_CHUNKS = 131072

FP8_E4M3, FP8_E5M2 = 0, 1


def gpt_fp8_workspace_bytes(n: int) -> int:
    return lib().gpt_fp8_workspace_bytes(int(n))


def gpt_fp8_quantize(x, fmt, q, scale, ws, stream=None):
    """x: bf16 tensor; q: uint8 tensor of x.numel(); scale: fp32 tensor of >= 3."""
    import torch
    if x.dtype != torch.bfloat16 or q.dtype != torch.uint8 or q.numel() != x.numel():
        raise TypeError("x must be bf16 and q a uint8 tensor of the same size")
    _check(lib().gpt_fp8_quantize(x.numel(), _p(x), int(fmt), _p(q), _p(scale, "f32"), _p(ws), _nbytes(ws),
                                  _stream(stream)))


def gpt_fp8_gemm(qa, fmt_a, scale_a, qb, fmt_b, scale_b, out, stream=None):
    """qa [M, K], qb [N, K] uint8 codes (row-major); out bf16 [M, N]."""
    import torch
    M, K = qa.shape
    N, K2 = qb.shape
    if K != K2 or out.shape != (M, N) or out.dtype != torch.bfloat16:
        raise ValueError("shapes: qa [M, K], qb [N, K], out bf16 [M, N]")
    _check(lib().gpt_fp8_gemm(M, N, K, _p(qa), qa.stride(0), int(fmt_a), _p(scale_a, "f32"), _p(qb), qb.stride(0),
                              int(fmt_b), _p(scale_b, "f32"), _p(out), out.stride(0), _stream(stream)))
