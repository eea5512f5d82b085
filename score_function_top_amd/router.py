"""Thin Python binding of the router C ABI (include/router.h).

Argument marshalling only: every step of the router runs in the HIP
kernels of librouter.so.  PyTorch provides device memory and the stream;
outputs are allocated with torch.empty unless passed in, and work is
enqueued on the current stream of the input's device.  There is no CPU
fallback: if librouter.so is not built, every call raises.

Entry points carry the C names: router_topk_fwd, router_topk_bwd,
router_aux_scores, router_aux_scores_bwd.
"""
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "librouter.so")

OK, ERR_INVALID_ARG, ERR_OVERFLOW, ERR_UNSUPPORTED, ERR_HIP = 0, 1, 2, 3, 4
F32, BF16 = 0, 1
SOFTMAX, SIGMOID = 0, 1
MAX_EXPERTS = 4096

_SCORE = {"softmax": SOFTMAX, "sigmoid": SIGMOID, SOFTMAX: SOFTMAX,
          SIGMOID: SIGMOID}
_DTYPE = {torch.float32: F32, torch.bfloat16: BF16}

_lib = None


class RouterError(RuntimeError):
    """A router call returned a status other than ROUTER_OK."""

    def __init__(self, status, msg):
        super().__init__(msg)
        self.status = status


def load():
    """Loads librouter.so (once); raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built: run `python score_function_top_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
    ci = ctypes.c_int
    lib.router_topk_fwd.argtypes = [vp, ci, i64, i32, i32, ci, ci, i32, i32, f32, vp,
                                    vp, vp, vp, vp]
    lib.router_topk_bwd.argtypes = [vp, vp, vp, ci, i64, i32, i32, ci, ci, f32, vp, vp]
    lib.router_aux_scores.argtypes = [vp, ci, i64, i32, i32, ci, ci, vp, vp, vp, vp]
    lib.router_aux_scores_bwd.argtypes = [vp, vp, ci, i64, i32, ci, ci, vp, vp]
    for f in (lib.router_topk_fwd, lib.router_topk_bwd, lib.router_aux_scores,
              lib.router_aux_scores_bwd, lib.router_set_topk_path_threshold):
        f.restype = ci
    lib.router_set_topk_path_threshold.argtypes = [ci]
    lib.router_get_topk_path_threshold.argtypes = []
    lib.router_get_topk_path_threshold.restype = ci
    lib.router_status_str.argtypes = [ci]
    lib.router_status_str.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_str(status):
    return load().router_status_str(status).decode()


def check(status):
    if status != OK:
        raise RouterError(status, status_str(status))


def set_topk_path_threshold(threshold):
    check(load().router_set_topk_path_threshold(int(threshold)))


def get_topk_path_threshold():
    return load().router_get_topk_path_threshold()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _rows(x, name):
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError(f"{name} must be a 2-D tensor [tokens, experts]")
    if not x.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if x.dtype not in _DTYPE:
        raise ValueError(f"{name} must be float32 or bfloat16")
    return x.shape[0], x.shape[1]


def _out(t, shape, dtype, device, name):
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    if (t.shape != shape or t.dtype != dtype or t.device != device
            or not t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape "
                         f"{tuple(shape)} on {device}")
    return t


def router_topk_fwd(logits, topk, score_function="softmax", renorm=False,
                    num_groups=0, group_topk=0, scaling_factor=1.0,
                    expert_bias=None, out=None):
    """fused_topk_with_score_function forward.  Returns (probs [T,E] in the
    logits dtype, routing_map [T,E] bool, intermediate [T,E] float32);
    `out` may pass those three tensors preallocated."""
    T, E = _rows(logits, "logits")
    dev = logits.device
    probs, rmap, inter = out if out is not None else (None, None, None)
    probs = _out(probs, logits.shape, logits.dtype, dev, "probs")
    rmap = _out(rmap, logits.shape, torch.bool, dev, "routing_map")
    inter = _out(inter, logits.shape, torch.float32, dev, "intermediate")
    if expert_bias is not None:
        if (expert_bias.dtype != torch.float32 or expert_bias.shape != (E,)
                or expert_bias.device != dev or not expert_bias.is_contiguous()):
            raise ValueError("expert_bias must be a contiguous float32 [E] tensor "
                             "on the logits' device")
    check(load().router_topk_fwd(
        _ptr(logits), _DTYPE[logits.dtype], T, E, int(topk), _SCORE[score_function],
        int(bool(renorm)), int(num_groups), int(group_topk), float(scaling_factor),
        _ptr(expert_bias), _ptr(probs), _ptr(rmap), _ptr(inter), _stream(logits)))
    return probs, rmap, inter


def router_topk_bwd(grad_probs, intermediate, routing_map, topk,
                    score_function="softmax", renorm=False, scaling_factor=1.0,
                    out=None):
    """fused_topk_with_score_function backward: grad_logits [T,E] in the
    grad_probs dtype."""
    T, E = _rows(grad_probs, "grad_probs")
    dev = grad_probs.device
    for t, dt, name in ((intermediate, torch.float32, "intermediate"),
                        (routing_map, torch.bool, "routing_map")):
        _out(t, grad_probs.shape, dt, dev, name)
    dx = _out(out, grad_probs.shape, grad_probs.dtype, dev, "grad_logits")
    check(load().router_topk_bwd(
        _ptr(grad_probs), _ptr(intermediate), _ptr(routing_map),
        _DTYPE[grad_probs.dtype], T, E, int(topk), _SCORE[score_function],
        int(bool(renorm)), float(scaling_factor), _ptr(dx), _stream(grad_probs)))
    return dx


def router_aux_scores(logits, topk, score_function="softmax", renorm=True, out=None):
    """fused_score_for_moe_aux_loss forward.  Returns (scores [T,E] in the
    logits dtype, routing_map [T,E] bool, intermediate [T,E] float32)."""
    T, E = _rows(logits, "logits")
    dev = logits.device
    scores, rmap, inter = out if out is not None else (None, None, None)
    scores = _out(scores, logits.shape, logits.dtype, dev, "scores")
    rmap = _out(rmap, logits.shape, torch.bool, dev, "routing_map")
    inter = _out(inter, logits.shape, torch.float32, dev, "intermediate")
    check(load().router_aux_scores(
        _ptr(logits), _DTYPE[logits.dtype], T, E, int(topk), _SCORE[score_function],
        int(bool(renorm)), _ptr(scores), _ptr(rmap), _ptr(inter), _stream(logits)))
    return scores, rmap, inter


def router_aux_scores_bwd(grad_scores, intermediate, score_function="softmax",
                          renorm=True, out=None):
    """fused_score_for_moe_aux_loss backward: grad_logits [T,E] in the
    grad_scores dtype."""
    T, E = _rows(grad_scores, "grad_scores")
    dev = grad_scores.device
    _out(intermediate, grad_scores.shape, torch.float32, dev, "intermediate")
    dx = _out(out, grad_scores.shape, grad_scores.dtype, dev, "grad_logits")
    check(load().router_aux_scores_bwd(
        _ptr(grad_scores), _ptr(intermediate), _DTYPE[grad_scores.dtype], T, E,
        _SCORE[score_function], int(bool(renorm)), _ptr(dx), _stream(grad_scores)))
    return dx
