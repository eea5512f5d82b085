"""Thin Python binding of the router C ABI (include/router.h).

Argument marshalling only: every step of the router runs in the HIP
kernels of librouter.so.  PyTorch provides device memory and the stream;
outputs are allocated with torch.empty unless passed in, and work is
enqueued on the current stream of the input's device.  There is no CPU
fallback: if librouter.so is not built, every call raises.

Entry points carry the C names: router_topk_fwd, router_topk_bwd,
router_aux_scores, router_aux_scores_bwd, router_tokens_per_expert,
router_tokens_per_expert_workspace_bytes, router_aux_loss_fwd,
router_aux_loss_fwd_noalloc, router_aux_loss_bwd, router_aux_loss_workspace_bytes,
router_route_maps, router_topk_shared_gate.
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
ROUTE_MAX_ROWS, ROUTE_MAX_EXPERTS, ROUTE_MAX_K = 16, 1024, 32
GATE_MAX_EXPERTS, GATE_MAX_K, GATE_MAX_SHARED = 1024, 32, 16

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
    lib.router_aux_loss_workspace_bytes.argtypes = [i64, i32]
    lib.router_aux_loss_workspace_bytes.restype = ctypes.c_size_t
    sz = ctypes.c_size_t
    lib.router_tokens_per_expert.argtypes = [vp, i64, i32, vp, vp, sz, vp]
    lib.router_tokens_per_expert_workspace_bytes.argtypes = [i64, i32]
    lib.router_tokens_per_expert_workspace_bytes.restype = ctypes.c_size_t
    lib.router_aux_loss_fwd.argtypes = [vp, ci, i64, i32, vp, i64, i32, f32, vp, vp, sz, vp]
    lib.router_aux_loss_bwd.argtypes = [vp, vp, ci, i64, i32, i64, i32, f32, vp, vp]
    lib.router_aux_loss_fwd_noalloc.argtypes = [vp, ci, i64, i32, vp, i64, i32, f32, vp, vp]
    lib.router_aux_loss_fwd_noalloc.restype = ci
    lib.router_route_maps.argtypes = [vp, ci, i32, i32, i32, ci, ci, vp, vp, vp, vp, vp, vp, vp]
    lib.router_route_maps.restype = ci
    lib.router_topk_shared_gate.argtypes = [vp, vp, vp, ci, i64, i32, i32, i32, i32, ci, f32,
                                            i32, vp, vp, i64, vp]
    lib.router_topk_shared_gate.restype = ci
    for f in (lib.router_topk_fwd, lib.router_topk_bwd, lib.router_aux_scores,
              lib.router_aux_scores_bwd, lib.router_set_topk_path_threshold,
              lib.router_tokens_per_expert, lib.router_aux_loss_fwd, lib.router_aux_loss_bwd):
        f.restype = ci
    lib.router_set_topk_path_threshold.argtypes = [ci]
    lib.router_get_topk_path_threshold.argtypes = []
    lib.router_get_topk_path_threshold.restype = ci
    lib.router_device_query.argtypes = [vp, vp, vp, vp]
    lib.router_device_query.restype = ci
    lib.router_set_group_stage.argtypes = [ci]
    lib.router_set_group_stage.restype = ci
    lib.router_get_group_stage.argtypes = []
    lib.router_get_group_stage.restype = ci
    lib.router_set_grid_mode.argtypes = [ci]
    lib.router_set_grid_mode.restype = ci
    lib.router_get_grid_mode.argtypes = []
    lib.router_get_grid_mode.restype = ci
    lib.router_stream_bandwidth.argtypes = [vp, i64, vp, i64, ci, vp]
    lib.router_stream_bandwidth.restype = ci
    lib.router_row_stream_bandwidth.argtypes = [vp, vp, vp, vp, i64, i64, vp]
    lib.router_row_stream_bandwidth.restype = ci
    lib.router_status_str.argtypes = [ci]
    lib.router_status_str.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_str(status):
    return load().router_status_str(status).decode()


def check(status):
    if status != OK:
        raise RouterError(status, status_str(status))


TOPK_PATH_AUTO = -1  # crossover chosen from the row layout (the default)


def set_topk_path_threshold(threshold):
    check(load().router_set_topk_path_threshold(int(threshold)))


def get_topk_path_threshold():
    return load().router_get_topk_path_threshold()


def device_query():
    """Attributes of the current device: compute units, peak engine and
    memory clocks (kHz), memory bus width (bits)."""
    vals = [ctypes.c_int32() for _ in range(4)]
    check(load().router_device_query(*[ctypes.byref(v) for v in vals]))
    return dict(zip(("compute_units", "clock_khz", "memory_clock_khz", "memory_bus_bits"),
                    (v.value for v in vals)))


GROUP_STAGE_AUTO = 0
GROUP_STAGE_LDS = 1


def stream_bandwidth(src, read_bytes, dst, write_bytes, units=1):
    """Reads read_bytes of src and writes write_bytes of dst (uint8 GPU
    tensors) with the router kernels' access style and no other work,
    `units` 16-byte units per thread (1, 2, 4 or 8): the bandwidth reference
    of a read:write mix (a measurement utility)."""
    check(load().router_stream_bandwidth(_ptr(src), int(read_bytes), _ptr(dst),
                                         int(write_bytes), int(units), _stream(src)))


def row_stream_bandwidth(x, out_a, out_b, out_map):
    """Moves the forward's bytes in the forward's own pattern (one wave per
    row of x [T, E] fp32: the row read whole, then written to out_a and
    out_b, one byte per element to out_map) with no other work: the
    bandwidth reference of a one-row-per-wave forward (a measurement
    utility)."""
    T, E = x.shape
    check(load().router_row_stream_bandwidth(_ptr(x), _ptr(out_a), _ptr(out_b), _ptr(out_map),
                                             int(T), int(E), _stream(x)))


GRID_FULL = 0
GRID_PERSISTENT = 1


def set_grid_mode(mode):
    check(load().router_set_grid_mode(int(mode)))


def get_grid_mode():
    return load().router_get_grid_mode()


def set_group_stage(stage):
    check(load().router_set_group_stage(int(stage)))


def get_group_stage():
    return load().router_get_group_stage()


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


def router_aux_loss_workspace_bytes(T, E):
    """Workspace bytes of router_aux_loss_fwd for T rows of E experts (0 if
    T, E are out of range)."""
    return load().router_aux_loss_workspace_bytes(int(T), int(E))


def _workspace(ws, T, E, device):
    need = router_aux_loss_workspace_bytes(T, E)
    if ws is None:
        return torch.empty((max(need, 256),), dtype=torch.uint8, device=device)
    if ws.device != device or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the input's device")
    return ws


def _counts(c, E, device):
    if (not isinstance(c, torch.Tensor) or c.dtype != torch.int64 or c.shape != (E,)
            or c.device != device or not c.is_contiguous()):
        raise ValueError(f"tokens_per_expert must be a contiguous int64 [{E}] tensor on "
                         f"{device}")
    return c


def router_tokens_per_expert_workspace_bytes(T, E):
    """Workspace bytes of router_tokens_per_expert (0 if T, E are out of
    range)."""
    return load().router_tokens_per_expert_workspace_bytes(int(T), int(E))


def router_tokens_per_expert(routing_map, out=None, workspace=None):
    """Tokens routed to each expert: int64 [E] column counts of the bool (or
    uint8) routing map [T,E].  `workspace`: a device tensor of at least
    router_tokens_per_expert_workspace_bytes(T, E) bytes that is
    zero-filled before its first use; every call leaves it zero-filled
    (without one, a zero-filled one is allocated for the call)."""
    if (not isinstance(routing_map, torch.Tensor) or routing_map.dim() != 2
            or not routing_map.is_cuda or not routing_map.is_contiguous()
            or routing_map.dtype not in (torch.bool, torch.uint8)):
        raise ValueError("routing_map must be a contiguous bool/uint8 [T,E] GPU tensor")
    T, E = routing_map.shape
    dev = routing_map.device
    counts = _out(out, (E,), torch.int64, dev, "tokens_per_expert")
    need = router_tokens_per_expert_workspace_bytes(T, E)
    if workspace is None:
        workspace = torch.zeros((max(need, 256),), dtype=torch.uint8, device=dev)
    elif workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the map's device")
    check(load().router_tokens_per_expert(_ptr(routing_map), T, E, _ptr(counts),
                                          _ptr(workspace),
                                          workspace.numel() * workspace.element_size(),
                                          _stream(routing_map)))
    return counts


def router_aux_loss_fwd(scores, tokens_per_expert, total_tokens, topk, coeff,
                        out=None, workspace=None):
    """Load-balancing loss coeff*E/(N^2 K) * sum_i n_i sum_t scores[t,i] as a
    0-dim float32 tensor (N = total_tokens, n = tokens_per_expert)."""
    T, E = _rows(scores, "scores")
    dev = scores.device
    counts = _counts(tokens_per_expert, E, dev)
    loss = _out(out, (), torch.float32, dev, "loss")
    ws = _workspace(workspace, T, E, dev)
    check(load().router_aux_loss_fwd(
        _ptr(scores), _DTYPE[scores.dtype], T, E, _ptr(counts), int(total_tokens),
        int(topk), float(coeff), _ptr(loss), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(scores)))
    return loss


def router_aux_loss_fwd_noalloc(scores, tokens_per_expert, total_tokens, topk, coeff, out):
    """router_aux_loss_fwd into a preallocated 0-dim float32 `out`, with the
    library's own scratch buffer instead of a workspace: allocates nothing
    (for callers that cannot allocate); calls that overlap on one GPU race."""
    T, E = _rows(scores, "scores")
    dev = scores.device
    counts = _counts(tokens_per_expert, E, dev)
    loss = _out(out, (), torch.float32, dev, "loss")
    check(load().router_aux_loss_fwd_noalloc(
        _ptr(scores), _DTYPE[scores.dtype], T, E, _ptr(counts), int(total_tokens), int(topk),
        float(coeff), _ptr(loss), _stream(scores)))
    return loss


def router_aux_loss_bwd(grad_loss, tokens_per_expert, num_tokens, total_tokens, topk,
                        coeff, dtype=torch.float32, out=None):
    """Gradient of the loss with respect to the scores: [num_tokens, E] in
    `dtype`, equal to grad_loss * coeff * E * n_i / (N^2 K) in column i."""
    if (not isinstance(grad_loss, torch.Tensor) or grad_loss.dtype != torch.float32
            or grad_loss.numel() != 1 or not grad_loss.is_cuda):
        raise ValueError("grad_loss must be a one-element float32 GPU tensor")
    dev = grad_loss.device
    E = tokens_per_expert.shape[0] if isinstance(tokens_per_expert, torch.Tensor) else -1
    counts = _counts(tokens_per_expert, E, dev)
    if dtype not in _DTYPE:
        raise ValueError("dtype must be float32 or bfloat16")
    T = int(num_tokens)
    dx = _out(out, (T, E), dtype, dev, "grad_scores")
    check(load().router_aux_loss_bwd(
        _ptr(grad_loss), _ptr(counts), _DTYPE[dtype], T, E, int(total_tokens), int(topk),
        float(coeff), _ptr(dx), _stream(grad_loss)))
    return dx


def router_route_maps(logits, topk, score_function="softmax", renorm=False, out=None):
    """Decode-shape routing with expert maps (T <= 16 rows, E <= 1024,
    K <= 32).  Returns a dict of device tensors: topk_weights [T,K] float32,
    topk_ids [T,K] int32, perm_to_unperm / unperm_to_perm / perm_expert
    [T*K] int32 and expert_offsets [E+1] int64; `out` may pass the same
    dict preallocated."""
    T, E = _rows(logits, "logits")
    K = int(topk)
    dev = logits.device
    n = T * K
    shapes = {"topk_weights": ((T, K), torch.float32), "topk_ids": ((T, K), torch.int32),
              "perm_to_unperm": ((n,), torch.int32), "unperm_to_perm": ((n,), torch.int32),
              "perm_expert": ((n,), torch.int32), "expert_offsets": ((E + 1,), torch.int64)}
    res = {k: _out(None if out is None else out.get(k), shp, dt, dev, k)
           for k, (shp, dt) in shapes.items()}
    check(load().router_route_maps(
        _ptr(logits), _DTYPE[logits.dtype], T, E, K, _SCORE[score_function],
        int(bool(renorm)), _ptr(res["topk_weights"]), _ptr(res["topk_ids"]),
        _ptr(res["perm_to_unperm"]), _ptr(res["unperm_to_perm"]), _ptr(res["perm_expert"]),
        _ptr(res["expert_offsets"]), _stream(logits)))
    return res


def router_topk_shared_gate(gating, hidden, gate_weight, topk, renorm=True, shared_scale=1.0,
                            shared_base=None, out=None):
    """Routed softmax top-k plus shared-expert sigmoid gates.  gating [M,E],
    hidden [M,H], gate_weight [S,H] (one dtype, float32 or bfloat16).
    Returns (weights [M, K+S] float32, ids [M, K+S] int32); `out` may pass
    that pair preallocated, also as column views of wider rows (row stride
    taken from the tensors, unit column stride)."""
    M, E = _rows(gating, "gating")
    Mh, H = _rows(hidden, "hidden")
    S, Hw = _rows(gate_weight, "gate_weight")
    if Mh != M or Hw != H or hidden.dtype != gating.dtype or gate_weight.dtype != gating.dtype:
        raise ValueError("hidden must be [M,H] and gate_weight [S,H], all in the gating dtype")
    K = int(topk)
    dev = gating.device
    base = E if shared_base is None else int(shared_base)
    if out is None:
        w = torch.empty((M, K + S), dtype=torch.float32, device=dev)
        ids = torch.empty((M, K + S), dtype=torch.int32, device=dev)
    else:
        w, ids = out
        for t, dt, name in ((w, torch.float32, "weights"), (ids, torch.int32, "ids")):
            if (t.dtype != dt or t.device != dev or t.dim() != 2 or t.shape != (M, K + S)
                    or (M > 1 and t.stride(1) != 1)):
                raise ValueError(f"{name} must be a {dt} [{M}, {K + S}] tensor with unit "
                                 f"column stride on {dev}")
        if w.stride(0) != ids.stride(0):
            raise ValueError("weights and ids must share one row stride")
    ld = w.stride(0) if M > 1 else K + S
    check(load().router_topk_shared_gate(
        _ptr(gating), _ptr(hidden), _ptr(gate_weight), _DTYPE[gating.dtype], M, E, H, K, S,
        int(bool(renorm)), float(shared_scale), base, _ptr(w), _ptr(ids), ld, _stream(gating)))
    return w, ids
