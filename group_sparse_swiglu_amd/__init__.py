"""group_sparse_swiglu_amd -- group-sparse SwiGLU feed-forward layer for AMD MI355X.

A thin ctypes binding of ``libesg.so`` (declared in ``include/esg.h``).  Torch
supplies device memory and the current HIP stream; every computation runs in
the library's HIP kernels.  There is no fallback: if the library is not built
or no GPU is present, the calls raise.

Names follow the eugen_sparse README ("What it does"): make_subsample_index,
grouped_topk_select, sparse_swiglu_ffn (forward + backward),
update_load_balance_bias; and, from the Megatron-Core developer guide page
"core.inference.moe.sigmoid_topk", sigmoid_topk_routing; and, from the
parameter-golf pull request 1105 page, the LeakyReLU(0.5)^2 MLP with a stored
activation gradient (leaky_mlp_fwd / leaky_mlp_bwd); and, from the FlashFFN
README, the multi-head sub-network FFN core (mhffn_fwd / mhffn_bwd).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

__all__ = [
    "ESG_F32", "ESG_BF16", "EsgError", "lib", "library_path", "make_subsample_index", "grouped_topk_select",
    "select_workspace_size", "bucket_by_group", "sparse_swiglu_fwd", "sparse_swiglu_bwd", "sparse_swiglu_ffn",
    "update_load_balance_bias", "update_load_balance_bias_from_routing",
    "update_load_balance_bias_from_counts", "workspace_size", "mfma_rate_probe", "timing_enable", "timing_reset", "timing_read",
    "FfnContext", "EXPORTED_SYMBOLS", "sigmoid_topk_supported", "sigmoid_topk_routing",
    "leaky_mlp_workspace_size", "leaky_mlp_fwd", "leaky_mlp_bwd", "leaky_mlp_saved_views",
    "mhffn_supported", "mhffn_fwd", "mhffn_bwd",
]

ESG_F32 = 0
ESG_BF16 = 1
STATUS_GROUP_OUT_OF_RANGE = 1
STATUS_GROUP_DUPLICATE = 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

_c_int, _c_size, _c_vp, _c_f = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float
_c_i32p = ctypes.POINTER(ctypes.c_int32)

# name -> (restype, argtypes)
_SIGNATURES = {
    "esg_status_string": (ctypes.c_char_p, [_c_int]),
    "esg_version": (_c_int, []),
    "esg_make_subsample_index": (_c_int, [_c_int, _c_int, _c_int, ctypes.c_uint64, _c_vp]),
    "esg_grouped_topk_select": (_c_int, [_c_vp, _c_vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_vp,
                                         _c_int, _c_vp, _c_vp, _c_vp, _c_vp]),
    "esg_grouped_topk_select_workspace_size": (_c_int, [_c_int, _c_int, _c_int, ctypes.POINTER(_c_size)]),
    "esg_grouped_topk_select_ws": (_c_int, [_c_vp, _c_vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_vp,
                                            _c_int, _c_vp, _c_vp, _c_vp, _c_vp, _c_size, _c_vp]),
    "esg_bucket_workspace_size": (_c_int, [_c_int, _c_int, _c_int, ctypes.POINTER(_c_size)]),
    "esg_bucket_by_group": (_c_int, [_c_vp, _c_int, _c_int, _c_int, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_size,
                                     _c_vp]),
    "esg_sparse_swiglu_workspace_size": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                                  ctypes.POINTER(_c_size), ctypes.POINTER(_c_size),
                                                  ctypes.POINTER(_c_size)]),
    "esg_sparse_swiglu_fwd": (_c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                       _c_vp, _c_vp, _c_vp, _c_size, _c_vp, _c_size, _c_vp, _c_vp]),
    "esg_sparse_swiglu_fwd_noalloc": (_c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_int, _c_int, _c_int, _c_int, _c_int,
                                               _c_int, _c_vp, _c_vp, _c_vp, _c_vp]),
    "esg_sparse_swiglu_bwd": (_c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_int, _c_int, _c_int, _c_int, _c_int,
                                       _c_int, _c_vp, _c_vp, _c_size, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_size,
                                       _c_vp]),
    "esg_sparse_swiglu_bwd_overlap": (_c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_int, _c_int, _c_int, _c_int,
                                               _c_int, _c_int, _c_vp, _c_vp, _c_size, _c_vp, _c_vp, _c_vp, _c_vp,
                                               _c_vp, _c_size, _c_vp, _c_vp]),
    "esg_update_load_balance_bias": (_c_int, [_c_vp, _c_vp, _c_vp, _c_f, _c_f, _c_f, _c_f, _c_int, _c_vp]),
    "esg_update_load_balance_bias_from_counts": (_c_int, [_c_vp, _c_vp, _c_vp, _c_int, _c_f, _c_f, _c_f, _c_f,
                                                          _c_int, _c_vp]),
    "esg_update_load_balance_bias_from_routing": (_c_int, [_c_vp, _c_vp, _c_vp, _c_size, _c_int, _c_int, _c_int,
                                                           _c_int, _c_int, _c_int, _c_f, _c_f, _c_f, _c_f, _c_vp]),
    "esg_leaky_mlp_workspace_size": (_c_int, [_c_int, _c_int, _c_int, ctypes.POINTER(_c_size),
                                              ctypes.POINTER(_c_size)]),
    "esg_leaky_mlp_fwd": (_c_int, [_c_vp, _c_vp, _c_vp, _c_int, _c_int, _c_int, _c_vp, _c_vp, _c_size, _c_vp]),
    "esg_leaky_mlp_bwd": (_c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_int, _c_int, _c_int, _c_vp, _c_vp, _c_vp, _c_vp,
                                   _c_vp, _c_size, _c_vp]),
    "esg_mhffn_supported": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int]),
    "esg_mhffn_fwd": (_c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_vp, _c_vp]),
    "esg_mhffn_bwd": (_c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_vp,
                               _c_vp, _c_vp, _c_vp, _c_vp, _c_vp]),
    "esg_sigmoid_topk_supported": (_c_int, [_c_int, _c_int]),
    "esg_sigmoid_topk_routing": (_c_int, [_c_vp, _c_vp, _c_int, _c_int, _c_int, _c_int, _c_f, _c_int, _c_vp, _c_vp,
                                          _c_vp]),
    "esg_mfma_rate_probe": (_c_int, [_c_int, _c_int, _c_vp, _c_vp]),
    "esg_timing_enable": (_c_int, [_c_int]),
    "esg_timing_reset": (_c_int, []),
    "esg_timing_read": (_c_int, [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_c_int)]),
}
EXPORTED_SYMBOLS = tuple(_SIGNATURES)


class EsgError(RuntimeError):
    pass


def library_path() -> str:
    return os.path.join(_HERE, "libesg.so")


def lib():
    """Load libesg.so (built in-tree by ``python -m group_sparse_swiglu_amd.build``)."""
    global _LIB
    if _LIB is None:
        path = library_path()
        if not os.path.exists(path):
            raise EsgError(f"{path} is not built; run `python -m group_sparse_swiglu_amd.build`")
        handle = ctypes.CDLL(path)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = handle
    return _LIB


def _check(status: int, what: str) -> None:
    if status != 0:
        msg = lib().esg_status_string(status).decode()
        raise EsgError(f"{what}: {msg} (status {status})")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return ESG_F32
    if t.dtype == torch.bfloat16:
        return ESG_BF16
    raise EsgError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _dev(t: Optional[torch.Tensor], name: str, dtype=None):
    """Device pointer of a contiguous GPU tensor (None -> NULL)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise EsgError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise EsgError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise EsgError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(device: torch.device):
    return torch.cuda.current_stream(device).cuda_stream


def make_subsample_index(d_ff: int, group_size: int, samples_per_group: int, seed: int):
    """Fixed random subset of gate rows per group -> (int32 CPU tensor [G*spg], spg)."""
    groups = d_ff // group_size if group_size > 0 else 0
    out = torch.empty(max(groups * samples_per_group, 1), dtype=torch.int32)
    _check(lib().esg_make_subsample_index(d_ff, group_size, samples_per_group, seed, out.data_ptr()),
           "make_subsample_index")
    return out[:groups * samples_per_group], samples_per_group


def select_workspace_size(tokens: int, d_ff: int, group_size: int) -> int:
    """Bytes of the energy table esg_grouped_topk_select_ws can use."""
    need = _c_size()
    _check(lib().esg_grouped_topk_select_workspace_size(tokens, d_ff, group_size, ctypes.byref(need)),
           "grouped_topk_select_workspace_size")
    return need.value


def grouped_topk_select(x, w_gate, group_size: int, num_active_groups: int, subsample_idx=None,
                        samples_per_group: Optional[int] = None, load_balance_bias=None, return_counts=False,
                        out=None, counts_out=None, workspace=None):
    """Per-token top-k groups by energy -> int32 [T, k] (and int32 counts [G]).

    workspace: None allocates the energy table for batches of fewer 32-token
    blocks than the device has CUs (the selection is the same either way);
    False never uses one; a uint8 device tensor is passed as given."""
    T, d = x.shape
    F = w_gate.shape[0]
    G = F // group_size
    code = _dtype_code(x)
    if w_gate.dtype != x.dtype:
        raise EsgError("x and w_gate must share a dtype")
    idx = out if out is not None else torch.empty(T, num_active_groups, dtype=torch.int32, device=x.device)
    counts = None
    if return_counts:
        counts = counts_out if counts_out is not None else torch.empty(G, dtype=torch.int32, device=x.device)
    spg = samples_per_group if samples_per_group is not None else 0
    if workspace is None:
        cus = torch.cuda.get_device_properties(x.device).multi_processor_count
        workspace = False
        if 0 < (T + 31) // 32 < cus:
            workspace = torch.empty(select_workspace_size(T, F, group_size), dtype=torch.uint8, device=x.device)
    ws = workspace if workspace is not False else None
    _check(lib().esg_grouped_topk_select_ws(
        _dev(x, "x"), _dev(w_gate, "w_gate"), code, T, d, F, group_size, num_active_groups,
        _dev(subsample_idx, "subsample_idx", torch.int32), spg, _dev(load_balance_bias, "bias", torch.float32),
        _dev(idx, "idx"), _dev(counts, "counts"), _dev(ws, "workspace"), 0 if ws is None else ws.numel(),
        _stream(x.device)), "grouped_topk_select")
    return (idx, counts) if return_counts else idx


def bucket_by_group(idx, groups: int, status=None):
    """CSR of (token, slot) pairs by group -> (offsets [G+1], perm_token [T*k], inv [T, k])."""
    T, k = idx.shape
    need = _c_size()
    _check(lib().esg_bucket_workspace_size(T, k, groups, ctypes.byref(need)), "bucket_workspace_size")
    dev = idx.device
    scratch = torch.empty(max(need.value, 16), dtype=torch.uint8, device=dev)
    offsets = torch.empty(groups + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(max(T * k, 1), dtype=torch.int32, device=dev)
    inv = torch.empty(T, k, dtype=torch.int32, device=dev)
    _check(lib().esg_bucket_by_group(_dev(idx, "idx", torch.int32), T, k, groups, _dev(offsets, "offsets"),
                                     _dev(perm, "perm"), _dev(inv, "inv"), _dev(status, "status", torch.int32),
                                     _dev(scratch, "scratch"), scratch.numel(), _stream(dev)), "bucket_by_group")
    return offsets, perm[:T * k], inv


def workspace_size(tokens, d_model, d_ff, group_size, k, dtype_code, dense=False):
    sv, fw, bw = _c_size(), _c_size(), _c_size()
    _check(lib().esg_sparse_swiglu_workspace_size(tokens, d_model, d_ff, group_size, k, dtype_code, int(dense),
                                                  ctypes.byref(sv), ctypes.byref(fw), ctypes.byref(bw)),
           "workspace_size")
    return sv.value, fw.value, bw.value


@dataclass
class FfnContext:
    """What the backward needs from the forward (caller-owned buffers), and the
    forward's shape (for the bias update from its routing)."""
    saved: torch.Tensor
    idx: Optional[torch.Tensor]
    group_size: int
    k: int
    tokens: int = 0
    d_model: int = 0
    d_ff: int = 0
    dtype_code: int = ESG_BF16


def _ws(nbytes: int, dev, cache: Optional[dict], key: str) -> torch.Tensor:
    nbytes = max(int(nbytes), 256)
    if cache is not None:
        buf = cache.get(key)
        if buf is None or buf.numel() < nbytes or buf.device != dev:
            buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
            cache[key] = buf
        return buf
    return torch.empty(nbytes, dtype=torch.uint8, device=dev)


def sparse_swiglu_fwd(x, w_gate, w_up, w_down, group_idx, group_size: int, status=None, workspace=None,
                      out=None, saved=None, for_backward: bool = True):
    """Forward -> (y [T, d], FfnContext).  group_idx None = every group active.

    ``workspace``: optional dict reused across calls to hold scratch buffers.
    ``for_backward=False``: inference, nothing is saved (the context then cannot
    be passed to the backward)."""
    T, d = x.shape
    F = w_gate.shape[0]
    code = _dtype_code(x)
    for name, w in (("w_gate", w_gate), ("w_up", w_up), ("w_down", w_down)):
        if w.dtype != x.dtype:
            raise EsgError(f"{name} must have the dtype of x")
    k = group_idx.shape[1] if group_idx is not None else F // group_size
    sv, fw, _ = workspace_size(T, d, F, group_size, k, code, group_idx is None)
    dev = x.device
    if not for_backward:
        saved = None
    elif saved is None or saved.numel() < sv:
        saved = torch.empty(max(sv, 256), dtype=torch.uint8, device=dev)
    scratch = _ws(fw, dev, workspace, "fwd")
    y = out if out is not None else torch.empty(T, d, dtype=x.dtype, device=dev)
    _check(lib().esg_sparse_swiglu_fwd(
        _dev(x, "x"), _dev(w_gate, "w_gate"), _dev(w_up, "w_up"), _dev(w_down, "w_down"), code, T, d, F,
        group_size, k, _dev(group_idx, "group_idx", torch.int32), _dev(y, "y"), _dev(saved, "saved"),
        saved.numel() if saved is not None else 0,
        _dev(scratch, "scratch"), scratch.numel(), _dev(status, "status", torch.int32), _stream(dev)),
        "sparse_swiglu_fwd")
    return y, FfnContext(saved, group_idx, group_size, k, T, d, F, code)


def sparse_swiglu_bwd(dy, x, w_gate, w_up, w_down, ctx: FfnContext, workspace=None, outs=None, aux_stream=None):
    """Backward -> (dx, dW_gate, dW_up, dW_down), all overwritten.

    ``aux_stream``: an optional second torch stream on which the weight
    gradients run beside the dx sum (esg_sparse_swiglu_bwd_overlap); every
    result is ordered on the current stream on return."""
    if ctx.saved is None and ctx.idx is not None:
        raise EsgError("the forward ran with for_backward=False: nothing was saved for a backward")
    T, d = x.shape
    F = w_gate.shape[0]
    code = _dtype_code(x)
    if dy.dtype != x.dtype:
        raise EsgError("dy must have the dtype of x")
    _, _, bw = workspace_size(T, d, F, ctx.group_size, ctx.k, code, ctx.idx is None)
    dev = x.device
    scratch = _ws(bw, dev, workspace, "bwd")
    if outs is None:
        outs = (torch.empty_like(x), torch.empty_like(w_gate), torch.empty_like(w_up), torch.empty_like(w_down))
    dx, dwg, dwu, dwd = outs
    _check(lib().esg_sparse_swiglu_bwd_overlap(
        _dev(dy, "dy"), _dev(x, "x"), _dev(w_gate, "w_gate"), _dev(w_up, "w_up"), _dev(w_down, "w_down"), code, T,
        d, F, ctx.group_size, ctx.k, _dev(ctx.idx, "group_idx", torch.int32), _dev(ctx.saved, "saved"),
        ctx.saved.numel() if ctx.saved is not None else 0, _dev(dx, "dx"), _dev(dwg, "dw_gate"), _dev(dwu, "dw_up"),
        _dev(dwd, "dw_down"), _dev(scratch, "scratch"), scratch.numel(), _stream(dev),
        None if aux_stream is None else aux_stream.cuda_stream), "sparse_swiglu_bwd")
    return dx, dwg, dwu, dwd


class _SparseSwiGLU(torch.autograd.Function):
    @staticmethod
    def forward(fctx, x, w_gate, w_up, w_down, group_idx, group_size):
        y, c = sparse_swiglu_fwd(x.contiguous(), w_gate.contiguous(), w_up.contiguous(), w_down.contiguous(),
                                 group_idx, group_size)
        fctx.save_for_backward(x, w_gate, w_up, w_down)
        fctx.esg = c
        return y

    @staticmethod
    def backward(fctx, dy):
        x, w_gate, w_up, w_down = fctx.saved_tensors
        dx, dwg, dwu, dwd = sparse_swiglu_bwd(dy.contiguous(), x, w_gate, w_up, w_down, fctx.esg)
        return dx, dwg, dwu, dwd, None, None


def sparse_swiglu_ffn(x, W_gate, W_up, W_down, group_idx, group_size: int):
    """Autograd entry: y = sum over selected groups of (SiLU(x W_g^T) * x W_u^T) W_d^T."""
    return _SparseSwiGLU.apply(x, W_gate, W_up, W_down, group_idx, group_size)


def update_load_balance_bias(bias, freq_ema, current_freq, target_freq: float, gamma: float, bias_max: float,
                             momentum: float):
    """In-place bias / EMA update (float32 device tensors [G])."""
    G = bias.numel()
    _check(lib().esg_update_load_balance_bias(
        _dev(bias, "bias", torch.float32), _dev(freq_ema, "freq_ema", torch.float32),
        _dev(current_freq, "current_freq", torch.float32), target_freq, gamma, bias_max, momentum, G,
        _stream(bias.device)), "update_load_balance_bias")


def update_load_balance_bias_from_counts(bias, freq_ema, counts, tokens: int, target_freq: float, gamma: float,
                                         bias_max: float, momentum: float):
    G = bias.numel()
    _check(lib().esg_update_load_balance_bias_from_counts(
        _dev(bias, "bias", torch.float32), _dev(freq_ema, "freq_ema", torch.float32),
        _dev(counts, "counts", torch.int32), tokens, target_freq, gamma, bias_max, momentum, G,
        _stream(bias.device)), "update_load_balance_bias_from_counts")


def update_load_balance_bias_from_routing(bias, freq_ema, ctx: FfnContext, target_freq: float, gamma: float,
                                          bias_max: float, momentum: float):
    """Bias update with the per-group counts of the routing a training forward saved in ``ctx``."""
    if ctx.saved is None or ctx.idx is None:
        raise EsgError("the context holds no saved routing (inference or dense forward)")
    _check(lib().esg_update_load_balance_bias_from_routing(
        _dev(bias, "bias", torch.float32), _dev(freq_ema, "freq_ema", torch.float32), _dev(ctx.saved, "saved"),
        ctx.saved.numel(), ctx.tokens, ctx.d_model, ctx.d_ff, ctx.group_size, ctx.k, ctx.dtype_code, target_freq,
        gamma, bias_max, momentum, _stream(bias.device)), "update_load_balance_bias_from_routing")


def leaky_mlp_workspace_size(tokens: int, d_model: int, d_ff: int):
    """(saved_bytes, scratch_bytes) of the LeakyReLU(0.5)^2 MLP."""
    sv, sc = _c_size(), _c_size()
    _check(lib().esg_leaky_mlp_workspace_size(tokens, d_model, d_ff, ctypes.byref(sv), ctypes.byref(sc)),
           "leaky_mlp_workspace_size")
    return sv.value, sc.value


def leaky_mlp_saved_views(saved: torch.Tensor, tokens: int, d_ff: int):
    """(post, act_grad) bf16 [tokens, d_ff] views of a forward's saved buffer."""
    n = tokens * d_ff
    off = (n * 2 + 255) // 256 * 256
    post = saved[: n * 2].view(torch.bfloat16).view(tokens, d_ff)
    act = saved[off: off + n * 2].view(torch.bfloat16).view(tokens, d_ff)
    return post, act


def leaky_mlp_fwd(x, w_up, w_down, out=None, saved=None):
    """y = LeakyReLU(0.5)(x W_up^T)^2 W_down^T (bf16).  Returns (y, saved): saved
    holds post and act_grad for leaky_mlp_bwd."""
    T, d = x.shape
    F = w_up.shape[0]
    if w_up.shape != (F, d) or w_down.shape != (d, F):
        raise EsgError("w_up must be [d_ff, d_model] and w_down [d_model, d_ff]")
    sv, _ = leaky_mlp_workspace_size(T, d, F)
    y = torch.empty_like(x) if out is None else out
    if saved is None or saved.numel() < sv:
        saved = torch.empty(max(sv, 1), dtype=torch.uint8, device=x.device)
    bf = torch.bfloat16
    _check(lib().esg_leaky_mlp_fwd(_dev(x, "x", bf), _dev(w_up, "w_up", bf), _dev(w_down, "w_down", bf), T, d, F,
                                   _dev(y, "y", bf), _dev(saved, "saved"), saved.numel(), _stream(x.device)),
           "leaky_mlp_fwd")
    return y, saved


def leaky_mlp_bwd(dy, x, w_up, w_down, saved, workspace: Optional[dict] = None, outs=None):
    """(dx, dW_up, dW_down) of the LeakyReLU(0.5)^2 MLP (overwritten)."""
    T, d = x.shape
    F = w_up.shape[0]
    _, sc = leaky_mlp_workspace_size(T, d, F)
    if outs is None:
        outs = (torch.empty_like(x), torch.empty_like(w_up), torch.empty_like(w_down))
    dx, dwu, dwd = outs
    scratch = _ws(sc, x.device, workspace, "mlp_scratch")
    bf = torch.bfloat16
    _check(lib().esg_leaky_mlp_bwd(_dev(dy, "dy", bf), _dev(x, "x", bf), _dev(w_up, "w_up", bf),
                                   _dev(w_down, "w_down", bf), T, d, F, _dev(saved, "saved"), _dev(dx, "dx", bf),
                                   _dev(dwu, "dw_up", bf), _dev(dwd, "dw_down", bf), _dev(scratch, "scratch"),
                                   scratch.numel(), _stream(x.device)), "leaky_mlp_bwd")
    return dx, dwu, dwd


def mhffn_supported(tokens: int, heads: int, d_head: int, subnets: int, d_sub: int) -> bool:
    return bool(lib().esg_mhffn_supported(tokens, heads, d_head, subnets, d_sub))


def mhffn_fwd(q, r, k, u, v, out=None):
    """O[t,h] = sum_e R[t,h,e] ((SiLU(Q K_e^T) * (Q U_e^T)) V_e) per head.
    q: bf16 [T, H, d_h]; r: float32 [T, H, E]; k, u, v: bf16 [H, E, d_e, d_h]."""
    T, H, dh = q.shape
    _, E, de, _ = k.shape
    if r.shape != (T, H, E) or u.shape != k.shape or v.shape != k.shape or k.shape[0] != H or k.shape[3] != dh:
        raise EsgError("shapes: q [T,H,d_h], r [T,H,E], k/u/v [H,E,d_e,d_h]")
    o = torch.empty_like(q) if out is None else out
    bf = torch.bfloat16
    _check(lib().esg_mhffn_fwd(_dev(q, "q", bf), _dev(r, "r", torch.float32), _dev(k, "k", bf), _dev(u, "u", bf),
                               _dev(v, "v", bf), T, H, dh, E, de, _dev(o, "out", bf), _stream(q.device)),
           "mhffn_fwd")
    return o


def mhffn_bwd(dout, q, r, k, u, v, outs=None):
    """(dQ, dR, dK, dU, dV) of the multi-head core (overwritten)."""
    T, H, dh = q.shape
    _, E, de, _ = k.shape
    if outs is None:
        outs = (torch.empty_like(q), torch.empty_like(r), torch.empty_like(k), torch.empty_like(u),
                torch.empty_like(v))
    dq, dr, dk, du, dv = outs
    bf, f32 = torch.bfloat16, torch.float32
    _check(lib().esg_mhffn_bwd(_dev(dout, "dout", bf), _dev(q, "q", bf), _dev(r, "r", f32), _dev(k, "k", bf),
                               _dev(u, "u", bf), _dev(v, "v", bf), T, H, dh, E, de, _dev(dq, "dq", bf),
                               _dev(dr, "dr", f32), _dev(dk, "dk", bf), _dev(du, "du", bf), _dev(dv, "dv", bf),
                               _stream(k.device)), "mhffn_bwd")
    return dq, dr, dk, du, dv


def sigmoid_topk_supported(num_experts: int, topk: int) -> bool:
    """Whether the routing kernel takes this shape (1 <= topk <= min(32, E), E <= 2048)."""
    return bool(lib().esg_sigmoid_topk_supported(num_experts, topk))


def sigmoid_topk_routing(logits, expert_bias, topk: int, scaling_factor: Optional[float] = None, out=None):
    """Top-k of sigmoid(logits) + bias per row; weights from sigmoid(logits),
    normalised by their left-folded sum (+1e-20) and optionally scaled.

    logits: float32 [T, E] contiguous GPU tensor; expert_bias: float32 [E]
    (a strided view is accepted).  Returns (probs float32 [T, k], indices
    int64 [T, k]); ``out`` may supply both."""
    if logits.dim() != 2:
        raise EsgError("logits must be [tokens, num_experts]")
    T, E = logits.shape
    if expert_bias.dim() != 1 or expert_bias.shape[0] != E or expert_bias.dtype != torch.float32:
        raise EsgError("expert_bias must be float32 [num_experts]")
    if not expert_bias.is_cuda or expert_bias.device != logits.device:
        raise EsgError("expert_bias must be on the logits' GPU")
    stride = expert_bias.stride(0) if E > 1 else 1
    if stride < 1:
        raise EsgError("expert_bias must have a positive stride")
    if out is None:
        probs = torch.empty(T, topk, dtype=torch.float32, device=logits.device)
        indices = torch.empty(T, topk, dtype=torch.int64, device=logits.device)
    else:
        probs, indices = out
    _check(lib().esg_sigmoid_topk_routing(
        _dev(logits, "logits", torch.float32), expert_bias.data_ptr(), stride, T, E, topk,
        1.0 if scaling_factor is None else float(scaling_factor), int(scaling_factor is not None),
        _dev(probs, "probs", torch.float32), _dev(indices, "indices", torch.int64), _stream(logits.device)),
        "sigmoid_topk_routing")
    return probs, indices


def mfma_rate_probe(blocks: int, iters: int, out: torch.Tensor) -> None:
    """Launch the bf16 matrix-core rate probe on the current stream (a
    measurement helper): blocks * 4 waves * iters * 8 MFMAs of 16x16x32.
    out: float32 device tensor of at least blocks * 256 elements."""
    if out.dtype != torch.float32 or not out.is_cuda or out.numel() < blocks * 256:
        raise ValueError("out must be a float32 device tensor of blocks * 256 elements")
    _check(lib().esg_mfma_rate_probe(blocks, iters, _dev(out, "out"), _stream(out.device)), "mfma_rate_probe")


def timing_enable(on: bool = True) -> None:
    _check(lib().esg_timing_enable(int(on)), "timing_enable")


def timing_reset() -> None:
    _check(lib().esg_timing_reset(), "timing_reset")


def timing_read(kernel: str):
    """(total milliseconds, launches) of a library kernel since the last reset."""
    ms, n = ctypes.c_double(), _c_int()
    _check(lib().esg_timing_read(kernel.encode(), ctypes.byref(ms), ctypes.byref(n)), "timing_read")
    return ms.value, n.value
