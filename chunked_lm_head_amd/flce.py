"""Python binding of libflce.so (argument marshalling only).

Every step of the computation runs in the HIP kernels behind the C ABI of
``include/flce.h``; this module checks tensor dtypes, devices and layouts,
allocates outputs and the workspace with PyTorch, and passes raw pointers and
the current HIP stream.  There is no fallback: if the library is missing the
import fails.

The autograd wrapper follows the pattern of Unsloth's offloaded log-softmax
(GRPO long-context page, section "Auslagern von Aktivierungen fuer
Log-Softmax"): the forward keeps no logits, only what the backward needs to
recompute them (hidden states, lm_head, labels and the per-token lse).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# FLCE_LIB may name another build of the same library (e.g. to compare two builds).
LIB_PATH = os.environ.get("FLCE_LIB") or os.path.join(_HERE, "libflce.so")

MODE_NLL = 0
MODE_LOGPROB = 1
_MODES = {"nll": MODE_NLL, "logprob": MODE_LOGPROB}
STATUS = {0: "FLCE_OK", 1: "FLCE_ERR_ARG", 2: "FLCE_ERR_SHAPE", 3: "FLCE_ERR_WORKSPACE",
          4: "FLCE_ERR_UNSUPPORTED", 5: "FLCE_ERR_HIP"}
EXPORTS = ("flce_workspace_bytes", "flce_forward", "flce_backward", "flce_describe_plan",
           "flce_status_string", "flce_last_error", "flce_distill_workspace_bytes",
           "flce_distill", "flce_chunk_rows_for", "flce_tune", "flce_policy_workspace_bytes",
           "flce_grpo_loss", "flce_dpo_loss", "flce_kto_loss", "flce_distill_jsd",
           "flce_forward_noalloc", "flce_timing_begin", "flce_timing_end",
           "flce_kernel_name")


class LogitTransform(ctypes.Structure):
    """``flce_logit_transform``: multiply, divide, softcap, temperature (0 = skipped)."""
    _fields_ = [("scale_multiply", ctypes.c_float), ("scale_divide", ctypes.c_float),
                ("softcap", ctypes.c_float), ("temperature", ctypes.c_float)]


class PolicyParams(ctypes.Structure):
    """``flce_policy_params``: beta, GRPO's clip range, KTO's weights."""
    _fields_ = [("beta", ctypes.c_float), ("eps_low", ctypes.c_float),
                ("eps_high", ctypes.c_float), ("desirable_weight", ctypes.c_float),
                ("undesirable_weight", ctypes.c_float)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(LIB_PATH)
    i64, vp, f32p, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t
    lib.flce_workspace_bytes.argtypes = [i64, i64, i64, i64]
    lib.flce_workspace_bytes.restype = sz
    xp = ctypes.POINTER(LogitTransform)
    lib.flce_forward.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_int, xp,
                                 f32p, f32p, f32p, vp, sz, vp]
    lib.flce_forward.restype = ctypes.c_int
    lib.flce_forward_noalloc.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_int, xp,
                                         f32p, f32p, f32p, vp]
    lib.flce_forward_noalloc.restype = ctypes.c_int
    lib.flce_backward.argtypes = [vp, vp, vp, f32p, i64, i64, i64, i64, i64, ctypes.c_int,
                                  xp, f32p, f32p, vp, f32p, ctypes.c_int, vp, sz, vp]
    lib.flce_backward.restype = ctypes.c_int
    lib.flce_distill_workspace_bytes.argtypes = [i64, i64, i64, i64, i64]
    lib.flce_distill_workspace_bytes.restype = sz
    lib.flce_distill.argtypes = [vp, vp, i64, vp, vp, i64, vp, i64, i64, i64, i64, xp,
                                 f32p, f32p, f32p, f32p, vp, f32p, ctypes.c_int, vp, sz, vp]
    lib.flce_distill.restype = ctypes.c_int
    lib.flce_distill_jsd.argtypes = [vp, vp, i64, vp, vp, i64, vp, i64, i64, i64, i64, xp,
                                     ctypes.c_float, f32p, f32p, f32p, f32p, vp, f32p,
                                     ctypes.c_int, vp, sz, vp]
    lib.flce_distill_jsd.restype = ctypes.c_int
    lib.flce_chunk_rows_for.argtypes = [i64, i64]
    lib.flce_chunk_rows_for.restype = i64
    lib.flce_tune.argtypes = [i64, i64, i64, i64, sz, ctypes.POINTER(ctypes.c_int64),
                              ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_size_t)]
    lib.flce_tune.restype = ctypes.c_int
    pp = ctypes.POINTER(PolicyParams)
    lib.flce_policy_workspace_bytes.argtypes = [i64, i64, i64, i64, i64]
    lib.flce_policy_workspace_bytes.restype = sz
    head = [vp, vp, vp, i64, i64, i64, i64, i64, xp, i64]  # hidden .. transform, n_seq
    tail = [pp, f32p, f32p, f32p, vp, f32p, ctypes.c_int, vp, sz, vp]
    lib.flce_grpo_loss.argtypes = head + [f32p, f32p, f32p] + tail
    lib.flce_grpo_loss.restype = ctypes.c_int
    lib.flce_dpo_loss.argtypes = head + [f32p] + tail
    lib.flce_dpo_loss.restype = ctypes.c_int
    lib.flce_kto_loss.argtypes = head + [f32p, vp, f32p] + tail
    lib.flce_kto_loss.restype = ctypes.c_int
    lib.flce_describe_plan.argtypes = [i64, i64, i64, i64, ctypes.POINTER(ctypes.c_int64)]
    lib.flce_describe_plan.restype = ctypes.c_int
    lib.flce_status_string.argtypes = [ctypes.c_int]
    lib.flce_status_string.restype = ctypes.c_char_p
    lib.flce_last_error.argtypes = []
    lib.flce_last_error.restype = ctypes.c_char_p
    i32p = ctypes.POINTER(ctypes.c_int32)
    lib.flce_timing_begin.argtypes = [ctypes.c_int32]
    lib.flce_timing_begin.restype = ctypes.c_int
    lib.flce_timing_end.argtypes = [i32p, ctypes.POINTER(ctypes.c_float), ctypes.c_int32, i32p,
                                    i32p]
    lib.flce_timing_end.restype = ctypes.c_int
    lib.flce_kernel_name.argtypes = [ctypes.c_int32]
    lib.flce_kernel_name.restype = ctypes.c_char_p
    return lib


lib = _load()


class FlceError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        msg = lib.flce_last_error().decode() or lib.flce_status_string(status).decode()
        super().__init__(f"{STATUS.get(status, status)}: {msg}")


def _check(status: int) -> None:
    if status != 0:
        raise FlceError(status)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def make_transform(logit_scale_multiply: float = 0.0, logit_scale_divide: float = 0.0,
                   logit_softcapping: float = 0.0, temperature: float = 1.0):
    """The C struct for these values, or None (no transform) for the defaults.

    The library applies, per raw logit z: z * multiply (if nonzero), / divide
    (if nonzero), softcap * tanh(. / softcap) (if nonzero), / temperature, and
    checks the values (FLCE_ERR_ARG when out of range)."""
    vals = (float(logit_scale_multiply), float(logit_scale_divide), float(logit_softcapping),
            float(temperature))
    if vals == (0.0, 0.0, 0.0, 1.0):
        return None
    return ctypes.byref(LogitTransform(*vals))


def workspace_bytes(T: int, D: int, V: int, chunk_rows: int = 256) -> int:
    n = lib.flce_workspace_bytes(T, D, V, chunk_rows)
    if n == 0:
        raise ValueError(f"invalid shape T={T} D={D} V={V} chunk_rows={chunk_rows}")
    return n


PLAN_KEYS = ("token_tiles", "vocab_tiles", "fwd_splits", "row_block", "row_blocks",
             "vocab_chunk", "vocab_chunks", "dh_splits", "fwd_workspace", "bwd_workspace",
             "grad_tile_bytes", "chunk_logit_bytes")


def describe_plan(T: int, D: int, V: int, chunk_rows: int = 256) -> dict:
    info = (ctypes.c_int64 * 12)()
    _check(lib.flce_describe_plan(T, D, V, chunk_rows, info))
    return dict(zip(PLAN_KEYS, list(info)))


def timing_begin(capacity: int) -> None:
    """Turn the library's per-launch kernel timing on (``capacity`` HIP events on the
    current device): every kernel launched until ``timing_end`` is followed by an event
    on its stream."""
    _check(lib.flce_timing_begin(capacity))


def timing_end(capacity: int) -> tuple:
    """Turn timing off and return ([(kernel name, ms), ...] in launch order, number of
    kernels recorded, marks dropped for lack of events); ms is -1 where unknown."""
    ids = (ctypes.c_int32 * capacity)()
    ms = (ctypes.c_float * capacity)()
    n, dropped = ctypes.c_int32(), ctypes.c_int32()
    _check(lib.flce_timing_end(ids, ms, capacity, ctypes.byref(n), ctypes.byref(dropped)))
    rows = [(lib.flce_kernel_name(ids[i]).decode(), ms[i]) for i in range(min(n.value, capacity))]
    return rows, n.value, dropped.value


def chunk_rows_for(context_length: int, multiplier: int = 0) -> int:
    """Rows per chunk when each sequence is cut into ``multiplier`` chunks
    (0: the default max(4, context_length // 4096))."""
    n = lib.flce_chunk_rows_for(context_length, multiplier)
    if n == 0:
        raise ValueError(f"context_length = {context_length} must be >= 1")
    return n


def tune(batch: int, context_length: int, D: int, V: int, budget_bytes: int) -> dict:
    """Fewest hidden-state mini-batches, then the largest chunk (smallest multiplier
    not below the default), whose per-mini-batch device memory fits the budget."""
    m, cr, need = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_size_t()
    _check(lib.flce_tune(batch, context_length, D, V, budget_bytes, ctypes.byref(m),
                         ctypes.byref(cr), ctypes.byref(need)))
    return dict(mini_batches=m.value, chunk_rows=cr.value, bytes_needed=need.value)


def auto_tune(batch: int, context_length: int, D: int, V: int, device=None,
              fraction: float = 0.9) -> dict:
    """``tune`` against a fraction of the free memory the device reports now."""
    free, _ = torch.cuda.mem_get_info(device)
    return tune(batch, context_length, D, V, int(free * fraction))


def _validate(hidden: torch.Tensor, weight: torch.Tensor, labels: torch.Tensor) -> None:
    if hidden.dtype != torch.bfloat16 or weight.dtype != torch.bfloat16:
        raise TypeError("hidden and weight must be bfloat16")
    if labels.dtype != torch.int64:
        raise TypeError("labels must be int64")
    if hidden.dim() != 2 or weight.dim() != 2 or labels.dim() != 1:
        raise ValueError("hidden [T, D], weight [V, D], labels [T] expected")
    if hidden.shape[1] != weight.shape[1] or labels.shape[0] != hidden.shape[0]:
        raise ValueError("shape mismatch between hidden, weight and labels")
    for t in (hidden, weight, labels):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("tensors must be contiguous and on the GPU")
        if t.device != hidden.device:
            raise ValueError("tensors on different devices")


def _check_buffer(name: str, t: torch.Tensor, dtype, shape, device) -> None:
    """A caller-provided output or workspace: the library writes through its pointer, so its
    dtype, device, layout and size must be exactly what the call needs."""
    if t.dtype != dtype or t.device != device or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor on {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _check_workspace(t: torch.Tensor, need: int, device) -> None:
    if t.dtype != torch.uint8 or t.device != device or not t.is_contiguous() or t.dim() != 1:
        raise ValueError(f"workspace must be a contiguous 1-D uint8 tensor on {device}")
    if t.numel() < need:
        raise ValueError(f"workspace has {t.numel()} bytes, {need} needed")


def alloc_workspace(T: int, D: int, V: int, chunk_rows: int, device) -> torch.Tensor:
    return torch.empty(workspace_bytes(T, D, V, chunk_rows), dtype=torch.uint8, device=device)


def forward(hidden: torch.Tensor, weight: torch.Tensor, labels: torch.Tensor, *,
            ignore_index: int = -100, chunk_rows: int = 256, mode: str = "nll",
            transform: Optional[dict] = None,
            workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
            lse: Optional[torch.Tensor] = None, mean: Optional[torch.Tensor] = None):
    """(out [T], lse [T], mean []) fp32: per-token NLL or log-prob, lse, mean over used tokens.

    ``transform`` holds keyword arguments of :func:`make_transform`."""
    _validate(hidden, weight, labels)
    T, D = hidden.shape
    V = weight.shape[0]
    dev = hidden.device
    out = torch.empty(T, dtype=torch.float32, device=dev) if out is None else out
    lse = torch.empty(T, dtype=torch.float32, device=dev) if lse is None else lse
    mean = torch.empty((), dtype=torch.float32, device=dev) if mean is None else mean
    _check_buffer("out", out, torch.float32, (T,), dev)
    _check_buffer("lse", lse, torch.float32, (T,), dev)
    _check_buffer("mean", mean, torch.float32, (), dev)
    if workspace is None:
        workspace = alloc_workspace(T, D, V, chunk_rows, dev)
    _check_workspace(workspace, workspace_bytes(T, D, V, chunk_rows), dev)
    _check(lib.flce_forward(_ptr(hidden), _ptr(weight), _ptr(labels), T, D, V, ignore_index,
                            chunk_rows, _MODES[mode], make_transform(**(transform or {})),
                            _ptr(out), _ptr(lse), _ptr(mean),
                            _ptr(workspace), workspace.numel(), _stream(dev)))
    return out, lse, mean


def forward_noalloc(hidden: torch.Tensor, weight: torch.Tensor, labels: torch.Tensor, *,
                    ignore_index: int = -100, chunk_rows: int = 256, mode: str = "nll",
                    transform: Optional[dict] = None, out: torch.Tensor, lse: torch.Tensor,
                    mean: Optional[torch.Tensor] = None):
    """``forward`` through ``flce_forward_noalloc``: no workspace and nothing allocated
    here either (the caller passes the outputs); the library's fixed per-GPU array holds
    the partial results, so calls that can overlap on one GPU must not be made."""
    _validate(hidden, weight, labels)
    T, D = hidden.shape
    V = weight.shape[0]
    dev = hidden.device
    _check_buffer("out", out, torch.float32, (T,), dev)
    _check_buffer("lse", lse, torch.float32, (T,), dev)
    if mean is not None:
        _check_buffer("mean", mean, torch.float32, (), dev)
    _check(lib.flce_forward_noalloc(_ptr(hidden), _ptr(weight), _ptr(labels), T, D, V,
                                    ignore_index, chunk_rows, _MODES[mode],
                                    make_transform(**(transform or {})), _ptr(out), _ptr(lse),
                                    _ptr(mean), _stream(dev)))
    return out, lse, mean


def backward(hidden: torch.Tensor, weight: torch.Tensor, labels: torch.Tensor,
             lse: torch.Tensor, *, grad_out: Optional[torch.Tensor] = None,
             grad_mean: Optional[torch.Tensor] = None, ignore_index: int = -100,
             chunk_rows: int = 256, mode: str = "nll", transform: Optional[dict] = None,
             grad_hidden: Optional[torch.Tensor] = None,
             grad_weight: Optional[torch.Tensor] = None, accumulate: bool = False,
             workspace: Optional[torch.Tensor] = None, need_hidden: bool = True,
             need_weight: bool = True):
    """(dH [T, D] bf16, dW [V, D] fp32) of the loss given dL/d out (per token) or dL/d mean.

    ``need_hidden=False`` / ``need_weight=False`` skip that gradient (returned as None;
    e.g. a frozen lm_head skips the dW products)."""
    _validate(hidden, weight, labels)
    T, D = hidden.shape
    V = weight.shape[0]
    dev = hidden.device
    if (grad_out is None) == (grad_mean is None):
        raise ValueError("give exactly one of grad_out and grad_mean")
    _check_buffer("lse", lse, torch.float32, (T,), dev)
    if grad_out is not None:
        _check_buffer("grad_out", grad_out, torch.float32, (T,), dev)
    if grad_mean is not None:
        _check_buffer("grad_mean", grad_mean, torch.float32, (), dev)
    if not (need_hidden or need_weight):
        raise ValueError("nothing to compute: need_hidden and need_weight are both False")
    if not need_hidden:
        grad_hidden = None
    elif grad_hidden is None:
        grad_hidden = torch.empty((T, D), dtype=torch.bfloat16, device=dev)
    if not need_weight:
        grad_weight = None
    elif grad_weight is None:
        if accumulate:
            raise ValueError("accumulate needs an existing grad_weight")
        grad_weight = torch.empty((V, D), dtype=torch.float32, device=dev)
    if grad_hidden is not None:
        _check_buffer("grad_hidden", grad_hidden, torch.bfloat16, (T, D), dev)
    if grad_weight is not None:
        _check_buffer("grad_weight", grad_weight, torch.float32, (V, D), dev)
    if workspace is None:
        workspace = alloc_workspace(T, D, V, chunk_rows, dev)
    _check_workspace(workspace, workspace_bytes(T, D, V, chunk_rows), dev)
    _check(lib.flce_backward(_ptr(hidden), _ptr(weight), _ptr(labels), _ptr(lse), T, D, V,
                             ignore_index, chunk_rows, _MODES[mode],
                             make_transform(**(transform or {})), _ptr(grad_out),
                             _ptr(grad_mean), _ptr(grad_hidden), _ptr(grad_weight),
                             1 if accumulate else 0, _ptr(workspace), workspace.numel(),
                             _stream(dev)))
    return grad_hidden, grad_weight


def _offload(t: torch.Tensor) -> torch.Tensor:
    """Copy to pinned host memory, enqueued on the current stream."""
    h = torch.empty(t.shape, dtype=t.dtype, device="cpu", pin_memory=True)
    h.copy_(t, non_blocking=True)
    return h


class _ChunkedLinearCE(torch.autograd.Function):
    """Mean NLL (``reduction="mean"``) or per-token NLL / log-prob (``"none"``).

    As the Unsloth page's offloaded log-softmax (section "Auslagern von
    Aktivierungen fuer Log-Softmax"): the forward keeps no logits; the backward
    recomputes them.  With ``offload`` the saved hidden states wait in pinned
    host memory between the two (the caller's GPU copy may then be freed)."""

    @staticmethod
    def forward(ctx, hidden, weight, labels, ignore_index, chunk_rows, mode, reduction,
                transform, offload):
        out, lse, mean = forward(hidden, weight, labels, ignore_index=ignore_index,
                                 chunk_rows=chunk_rows, mode=mode, transform=transform)
        if offload:
            ctx.hidden_host = _offload(hidden)
            ctx.save_for_backward(weight, labels, lse)
        else:
            ctx.save_for_backward(hidden, weight, labels, lse)
        ctx.cfg = (ignore_index, chunk_rows, mode, reduction, transform, offload)
        return mean if reduction == "mean" else out

    @staticmethod
    def backward(ctx, grad):
        ignore_index, chunk_rows, mode, reduction, transform, offload = ctx.cfg
        if offload:
            weight, labels, lse = ctx.saved_tensors
            hidden = ctx.hidden_host.to(weight.device, non_blocking=True)
            del ctx.hidden_host
        else:
            hidden, weight, labels, lse = ctx.saved_tensors
        need_h, need_w = ctx.needs_input_grad[0], ctx.needs_input_grad[1]
        if not (need_h or need_w):
            return (None,) * 9
        g = grad.float().contiguous()
        kw = dict(grad_mean=g.reshape(())) if reduction == "mean" else dict(grad_out=g)
        dh, dw = backward(hidden, weight, labels, lse, ignore_index=ignore_index,
                          chunk_rows=chunk_rows, mode=mode, transform=transform,
                          need_hidden=need_h, need_weight=need_w, **kw)
        return (dh, None if dw is None else dw.to(weight.dtype), None, None, None, None, None,
                None, None)


def _transform_kwargs(logit_scale_multiply, logit_scale_divide, logit_softcapping, temperature):
    return dict(logit_scale_multiply=logit_scale_multiply, logit_scale_divide=logit_scale_divide,
                logit_softcapping=logit_softcapping, temperature=temperature)


def chunked_linear_cross_entropy(hidden, weight, labels, *, ignore_index=-100, chunk_rows=256,
                                 reduction="mean", logit_scale_multiply=0.0,
                                 logit_scale_divide=0.0, logit_softcapping=0.0,
                                 temperature=1.0, offload=False):
    """Autograd-aware chunked NLL of ``hidden @ weight.T`` against ``labels``.

    The logit transform arguments follow the chunked call of the Unsloth GRPO
    page (section "Chunking der abgeflachten Sequenzlaenge"); 0 skips a step."""
    xf = _transform_kwargs(logit_scale_multiply, logit_scale_divide, logit_softcapping,
                           temperature)
    return _ChunkedLinearCE.apply(hidden, weight, labels, ignore_index, chunk_rows, "nll",
                                  reduction, xf, offload)


def selective_log_softmax(hidden, weight, labels, *, ignore_index=-100, chunk_rows=256,
                          logit_scale_multiply=0.0, logit_scale_divide=0.0,
                          logit_softcapping=0.0, temperature=1.0, offload=False):
    """Autograd-aware per-token log p(label) without materialising the logits."""
    xf = _transform_kwargs(logit_scale_multiply, logit_scale_divide, logit_softcapping,
                           temperature)
    return _ChunkedLinearCE.apply(hidden, weight, labels, ignore_index, chunk_rows, "logprob",
                                  "none", xf, offload)


def mini_batched_log_softmax(hidden_fn, weight, labels, mini_batches: int, *,
                             grad_out: Optional[torch.Tensor] = None, ignore_index=-100,
                             chunk_rows=256, transform: Optional[dict] = None):
    """Selective log-softmax over a batch whose hidden states are produced one
    mini-batch of sequences at a time (the page's hidden-state mini-batching).

    ``hidden_fn(i, m)`` returns the [T_i, D] hidden states of mini-batch i of
    m (contiguous rows of the flattened batch, in order); ``labels`` covers the
    whole batch.  Returns (log p [T], and, if ``grad_out`` (dL/d log p) is
    given, dH [T, D] bf16 and dW [V, D] fp32 accumulated over the mini-batches).
    Only one mini-batch's hidden states and workspace are alive at a time."""
    T = labels.shape[0]
    dev = labels.device
    logp = torch.empty(T, dtype=torch.float32, device=dev)
    dh = dw = None
    r0 = 0
    for i in range(mini_batches):
        h = hidden_fn(i, mini_batches)
        r1 = r0 + h.shape[0]
        y = labels[r0:r1]
        out, lse, _ = forward(h, weight, y, ignore_index=ignore_index, chunk_rows=chunk_rows,
                              mode="logprob", transform=transform, out=logp[r0:r1])
        if grad_out is not None:
            if dh is None:
                dh = torch.empty((T, h.shape[1]), dtype=torch.bfloat16, device=dev)
                dw = torch.empty((weight.shape[0], weight.shape[1]), dtype=torch.float32,
                                 device=dev)
            backward(h, weight, y, lse, grad_out=grad_out[r0:r1], ignore_index=ignore_index,
                     chunk_rows=chunk_rows, mode="logprob", transform=transform,
                     grad_hidden=dh[r0:r1], grad_weight=dw, accumulate=i > 0)
        del h
        r0 = r1
    if r0 != T:
        raise ValueError(f"mini-batches cover {r0} rows, labels {T}")
    return logp, dh, dw


# ---------------------------------------------------------------------------
# Distillation (student and teacher heads over one vocabulary)
# ---------------------------------------------------------------------------

def distill_workspace_bytes(T: int, Ds: int, Dt: int, V: int, chunk_rows: int = 256) -> int:
    n = lib.flce_distill_workspace_bytes(T, Ds, Dt, V, chunk_rows)
    if n == 0:
        raise ValueError(f"invalid shape T={T} Ds={Ds} Dt={Dt} V={V} chunk_rows={chunk_rows}")
    return n


def distill(student_hidden, student_weight, teacher_hidden, teacher_weight,
            labels: Optional[torch.Tensor] = None, *, ignore_index: int = -100,
            chunk_rows: int = 256, transform: Optional[dict] = None,
            grad_out: Optional[torch.Tensor] = None, grad_mean: Optional[torch.Tensor] = None,
            grad_hidden: Optional[torch.Tensor] = None,
            grad_weight: Optional[torch.Tensor] = None, accumulate: bool = False,
            workspace: Optional[torch.Tensor] = None, kl: Optional[torch.Tensor] = None,
            mean: Optional[torch.Tensor] = None, divergence: str = "kl", beta: float = 0.5,
            need_hidden: bool = True, need_weight: bool = True):
    """(kl [T], mean [], dHs or None, dWs or None): per-token KL(teacher || student)
    (``divergence="jsd"``: the generalized JSD with weight ``beta``), its mean over
    kept tokens and, when grad_out or grad_mean is given, the student's gradients
    (one call; the teacher gets none; ``need_hidden`` / ``need_weight`` False skip one)."""
    if divergence not in ("kl", "jsd"):
        raise ValueError(f"divergence {divergence!r} is neither 'kl' nor 'jsd'")
    for t in (student_hidden, student_weight, teacher_hidden, teacher_weight):
        if t.dtype != torch.bfloat16 or t.dim() != 2 or not t.is_cuda or not t.is_contiguous():
            raise ValueError("hidden states and lm_heads must be contiguous 2-D bf16 on the GPU")
    T, Ds = student_hidden.shape
    V = student_weight.shape[0]
    Dt = teacher_hidden.shape[1]
    if (student_weight.shape[1] != Ds or teacher_hidden.shape[0] != T
            or tuple(teacher_weight.shape) != (V, Dt)):
        raise ValueError("shape mismatch between student and teacher tensors")
    dev = student_hidden.device
    if labels is not None and (labels.dtype != torch.int64 or labels.shape != (T,)
                               or not labels.is_contiguous() or labels.device != dev):
        raise ValueError("labels must be a contiguous int64 [T] mask on the same device")
    if grad_out is not None and grad_mean is not None:
        raise ValueError("give at most one of grad_out and grad_mean")
    grads = grad_out is not None or grad_mean is not None
    if grad_out is not None:
        _check_buffer("grad_out", grad_out, torch.float32, (T,), dev)
    if grad_mean is not None:
        _check_buffer("grad_mean", grad_mean, torch.float32, (), dev)
    kl = torch.empty(T, dtype=torch.float32, device=dev) if kl is None else kl
    mean = torch.empty((), dtype=torch.float32, device=dev) if mean is None else mean
    _check_buffer("kl", kl, torch.float32, (T,), dev)
    _check_buffer("mean", mean, torch.float32, (), dev)
    if grads:
        if not (need_hidden or need_weight):
            raise ValueError("nothing to compute: need_hidden and need_weight are both False")
        if not need_hidden:
            grad_hidden = None
        elif grad_hidden is None:
            grad_hidden = torch.empty((T, Ds), dtype=torch.bfloat16, device=dev)
        if not need_weight:
            grad_weight = None
        elif grad_weight is None:
            if accumulate:
                raise ValueError("accumulate needs an existing grad_weight")
            grad_weight = torch.empty((V, Ds), dtype=torch.float32, device=dev)
        if grad_hidden is not None:
            _check_buffer("grad_hidden", grad_hidden, torch.bfloat16, (T, Ds), dev)
        if grad_weight is not None:
            _check_buffer("grad_weight", grad_weight, torch.float32, (V, Ds), dev)
    else:
        grad_hidden = grad_weight = None
    need = distill_workspace_bytes(T, Ds, Dt, V, chunk_rows)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _check_workspace(workspace, need, dev)
    head = (_ptr(student_hidden), _ptr(student_weight), Ds, _ptr(teacher_hidden),
            _ptr(teacher_weight), Dt, _ptr(labels), ignore_index, T, V, chunk_rows,
            make_transform(**(transform or {})))
    tail = (_ptr(kl), _ptr(mean), _ptr(grad_out), _ptr(grad_mean), _ptr(grad_hidden),
            _ptr(grad_weight), 1 if accumulate else 0, _ptr(workspace), workspace.numel(),
            _stream(dev))
    if divergence == "kl":
        _check(lib.flce_distill(*head, *tail))
    else:
        _check(lib.flce_distill_jsd(*head, float(beta), *tail))
    return kl, mean, grad_hidden, grad_weight


class _ChunkedDistillKL(torch.autograd.Function):
    """Mean (``reduction="mean"``) or per-token (``"none"``) KL(teacher || student), or
    the generalized JSD.

    The forward call computes the divergence only; the backward calls the library
    again with the upstream gradient (dL/d mean as ``grad_mean``, or dL/d kl_t as
    ``grad_out``), which recomputes both heads' logits and applies it in the
    kernels, so the student's gradients are rounded once."""

    @staticmethod
    def forward(ctx, s_hidden, s_weight, t_hidden, t_weight, labels, ignore_index, chunk_rows,
                reduction, transform, divergence="kl", beta=0.5):
        kw = dict(ignore_index=ignore_index, chunk_rows=chunk_rows, transform=transform,
                  divergence=divergence, beta=beta)
        kl, mean, _, _ = distill(s_hidden, s_weight, t_hidden, t_weight, labels, **kw)
        ctx.save_for_backward(s_hidden, s_weight, t_hidden, t_weight, labels)
        ctx.cfg = (reduction, kw)
        return mean if reduction == "mean" else kl

    @staticmethod
    def backward(ctx, grad):
        reduction, kw = ctx.cfg
        need_h, need_w = ctx.needs_input_grad[0], ctx.needs_input_grad[1]
        if not (need_h or need_w):
            return (None,) * 11
        s_hidden, s_weight, t_hidden, t_weight, labels = ctx.saved_tensors
        g = grad.float().contiguous()
        gkw = dict(grad_mean=g.reshape(())) if reduction == "mean" else dict(grad_out=g)
        _, _, dh, dw = distill(s_hidden, s_weight, t_hidden, t_weight, labels,
                               need_hidden=need_h, need_weight=need_w, **gkw, **kw)
        return (dh, None if dw is None else dw.to(s_weight.dtype), None, None, None, None, None,
                None, None, None, None)


def chunked_distill_kl(student_hidden, student_weight, teacher_hidden, teacher_weight,
                       labels=None, *, ignore_index=-100, chunk_rows=256, reduction="mean",
                       logit_scale_multiply=0.0, logit_scale_divide=0.0, logit_softcapping=0.0,
                       temperature=1.0, divergence="kl", beta=0.5):
    """Autograd-aware KL(teacher || student) of two LM heads, chunked (gradients reach
    the student's hidden states and lm_head only); ``divergence="jsd"`` takes the
    generalized Jensen-Shannon divergence with weight ``beta`` instead."""
    xf = _transform_kwargs(logit_scale_multiply, logit_scale_divide, logit_softcapping,
                           temperature)
    return _ChunkedDistillKL.apply(student_hidden, student_weight, teacher_hidden,
                                   teacher_weight, labels, ignore_index, chunk_rows, reduction,
                                   xf, divergence, beta)


# ---------------------------------------------------------------------------
# Policy-optimisation losses (GRPO, DPO, KTO) on the selective log-softmax
# ---------------------------------------------------------------------------

def policy_workspace_bytes(T: int, D: int, V: int, chunk_rows: int, n_seq: int) -> int:
    n = lib.flce_policy_workspace_bytes(T, D, V, chunk_rows, n_seq)
    if n == 0:
        raise ValueError(f"invalid shape T={T} D={D} V={V} chunk_rows={chunk_rows} "
                         f"n_seq={n_seq}")
    return n


def _f32_input(name, t, shape, dev, optional=True):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    _check_buffer(name, t, torch.float32, shape, dev)
    return t


def _policy(kind, hidden, weight, labels, n_seq, extra, params, *, ignore_index, chunk_rows,
            transform, grad_loss, grad_hidden, grad_weight, accumulate, workspace, loss, logp,
            need_hidden=True, need_weight=True):
    _validate(hidden, weight, labels)
    T, D = hidden.shape
    V = weight.shape[0]
    dev = hidden.device
    loss = torch.empty((), dtype=torch.float32, device=dev) if loss is None else loss
    _check_buffer("loss", loss, torch.float32, (), dev)
    if logp is not None:
        _check_buffer("logp", logp, torch.float32, (T,), dev)
    grads = grad_loss is not None
    if grads:
        _check_buffer("grad_loss", grad_loss, torch.float32, (), dev)
        if not (need_hidden or need_weight):
            raise ValueError("nothing to compute: need_hidden and need_weight are both False")
        if not need_hidden:
            grad_hidden = None
        elif grad_hidden is None:
            grad_hidden = torch.empty((T, D), dtype=torch.bfloat16, device=dev)
        if not need_weight:
            grad_weight = None
        elif grad_weight is None:
            if accumulate:
                raise ValueError("accumulate needs an existing grad_weight")
            grad_weight = torch.empty((V, D), dtype=torch.float32, device=dev)
        if grad_hidden is not None:
            _check_buffer("grad_hidden", grad_hidden, torch.bfloat16, (T, D), dev)
        if grad_weight is not None:
            _check_buffer("grad_weight", grad_weight, torch.float32, (V, D), dev)
    else:
        grad_hidden = grad_weight = None
    need = policy_workspace_bytes(T, D, V, chunk_rows, n_seq)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _check_workspace(workspace, need, dev)
    fn = {"grpo": lib.flce_grpo_loss, "dpo": lib.flce_dpo_loss, "kto": lib.flce_kto_loss}[kind]
    _check(fn(_ptr(hidden), _ptr(weight), _ptr(labels), ignore_index, T, D, V, chunk_rows,
              make_transform(**(transform or {})), n_seq, *extra, ctypes.byref(params),
              _ptr(loss), _ptr(logp), _ptr(grad_loss), _ptr(grad_hidden), _ptr(grad_weight),
              1 if accumulate else 0, _ptr(workspace), workspace.numel(), _stream(dev)))
    return loss, logp, grad_hidden, grad_weight


def grpo_loss(hidden, weight, labels, n_seq: int, advantages, *, old_logp=None, ref_logp=None,
              beta: float = 0.0, eps_low: float = 0.2, eps_high: float = 0.2,
              ignore_index: int = -100, chunk_rows: int = 256, transform=None,
              grad_loss=None, grad_hidden=None, grad_weight=None, accumulate=False,
              workspace=None, loss=None, logp=None, need_hidden=True, need_weight=True):
    """GRPO loss over n_seq sequences of the flattened batch (``flce_grpo_loss``):
    (loss [], logp [T] or None, dH or None, dW or None)."""
    T = hidden.shape[0]
    dev = hidden.device
    extra = (_ptr(_f32_input("advantages", advantages, (n_seq,), dev, optional=False)),
             _ptr(_f32_input("old_logp", old_logp, (T,), dev)),
             _ptr(_f32_input("ref_logp", ref_logp, (T,), dev)))
    prm = PolicyParams(beta, eps_low, eps_high, 0.0, 0.0)
    return _policy("grpo", hidden, weight, labels, n_seq, extra, prm, ignore_index=ignore_index,
                   chunk_rows=chunk_rows, transform=transform, grad_loss=grad_loss,
                   grad_hidden=grad_hidden, grad_weight=grad_weight, accumulate=accumulate,
                   workspace=workspace, loss=loss, logp=logp, need_hidden=need_hidden,
                   need_weight=need_weight)


def dpo_loss(hidden, weight, labels, n_seq: int, ref_seq_logp, *, beta: float = 0.1,
             ignore_index: int = -100, chunk_rows: int = 256, transform=None, grad_loss=None,
             grad_hidden=None, grad_weight=None, accumulate=False, workspace=None, loss=None,
             logp=None, need_hidden=True, need_weight=True):
    """DPO loss; sequences [0, n_seq/2) chosen, [n_seq/2, n_seq) rejected (``flce_dpo_loss``)."""
    dev = hidden.device
    extra = (_ptr(_f32_input("ref_seq_logp", ref_seq_logp, (n_seq,), dev, optional=False)),)
    prm = PolicyParams(beta, 0.0, 0.0, 0.0, 0.0)
    return _policy("dpo", hidden, weight, labels, n_seq, extra, prm, ignore_index=ignore_index,
                   chunk_rows=chunk_rows, transform=transform, grad_loss=grad_loss,
                   grad_hidden=grad_hidden, grad_weight=grad_weight, accumulate=accumulate,
                   workspace=workspace, loss=loss, logp=logp, need_hidden=need_hidden,
                   need_weight=need_weight)


def kto_loss(hidden, weight, labels, n_seq: int, ref_seq_logp, desirable, *, kl_ref=None,
             beta: float = 0.1, desirable_weight: float = 1.0, undesirable_weight: float = 1.0,
             ignore_index: int = -100, chunk_rows: int = 256, transform=None, grad_loss=None,
             grad_hidden=None, grad_weight=None, accumulate=False, workspace=None, loss=None,
             logp=None, need_hidden=True, need_weight=True):
    """KTO loss with the reference point kl_ref (device scalar, clamped at 0; None = 0)
    (``flce_kto_loss``)."""
    dev = hidden.device
    _check_buffer("desirable", desirable, torch.uint8, (n_seq,), dev)
    extra = (_ptr(_f32_input("ref_seq_logp", ref_seq_logp, (n_seq,), dev, optional=False)),
             _ptr(desirable), _ptr(_f32_input("kl_ref", kl_ref, (), dev)))
    prm = PolicyParams(beta, 0.0, 0.0, desirable_weight, undesirable_weight)
    return _policy("kto", hidden, weight, labels, n_seq, extra, prm, ignore_index=ignore_index,
                   chunk_rows=chunk_rows, transform=transform, grad_loss=grad_loss,
                   grad_hidden=grad_hidden, grad_weight=grad_weight, accumulate=accumulate,
                   workspace=workspace, loss=loss, logp=logp, need_hidden=need_hidden,
                   need_weight=need_weight)


class _PolicyLossFn(torch.autograd.Function):
    """A policy loss as a scalar of the policy's hidden states and lm_head.

    The forward call computes the loss only; the backward calls the library again
    with the upstream scalar as ``grad_loss`` (the log-prob forward, the loss
    kernels and the recomputing backward), so the kernels apply it and dH is
    rounded once."""

    @staticmethod
    def forward(ctx, hidden, weight, call):
        loss, _, _, _ = call(hidden, weight, None, True, True)
        ctx.save_for_backward(hidden, weight)
        ctx.call = call
        return loss

    @staticmethod
    def backward(ctx, grad):
        need_h, need_w = ctx.needs_input_grad[0], ctx.needs_input_grad[1]
        if not (need_h or need_w):
            return None, None, None
        hidden, weight = ctx.saved_tensors
        _, _, dh, dw = ctx.call(hidden, weight, grad.float().reshape(()).contiguous(), need_h,
                                need_w)
        return dh, None if dw is None else dw.to(weight.dtype), None


def grpo_loss_fn(hidden, weight, labels, n_seq: int, advantages, **kw):
    """Autograd-aware ``grpo_loss`` (keyword arguments as there, without the gradient ones)."""
    return _PolicyLossFn.apply(hidden, weight, lambda h, w, gl, nh, nw: grpo_loss(
        h.detach(), w.detach(), labels, n_seq, advantages, grad_loss=gl, need_hidden=nh,
        need_weight=nw, **kw))


def dpo_loss_fn(hidden, weight, labels, n_seq: int, ref_seq_logp, **kw):
    """Autograd-aware ``dpo_loss``."""
    return _PolicyLossFn.apply(hidden, weight, lambda h, w, gl, nh, nw: dpo_loss(
        h.detach(), w.detach(), labels, n_seq, ref_seq_logp, grad_loss=gl, need_hidden=nh,
        need_weight=nw, **kw))


def kto_loss_fn(hidden, weight, labels, n_seq: int, ref_seq_logp, desirable, **kw):
    """Autograd-aware ``kto_loss``."""
    return _PolicyLossFn.apply(hidden, weight, lambda h, w, gl, nh, nw: kto_loss(
        h.detach(), w.detach(), labels, n_seq, ref_seq_logp, desirable, grad_loss=gl,
        need_hidden=nh, need_weight=nw, **kw))
