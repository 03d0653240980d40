"""Python binding of libmoe: the sparse mixture-of-experts FFN forward with
expert capacity, as hand-written HIP kernels for MI355X (gfx950).

This module only marshals arguments: every step of the layer runs in the HIP
kernels behind the C ABI of include/moe.h.  PyTorch is used for device
memory (tensors are passed by ``data_ptr()``) and streams.  Importing it
loads ``libmoe.so`` built in-tree by ``sparse_mixture_experts_capacity_amd.build``
and raises if it is missing: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import numpy as np

from ._lib import (LIB, MoeConfig, MoeStats, MoeError, MOE_OK, MOE_EINVAL,  # noqa: F401
                   MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_EHIP, DTYPE_F32,
                   DTYPE_BF16, TOPK_THEN_SOFTMAX, SOFTMAX_THEN_TOPK, PATH_AUTO,
                   PATH_GROUPED, PATH_STREAM, OVERFLOW_DROP, OVERFLOW_REROUTE,
                   OVERFLOW_SEQUENTIAL, WEIGHTS_ROW_MAJOR, WEIGHTS_PACKED,
                   EXPORTED_SYMBOLS)

__all__ = [
    "MoeConfig", "MoeStats", "MoeError", "make_config", "moe_check_config",
    "moe_workspace_size", "moe_capacity", "moe_forward", "moe_forward_noalloc", "moe_route",
    "moe_route_logits", "moe_aux_loss", "moe_router_backward", "moe_last_error",
    "moe_packed_weight_bytes", "moe_pack_weights", "moe_entropy_coef", "moe_lb_trend",
    "moe_debug_canaries", "moe_debug_check",
    "LoadBalanceTrend",
    "moe_timing_enable", "moe_timing_only",
    "moe_timing_reset", "moe_timing_read", "Workspace",
]


def _ptr(t) -> Optional[int]:
    """Device address of a torch tensor (or an int / None passed through)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream_handle(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_config(T: int, d_model: int, d_ff: int, n_experts: int, top_k: int,
                n_shared: int = 0, gating: int = TOPK_THEN_SOFTMAX,
                renormalize: bool = True, capacity_factor: float = 0.0,
                dtype: str = "bf16", ffn_path: int = PATH_AUTO,
                logit_bias=None, workspace=None, workspace_bytes: int = 0,
                stream=0, overflow: int = OVERFLOW_DROP,
                weight_layout: int = WEIGHTS_ROW_MAJOR, out_fp32: bool = False) -> MoeConfig:
    """Fill a moe_config_t.  ``stream`` = None means torch's current stream.
    ``out_fp32``: the layer writes ``out`` as fp32 whatever its dtype."""
    c = MoeConfig()
    c.T = int(T)
    c.d_model = int(d_model)
    c.d_ff = int(d_ff)
    c.n_experts = int(n_experts)
    c.top_k = int(top_k)
    c.n_shared = int(n_shared)
    c.gating = int(gating)
    c.renormalize = 1 if renormalize else 0
    c.capacity_factor = float(capacity_factor)
    c.dtype = DTYPE_BF16 if dtype in ("bf16", DTYPE_BF16) else DTYPE_F32
    c.ffn_path = int(ffn_path)
    c.logit_bias = _ptr(logit_bias)
    c.workspace = _ptr(workspace)
    c.workspace_bytes = int(workspace_bytes)
    c.stream = _stream_handle(stream) if stream != 0 else None
    c.overflow = int(overflow)
    c.weight_layout = int(weight_layout)
    c.out_fp32 = int(out_fp32)
    return c


def _check(rc: int, what: str) -> int:
    if rc != MOE_OK:
        raise MoeError(rc, f"{what}: {LIB.moe_last_error().decode()}")
    return rc


def moe_check_config(cfg: MoeConfig) -> int:
    """Status of host-side validation (no exception; no GPU needed)."""
    return LIB.moe_check_config(ctypes.byref(cfg))


def moe_workspace_size(cfg: MoeConfig) -> int:
    return int(LIB.moe_workspace_size(ctypes.byref(cfg)))


def moe_capacity(cfg: MoeConfig) -> int:
    return int(LIB.moe_capacity(ctypes.byref(cfg)))


def moe_last_error() -> str:
    return LIB.moe_last_error().decode()


class Workspace:
    """A device scratch buffer (torch uint8 tensor, 256-byte aligned) bound
    to a config."""

    def __init__(self, nbytes: int, device="cuda"):
        import torch
        self.nbytes = int(nbytes)
        self.buf = torch.empty(max(self.nbytes, 1) + 256, dtype=torch.uint8,
                               device=device)
        base = self.buf.data_ptr()
        self.ptr = (base + 255) // 256 * 256

    def bind(self, cfg: MoeConfig) -> MoeConfig:
        cfg.workspace = self.ptr
        cfg.workspace_bytes = self.nbytes
        return cfg


def _stats_struct(E: int):
    st = MoeStats()
    counts = np.zeros(E, dtype=np.int64)
    kept = np.zeros(E, dtype=np.int64)
    st.counts = counts.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    st.kept = kept.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    return st, counts, kept


def _stats_dict(st, counts, kept) -> dict:
    return dict(capacity=st.capacity, assignments=st.assignments,
                dropped=st.dropped, counts=counts.copy(), kept=kept.copy(),
                aux_loss=st.aux_loss, aux_loss_kept=st.aux_loss_kept,
                overflow_rate=st.overflow_rate, entropy_load=st.entropy_load,
                entropy_token=st.entropy_token, overflowed=st.overflowed,
                rerouted=st.rerouted, rounds=st.rounds)


def moe_forward(x, W_gate, W1, W3, W2, cfg: MoeConfig, out,
                stats: bool = False):
    """Layer forward into ``out``.  Returns the statistics dict when
    ``stats`` is true (this waits for the stream), else None."""
    st = counts = kept = None
    if stats:
        st, counts, kept = _stats_struct(cfg.n_experts)
    rc = LIB.moe_forward(_ptr(x), _ptr(W_gate), _ptr(W1), _ptr(W3), _ptr(W2),
                         ctypes.byref(cfg), _ptr(out),
                         ctypes.byref(st) if st is not None else None)
    _check(rc, "moe_forward")
    return _stats_dict(st, counts, kept) if stats else None


def moe_forward_noalloc(x, W_gate, W1, W3, W2, cfg: MoeConfig, out,
                        stats: bool = False):
    """moe_forward with the library's fixed scratch array instead of a
    workspace (cfg.workspace is ignored): for callers that cannot allocate."""
    st = counts = kept = None
    if stats:
        st, counts, kept = _stats_struct(cfg.n_experts)
    rc = LIB.moe_forward_noalloc(_ptr(x), _ptr(W_gate), _ptr(W1), _ptr(W3), _ptr(W2),
                                 ctypes.byref(cfg), _ptr(out),
                                 ctypes.byref(st) if st is not None else None)
    _check(rc, "moe_forward_noalloc")
    return _stats_dict(st, counts, kept) if stats else None


def moe_route(x, W_gate, cfg: MoeConfig, logits=None, topk_idx=None,
              topk_w=None, counts=None, offsets=None, perm=None, slot=None,
              stats: bool = False):
    st = c = k = None
    if stats:
        st, c, k = _stats_struct(cfg.n_experts)
    rc = LIB.moe_route(_ptr(x), _ptr(W_gate), ctypes.byref(cfg), _ptr(logits),
                       _ptr(topk_idx), _ptr(topk_w), _ptr(counts),
                       _ptr(offsets), _ptr(perm), _ptr(slot),
                       ctypes.byref(st) if st is not None else None)
    _check(rc, "moe_route")
    return _stats_dict(st, c, k) if stats else None


def moe_route_logits(logits, cfg: MoeConfig, topk_idx=None, topk_w=None,
                     counts=None, offsets=None, perm=None, slot=None,
                     stats: bool = False):
    st = c = k = None
    if stats:
        st, c, k = _stats_struct(cfg.n_experts)
    rc = LIB.moe_route_logits(_ptr(logits), ctypes.byref(cfg), _ptr(topk_idx),
                              _ptr(topk_w), _ptr(counts), _ptr(offsets),
                              _ptr(perm), _ptr(slot),
                              ctypes.byref(st) if st is not None else None)
    _check(rc, "moe_route_logits")
    return _stats_dict(st, c, k) if stats else None


def moe_router_backward(x, W_gate, dout, cfg: MoeConfig, dlogits, dW_gate=None,
                        dbias=None, dx=None, aux_coef: float = 0.0,
                        entropy_coef: float = 0.0) -> None:
    """Router gradients after ``moe_forward`` with the same cfg and workspace
    (see include/moe.h)."""
    rc = LIB.moe_router_backward(_ptr(x), _ptr(W_gate), _ptr(dout), float(aux_coef),
                                 float(entropy_coef), ctypes.byref(cfg), _ptr(dlogits),
                                 _ptr(dW_gate), _ptr(dbias), _ptr(dx))
    _check(rc, "moe_router_backward")


def moe_aux_loss(logits, counts, cfg: MoeConfig) -> float:
    v = ctypes.c_double(0.0)
    rc = LIB.moe_aux_loss(_ptr(logits), _ptr(counts), ctypes.byref(cfg),
                          ctypes.byref(v))
    _check(rc, "moe_aux_loss")
    return v.value


def moe_packed_weight_bytes(cfg: MoeConfig):
    """(bytes of packed W1 = of packed W3, bytes of packed W2)."""
    a, b = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check(LIB.moe_packed_weight_bytes(ctypes.byref(cfg), ctypes.byref(a), ctypes.byref(b)),
           "moe_packed_weight_bytes")
    return a.value, b.value


def moe_pack_weights(W1, W3, W2, cfg: MoeConfig, W1p, W3p, W2p) -> None:
    """Write the packed copies of W1, W3, W2 into W1p, W3p, W2p (enqueued on
    cfg.stream)."""
    _check(LIB.moe_pack_weights(_ptr(W1), _ptr(W3), _ptr(W2), ctypes.byref(cfg), _ptr(W1p),
                                _ptr(W3p), _ptr(W2p)), "moe_pack_weights")


def moe_debug_canaries(enable: bool = True) -> None:
    """Workspace guards after every region (size workspaces after this)."""
    LIB.moe_debug_canaries(1 if enable else 0)


def moe_debug_check(cfg: MoeConfig) -> int:
    """Number of overwritten workspace guards of cfg.workspace (waits for
    cfg.stream)."""
    rc = LIB.moe_debug_check(ctypes.byref(cfg))
    if rc < 0:
        _check(rc, "moe_debug_check")
    return rc


def moe_entropy_coef(step: int, total_steps: int, high: float, low: float) -> float:
    """Weight of the mean router entropy in the loss at ``step`` (include/moe.h)."""
    return float(LIB.moe_entropy_coef(int(step), int(total_steps), float(high), float(low)))


def moe_lb_trend(values) -> tuple:
    """(slope per step, mean) of a series of load-balancing losses, oldest
    first (include/moe.h)."""
    v = np.ascontiguousarray(np.asarray(values, dtype=np.float64))
    slope, mean = ctypes.c_double(0.0), ctypes.c_double(0.0)
    _check(LIB.moe_lb_trend(v.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), int(v.size),
                            ctypes.byref(slope), ctypes.byref(mean)), "moe_lb_trend")
    return slope.value, mean.value


class LoadBalanceTrend:
    """The aux losses of the last ``window`` training steps (``add`` one per
    step, e.g. ``stats["aux_loss"]`` of the forward); ``slope()`` and
    ``mean()`` come from moe_lb_trend over that window."""

    def __init__(self, window: int = 100):
        if window < 2:
            raise ValueError("window must be at least 2")
        from collections import deque
        self.window = int(window)
        self._vals = deque(maxlen=self.window)
        self.steps = 0

    def add(self, aux_loss: float) -> None:
        self._vals.append(float(aux_loss))
        self.steps += 1

    def __len__(self) -> int:
        return len(self._vals)

    def last(self):
        return self._vals[-1] if self._vals else None

    def slope(self):
        return moe_lb_trend(list(self._vals))[0] if len(self._vals) >= 2 else None

    def mean(self):
        return moe_lb_trend(list(self._vals))[1] if len(self._vals) >= 2 else (
            self._vals[0] if self._vals else None)


def moe_timing_enable(enable: bool = True) -> None:
    LIB.moe_timing_enable(1 if enable else 0)


def moe_timing_only(names=None) -> None:
    """Time only the named kernels (a name or an iterable of names, as
    moe_timing_read reports them); None times every kernel."""
    if names is None:
        LIB.moe_timing_only(None)
    else:
        if isinstance(names, str):
            names = [names]
        LIB.moe_timing_only(",".join(names).encode())


def moe_timing_reset() -> None:
    LIB.moe_timing_reset()


def moe_timing_read(max_kernels: int = 64) -> dict:
    """{kernel name: (launches, total ms)} since the last reset."""
    names = ctypes.create_string_buffer(64 * max_kernels)
    launches = (ctypes.c_int64 * max_kernels)()
    total = (ctypes.c_double * max_kernels)()
    n = LIB.moe_timing_read(names, launches, total, max_kernels)
    res = {}
    for i in range(min(n, max_kernels)):
        nm = names.raw[64 * i:64 * (i + 1)].split(b"\0", 1)[0].decode()
        res[nm] = (int(launches[i]), float(total[i]))
    return res
