"""MI355X-native block-scaled (MXFP8 / NVFP4) quantization of MoE expert tensors.

Thin Python binding over the C ABI of ``libmxq.so`` (declared in
``include/mxq.h``).  PyTorch supplies device memory and the current HIP
stream; every quantization step runs in the library's HIP kernels.  The
binding only checks tensor metadata, allocates outputs when the caller does
not pass them, and forwards pointers.  There is no CPU fallback: without the
built library, or without GPU tensors, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

import torch

__all__ = [
    "MXFP8", "NVFP4", "LINEAR", "SWIZZLED", "MAX_GROUP", "SPLIT_MODES", "MxqError",
    "mx_quant_grouped", "nvfp4_quant_grouped_auto", "nvfp4_quant_split",
    "nvfp4_quant_split_row_scaled", "mxfp8_quant_split", "rmsnorm_quant_fused", "scale_swizzle",
    "GroupedCall", "GroupedAutoCall", "SplitCall", "FusedCall", "CHAIN", "issue_interleaved",
    "scale_bytes", "split_scale_offset", "set_max_workgroups", "library_path", "lib",
]

MXFP8, NVFP4 = 0, 1
LINEAR, SWIZZLED = 0, 1
MAX_GROUP = 16
CHAIN = 1  # mx_quant_grouped_batch flag: launches after the first dispatched any-order
_BLOCK = {MXFP8: 32, NVFP4: 16}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmxq.so")
_lib = None


class MxqError(RuntimeError):
    pass


class _Entry(ctypes.Structure):
    _fields_ = [("src", ctypes.c_void_p), ("payload", ctypes.c_void_p),
                ("scales", ctypes.c_void_p), ("global_scale", ctypes.c_void_p),
                ("rows", ctypes.c_int64), ("src_ld", ctypes.c_int64)]


def library_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """The loaded C library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise MxqError(f"{_LIB_PATH} is missing: build it with "
                           "`python -m nvfp4_quantization_moe_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        i64, vp, ci, cf = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        sigs = {
            "mx_quant_grouped": (ci, [ci, ci, i64, ctypes.POINTER(_Entry), ci, vp]),
            "mx_quant_grouped_batch": (ci, [ci, ci, i64, ctypes.POINTER(_Entry), ci, ci,
                                            ctypes.c_uint, vp]),
            "nvfp4_quant_grouped_auto": (ci, [ci, i64, ctypes.POINTER(_Entry), ci,
                                              ctypes.POINTER(ci), ci, vp, vp, vp]),
            "nvfp4_quant_split": (ci, [vp, i64, i64, ctypes.POINTER(i64), ci, vp, vp, vp, vp,
                                       ci, vp]),
            "nvfp4_quant_split_row_scaled": (ci, [vp, i64, i64, ctypes.POINTER(i64), ci, vp, vp,
                                                  vp, ci, vp]),
            "mxfp8_quant_split": (ci, [vp, i64, i64, ctypes.POINTER(i64), ci, vp, vp, vp, ci,
                                       vp]),
            "rmsnorm_quant_fused": (ci, [ci, ci, vp, vp, vp, cf, i64, i64, vp, vp, vp, vp, vp,
                                         vp]),
            "scale_swizzle": (ci, [vp, i64, i64, vp, vp]),
            "mxq_scale_bytes": (i64, [i64, i64, ci, ci]),
            "mxq_split_scale_offset": (i64, [ctypes.POINTER(i64), ci, ci, i64, ci, ci]),
            "mxq_status_str": (ctypes.c_char_p, [ci]),
            "mxq_set_max_workgroups": (None, [i64]),
        }
        for name, (res, args) in sigs.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(rc: int, what: str) -> None:
    if rc == 0:
        return
    msg = f"{what}: {lib().mxq_status_str(rc).decode()} (status {rc})"
    if rc in (1, 2):
        raise ValueError(msg)
    if rc == 3:
        raise NotImplementedError(msg)
    raise MxqError(msg)


def _stream(dev: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need_gpu(t: torch.Tensor, name: str, dtype=None) -> None:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def scale_bytes(rows: int, cols: int, fmt: int, layout: int) -> int:
    n = lib().mxq_scale_bytes(rows, cols, fmt, layout)
    if n < 0:
        raise ValueError("scale_bytes: invalid arguments")
    return n


def split_scale_offset(split_rows: Sequence[int], i: int, cols: int, fmt: int = NVFP4,
                       layout: int = SWIZZLED) -> int:
    arr = (ctypes.c_int64 * max(len(split_rows), 1))(*split_rows)
    n = lib().mxq_split_scale_offset(arr, len(split_rows), i, cols, fmt, layout)
    if n < 0:
        raise ValueError("split_scale_offset: invalid arguments")
    return n


def set_max_workgroups(n: int) -> None:
    """Debug knob: cap workgroups per launch (0 = default).  Outputs do not change."""
    lib().mxq_set_max_workgroups(int(n))


def _per_launch(max_per_launch) -> int:
    """The per-call expert cap: 1..MAX_GROUP; 1 is the one-launch-per-expert path."""
    n = int(max_per_launch)
    if n < 1 or n > MAX_GROUP:
        raise ValueError(f"max_per_launch must be in 1..{MAX_GROUP}, got {n}")
    return n


def mx_quant_grouped(fmt: int, layout: int, srcs: Sequence[torch.Tensor],
                     payloads: Optional[Sequence[torch.Tensor]] = None,
                     scales: Optional[Sequence[torch.Tensor]] = None,
                     global_scales: Optional[torch.Tensor] = None,
                     max_per_launch: int = MAX_GROUP):
    """Quantize same-width bf16 expert tensors, max_per_launch (1..16) per launch.

    srcs: 2-D bf16 GPU tensors [rows_i, cols] with unit column stride.
    global_scales: NVFP4 only, fp32 GPU tensor [len(srcs)] of encode scales.
    Returns (payloads, scales) lists of uint8 tensors (allocated when None):
    payload [rows, cols] (MXFP8) or [rows, cols/2] (NVFP4); scales flat,
    scale_bytes(rows, cols, fmt, layout) bytes.  The bytes do not depend on
    max_per_launch."""
    srcs = list(srcs)
    if not srcs:
        _per_launch(max_per_launch)
        return [], []
    call = GroupedCall(fmt, layout, srcs, payloads, scales, global_scales, max_per_launch)
    return call()


class GroupedCall:
    """Grouped quantization of same-width experts with the C descriptor array
    packed once: one mx_quant_grouped_batch call of max_per_launch (1..16)
    experts per launch on the current stream.

    For callers that issue the same grouped quantization repeatedly (a refit
    loop, a benchmark).  The tensors must stay alive and keep their storage.
    chain=True passes MXQ_CHAIN: launches after the first may start while the
    previous one drains (measured 348 -> 328 us on a Qwen3-30B-A3B layer's
    2 x 8 launches; no gain for launches of 300 MB and more)."""

    def __init__(self, fmt, layout, srcs, payloads=None, scales=None, global_scales=None,
                 max_per_launch=MAX_GROUP, chain=False):
        self.per = _per_launch(max_per_launch)
        self.fmt, self.layout = fmt, layout
        self.flags = CHAIN if chain else 0
        self.payloads, self.scales = _grouped_outputs(fmt, layout, srcs, payloads, scales,
                                                      global_scales)
        self.srcs = list(srcs)
        self.global_scales = global_scales
        self.cols = self.srcs[0].shape[1]
        self.device = self.srcs[0].device
        n = len(self.srcs)
        self._ents = (_Entry * n)()
        for i, s in enumerate(self.srcs):
            gs = None if fmt == MXFP8 else global_scales.data_ptr() + 4 * i
            self._ents[i] = _Entry(s.data_ptr(), self.payloads[i].data_ptr(),
                                   self.scales[i].data_ptr(), gs, s.shape[0], _row_stride(s))

    def __call__(self, stream: Optional[ctypes.c_void_p] = None):
        stream = _stream(self.device) if stream is None else stream
        _check(lib().mx_quant_grouped_batch(self.fmt, self.layout, self.cols, self._ents,
                                            len(self.srcs), self.per, self.flags, stream),
               "mx_quant_grouped_batch")
        return self.payloads, self.scales

    def issue(self, streams):
        """Issue launch j of this call (entries j*per .. j*per + per - 1) on
        streams[j % len(streams)], with no ordering against any other work:
        issue_interleaved orders the streams.  A launch position always goes
        to the same stream, so calls that reuse one set of outputs write each
        output from one stream."""
        n = len(self.srcs)
        size = ctypes.sizeof(_Entry)
        for j, b in enumerate(range(0, n, self.per)):
            ents = ctypes.cast(ctypes.byref(self._ents, b * size), ctypes.POINTER(_Entry))
            s = ctypes.c_void_p(streams[j % len(streams)].cuda_stream)
            _check(lib().mx_quant_grouped_batch(self.fmt, self.layout, self.cols, ents,
                                                min(self.per, n - b), self.per, 0, s),
                   "mx_quant_grouped_batch")
        return self.payloads, self.scales


def issue_interleaved(calls, streams):
    """Issue the launches of several GroupedCall objects over side streams.

    The streams (torch streams of the calls' device, default priority: work
    on streams of other priorities can starve) first wait for the work queued
    on the current stream; each call's launch j then goes to streams[j %
    len(streams)] (GroupedCall.issue); finally the current stream waits for
    every stream.  Launches on different streams may run at the same time,
    so no output may be written by two launches that land on different
    streams (calls that reuse one set of outputs with the same launch layout
    are safe: each output slice stays on one stream).  A process gets a few
    hardware queues (4 by default in HIP); streams beyond them share one and
    run one after another, so reuse a few side streams.  Two streams took a
    Qwen3-30B-A3B layer's 16 launches from 345 to 295 us per layer when the
    join covered 8 layers, 325 us when it covered one; launches of 300 MB and
    more gain about 1 %."""
    calls = list(calls)
    streams = list(streams)
    if not calls or not streams:
        raise ValueError("issue_interleaved needs at least one call and one stream")
    dev = calls[0].device
    for s in streams:
        if s.device != dev or s.priority != 0:
            raise ValueError("streams must be default-priority streams of the calls' device")
    for c in calls:
        if not isinstance(c, GroupedCall) or c.device != dev:
            raise ValueError("calls must be GroupedCall objects on one device")
    cur = torch.cuda.current_stream(dev)
    for s in streams:
        s.wait_stream(cur)
    for c in calls:
        c.issue(streams)
    for s in streams:
        cur.wait_stream(s)


class GroupedAutoCall:
    """nvfp4_quant_grouped_auto with its descriptor tables built once: NVFP4
    with per-slot encode scales computed from the data in the same call.

    slots: scale slot of each src (default: one per src).  Shared slots (the
    gate and up of one expert) must fall within one call of at most 16
    entries, so with shared slots len(srcs) <= 16; without, srcs are taken 16
    per call.  Calling returns (payloads, scales, g [n_slots], amax [n_slots])."""

    def __init__(self, layout, srcs, slots=None, payloads=None, scales=None, g_out=None,
                 amax_out=None):
        self.layout = layout
        self.srcs = list(srcs)
        n = len(self.srcs)
        if n == 0:
            raise ValueError("nvfp4_quant_grouped_auto needs at least one src")
        dummy_g = torch.ones(1, dtype=torch.float32, device=self.srcs[0].device)
        self.payloads, self.scales = _grouped_outputs(NVFP4, layout, self.srcs, payloads, scales,
                                                      dummy_g.expand(n).contiguous())
        if slots is not None:
            slots = [int(v) for v in slots]
            if n > MAX_GROUP or len(slots) != n or min(slots) < 0:
                raise ValueError("shared scale slots: at most 16 srcs, one slot index each")
            n_slots = max(slots) + 1
        else:
            n_slots = n
        dev = self.srcs[0].device
        self.g = torch.empty(n_slots, dtype=torch.float32, device=dev) if g_out is None else g_out
        self.amax = (torch.empty(n_slots, dtype=torch.float32, device=dev)
                     if amax_out is None else amax_out)
        _check_out(self.g, "g_out", torch.float32, n_slots, dev)
        _check_out(self.amax, "amax_out", torch.float32, n_slots, dev)
        self.cols = self.srcs[0].shape[1]
        self.device = dev
        self._batches = []
        for b in range(0, n, MAX_GROUP):
            m = min(MAX_GROUP, n - b)
            ents = (_Entry * m)()
            for j in range(m):
                i = b + j
                x = self.srcs[i]
                ents[j] = _Entry(x.data_ptr(), self.payloads[i].data_ptr(),
                                 self.scales[i].data_ptr(), None, x.shape[0], _row_stride(x))
            if slots is not None:
                sl, ns, off = (ctypes.c_int * m)(*slots), n_slots, 0
            else:
                sl, ns, off = None, m, b
            self._batches.append((ents, m, sl, ns, self.g.data_ptr() + 4 * off,
                                  self.amax.data_ptr() + 4 * off))

    def __call__(self, stream: Optional[ctypes.c_void_p] = None):
        stream = _stream(self.device) if stream is None else stream
        L = lib()
        for ents, m, sl, ns, gp, ap in self._batches:
            _check(L.nvfp4_quant_grouped_auto(self.layout, self.cols, ents, m, sl, ns, gp, ap,
                                              stream), "nvfp4_quant_grouped_auto")
        return self.payloads, self.scales, self.g, self.amax


def nvfp4_quant_grouped_auto(layout: int, srcs: Sequence[torch.Tensor], slots=None,
                             payloads=None, scales=None, g_out=None, amax_out=None):
    """NVFP4 grouped quantization with encode scales from the data (see
    GroupedAutoCall).  Returns (payloads, scales, g, amax)."""
    return GroupedAutoCall(layout, srcs, slots, payloads, scales, g_out, amax_out)()


def _grouped_outputs(fmt, layout, srcs, payloads, scales, global_scales):
    srcs = list(srcs)
    cols = srcs[0].shape[-1]
    dev = srcs[0].device
    for i, s in enumerate(srcs):
        _need_gpu(s, f"srcs[{i}]", torch.bfloat16)
        # an empty tensor holds no data: its strides (possibly 0) are not checked
        if s.dim() != 2 or s.shape[1] != cols or s.device != dev or \
                (s.shape[0] > 0 and s.stride(1) != 1):
            raise ValueError(f"srcs[{i}]: expected a row-major [rows, {cols}] bf16 tensor on {dev}")
    if fmt == NVFP4:
        if global_scales is None:
            raise ValueError("NVFP4 needs global_scales")
        _need_gpu(global_scales, "global_scales", torch.float32)
        if global_scales.numel() != len(srcs) or not global_scales.is_contiguous():
            raise ValueError("global_scales must be a contiguous fp32 tensor with one value per src")
    pw = cols if fmt == MXFP8 else cols // 2
    if payloads is None:
        payloads = [torch.empty((s.shape[0], pw), dtype=torch.uint8, device=dev) for s in srcs]
    if scales is None:
        scales = [torch.empty(scale_bytes(s.shape[0], cols, fmt, layout), dtype=torch.uint8,
                              device=dev) for s in srcs]
    payloads, scales = list(payloads), list(scales)
    for i, (s, p, c) in enumerate(zip(srcs, payloads, scales)):
        _need_gpu(p, f"payloads[{i}]", torch.uint8)
        _need_gpu(c, f"scales[{i}]", torch.uint8)
        if p.device != dev or c.device != dev:
            raise ValueError(f"payloads[{i}] and scales[{i}] must be on {dev}")
        if p.numel() < s.shape[0] * pw or not p.is_contiguous():
            raise ValueError(f"payloads[{i}] too small or not contiguous")
        if c.numel() < scale_bytes(s.shape[0], cols, fmt, layout) or not c.is_contiguous():
            raise ValueError(f"scales[{i}] too small or not contiguous")
    return payloads, scales


def _row_stride(s: torch.Tensor) -> int:
    """Row stride in elements for the descriptor; an empty tensor's is its width."""
    return s.stride(0) if s.shape[0] > 0 else s.shape[1]


def _check_out(t, name, dtype, numel, dev):
    _need_gpu(t, name, dtype)
    if t.device != dev:
        raise ValueError(f"{name} must be on {dev}")
    if not t.is_contiguous() or t.numel() < numel:
        raise ValueError(f"{name}: needs a contiguous tensor of at least {numel} elements")


SPLIT_MODES = ("nvfp4", "nvfp4_row_scaled", "mxfp8")


class SplitCall:
    """A split quantization with its arguments checked and packed once.

    mode: "nvfp4" (one encode scale, global_scale required),
    "nvfp4_row_scaled" (per-row encode scales) or "mxfp8".  Outputs are
    allocated when None: payload [T, H] (MXFP8) or [T, H/2], the bulk scale
    buffer (expert i at split_scale_offset(split_rows, i, H, fmt, layout)) and
    row_amax [T] (always for row-scaled; otherwise when want_row_amax).
    Calling returns (payload, scales, row_amax).  The tensors must stay alive."""

    def __init__(self, mode, src, split_rows, layout=SWIZZLED, global_scale=None, payload=None,
                 scales=None, row_amax=None, want_row_amax=True):
        if mode not in SPLIT_MODES:
            raise ValueError(f"mode must be one of {SPLIT_MODES}")
        fmt = MXFP8 if mode == "mxfp8" else NVFP4
        _need_gpu(src, "src", torch.bfloat16)
        if src.dim() != 2 or not src.is_contiguous():
            raise ValueError("src must be a contiguous [T, H] bf16 tensor")
        T, H = src.shape
        dev = src.device
        split_rows = [int(v) for v in split_rows]
        pw = H if fmt == MXFP8 else H // 2
        total = split_scale_offset(split_rows, len(split_rows), H, fmt, layout)
        if payload is None:
            payload = torch.empty((T, pw), dtype=torch.uint8, device=dev)
        if scales is None:
            scales = torch.empty(total, dtype=torch.uint8, device=dev)
        if row_amax is None and (want_row_amax or mode == "nvfp4_row_scaled"):
            row_amax = torch.empty(T, dtype=torch.float32, device=dev)
        _check_out(payload, "payload", torch.uint8, T * pw, dev)
        _check_out(scales, "scales", torch.uint8, total, dev)
        if row_amax is not None:
            _check_out(row_amax, "row_amax", torch.float32, T, dev)
        if mode == "nvfp4":
            if global_scale is None:
                raise ValueError("nvfp4 split needs global_scale")
            _need_gpu(global_scale, "global_scale", torch.float32)
        self.mode, self.device = mode, dev
        self.src, self.global_scale = src, global_scale
        self.payload, self.scales, self.row_amax = payload, scales, row_amax
        arr = (ctypes.c_int64 * max(len(split_rows), 1))(*split_rows)
        head = (src.data_ptr(), T, H, arr, len(split_rows))
        if mode == "nvfp4":
            self._fn, self._args = "nvfp4_quant_split", head + (
                global_scale.data_ptr(), payload.data_ptr(), scales.data_ptr(),
                _ptr(row_amax), layout)
        elif mode == "nvfp4_row_scaled":
            self._fn, self._args = "nvfp4_quant_split_row_scaled", head + (
                payload.data_ptr(), scales.data_ptr(), row_amax.data_ptr(), layout)
        else:
            self._fn, self._args = "mxfp8_quant_split", head + (
                payload.data_ptr(), scales.data_ptr(), _ptr(row_amax), layout)
        self._arr = arr  # keep the split table alive

    def __call__(self, stream: Optional[ctypes.c_void_p] = None):
        stream = _stream(self.device) if stream is None else stream
        _check(getattr(lib(), self._fn)(*self._args, stream), self._fn)
        return self.payload, self.scales, self.row_amax


def nvfp4_quant_split(src: torch.Tensor, split_rows: Sequence[int], global_scale: torch.Tensor,
                      layout: int = SWIZZLED, payload: Optional[torch.Tensor] = None,
                      scales: Optional[torch.Tensor] = None,
                      row_amax: Optional[torch.Tensor] = None, want_row_amax: bool = True):
    """Quantize a concatenated bf16 activation [T, H] once and split it per
    expert.  Returns (payload [T, H/2], bulk scales, row_amax [T] or None);
    expert i's scales start at split_scale_offset(split_rows, i, H)."""
    return SplitCall("nvfp4", src, split_rows, layout, global_scale, payload, scales, row_amax,
                     want_row_amax)()


def nvfp4_quant_split_row_scaled(src: torch.Tensor, split_rows: Sequence[int],
                                 layout: int = SWIZZLED, payload: Optional[torch.Tensor] = None,
                                 scales: Optional[torch.Tensor] = None,
                                 row_amax: Optional[torch.Tensor] = None):
    """Row-scaled NVFP4 split: row r under its own encode scale from its amax.
    Returns (payload [T, H/2], bulk scales, row_amax [T])."""
    return SplitCall("nvfp4_row_scaled", src, split_rows, layout, None, payload, scales,
                     row_amax)()


def mxfp8_quant_split(src: torch.Tensor, split_rows: Sequence[int], layout: int = SWIZZLED,
                      payload: Optional[torch.Tensor] = None,
                      scales: Optional[torch.Tensor] = None,
                      row_amax: Optional[torch.Tensor] = None, want_row_amax: bool = True):
    """MXFP8 split.  Returns (payload [T, H], bulk scales, row_amax [T] or
    None); expert i's scales start at split_scale_offset(split_rows, i, H, MXFP8)."""
    return SplitCall("mxfp8", src, split_rows, layout, None, payload, scales, row_amax,
                     want_row_amax)()


class FusedCall:
    """rmsnorm_quant_fused with its arguments checked and packed once; calling
    returns (residual_out, norm_out, payload, scales).  The tensors must stay
    alive."""

    def __init__(self, x, residual, gamma, eps=1e-6, fmt=MXFP8, layout=SWIZZLED,
                 global_scale=None, out=None):
        _need_gpu(x, "x", torch.bfloat16)
        _need_gpu(residual, "residual", torch.bfloat16)
        _need_gpu(gamma, "gamma", torch.bfloat16)
        if x.dim() != 2 or not x.is_contiguous() or residual.shape != x.shape or \
                not residual.is_contiguous() or gamma.shape != (x.shape[1],) or \
                not gamma.is_contiguous():
            raise ValueError("x, residual: contiguous [T, H]; gamma: contiguous [H]")
        T, H = x.shape
        dev = x.device
        if residual.device != dev or gamma.device != dev:
            raise ValueError("x, residual and gamma must be on one device")
        if fmt == NVFP4:
            if global_scale is None:
                raise ValueError("NVFP4 needs global_scale")
            _need_gpu(global_scale, "global_scale", torch.float32)
            if global_scale.device != dev:
                raise ValueError(f"global_scale must be on {dev}")
        pw = H if fmt == MXFP8 else H // 2
        nb = lib().mxq_scale_bytes(T, H, fmt, layout)
        if nb < 0:
            raise ValueError("rmsnorm_quant_fused: bad H for this format")
        if out is None:
            out = (torch.empty_like(x), torch.empty_like(x),
                   torch.empty((T, pw), dtype=torch.uint8, device=dev),
                   torch.empty(nb, dtype=torch.uint8, device=dev))
        res_out, norm_out, payload, scales = out
        _check_out(res_out, "residual_out", torch.bfloat16, T * H, dev)
        _check_out(norm_out, "norm_out", torch.bfloat16, T * H, dev)
        _check_out(payload, "payload", torch.uint8, T * pw, dev)
        _check_out(scales, "scales", torch.uint8, nb, dev)
        self.device = dev
        self.keep = (x, residual, gamma, global_scale)
        self.out = (res_out, norm_out, payload, scales)
        self._args = (fmt, layout, x.data_ptr(), residual.data_ptr(), gamma.data_ptr(),
                      float(eps), T, H, _ptr(global_scale), res_out.data_ptr(),
                      norm_out.data_ptr(), payload.data_ptr(), scales.data_ptr())

    def __call__(self, stream: Optional[ctypes.c_void_p] = None):
        stream = _stream(self.device) if stream is None else stream
        _check(lib().rmsnorm_quant_fused(*self._args, stream), "rmsnorm_quant_fused")
        return self.out


def rmsnorm_quant_fused(x: torch.Tensor, residual: torch.Tensor, gamma: torch.Tensor,
                        eps: float = 1e-6, fmt: int = MXFP8, layout: int = SWIZZLED,
                        global_scale: Optional[torch.Tensor] = None, out=None):
    """residual_out = bf16(x + residual); norm_out = RMSNorm(residual_out) * gamma
    (bf16); payload/scales = fmt quantization of norm_out.  Returns
    (residual_out, norm_out, payload, scales)."""
    return FusedCall(x, residual, gamma, eps, fmt, layout, global_scale, out)()


def scale_swizzle(linear: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Linear [rows, sf_cols] uint8 scales -> flat swizzled 128x4 layout."""
    _need_gpu(linear, "linear", torch.uint8)
    if linear.dim() != 2 or not linear.is_contiguous():
        raise ValueError("linear must be a contiguous [rows, sf_cols] uint8 tensor")
    rows, C = linear.shape
    n = (-(-rows // 128) * 128) * (-(-C // 4) * 4)
    if out is None:
        out = torch.empty(n, dtype=torch.uint8, device=linear.device)
    _check_out(out, "out", torch.uint8, n, linear.device)
    rc = lib().scale_swizzle(linear.data_ptr(), rows, C, out.data_ptr(), _stream(linear.device))
    _check(rc, "scale_swizzle")
    return out
