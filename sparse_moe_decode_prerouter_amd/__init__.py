"""Python binding of the MI355X MoE block library (libmoe_prerouter.so).

Argument marshalling only: every step of the block runs in the library's HIP
kernels. PyTorch provides device memory, pinned host memory and streams.
The binding has the C ABI's names (moe_layer_create, moe_stage_experts,
moe_decode_step, moe_prefill, ...) plus a small `MoeLayer` convenience class.
Importing raises if the compiled library is absent: there is no other path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("MOE_PREROUTER_LIB", os.path.join(_HERE, "libmoe_prerouter.so"))

MOE_OK = 0
MOE_E_INVALID = -1
MOE_E_UNSUPPORTED = -2
MOE_E_CAPACITY = -3
MOE_E_HIP = -4
MOE_E_NOT_STAGED = -5
MOE_E_BAD_INDEX = -6
MOE_E_TIMEOUT = -7

MOE_ACT_F32 = 0
MOE_ACT_BF16 = 1
MOE_FUSE_NORM_RESIDUAL = 0x1
MOE_RESIDENT_STORE = 0x2
MOE_DEVICE_STAGING = 0x4
MOE_DOUBLE_SLAB = 0x8
MOE_STAGE_OFF = 0
MOE_STAGE_PREROUTED = 1
MOE_STAGE_ON_DEMAND = 2


class moe_layer_desc(ctypes.Structure):
    _fields_ = [
        ("d_model", ctypes.c_int), ("n_experts", ctypes.c_int), ("top_k", ctypes.c_int),
        ("d_ff", ctypes.c_int), ("d_ff_shared", ctypes.c_int), ("group_size", ctypes.c_int),
        ("lora_rank", ctypes.c_int), ("lora_alpha", ctypes.c_float), ("rms_eps", ctypes.c_float),
        ("act_dtype", ctypes.c_int), ("max_tokens", ctypes.c_int), ("slab_slots", ctypes.c_int),
        ("next_n_experts", ctypes.c_int), ("next_top_k", ctypes.c_int), ("flags", ctypes.c_uint),
        ("head_hidden", ctypes.c_int), ("shared_lora_rank", ctypes.c_int), ("shared_lora_alpha", ctypes.c_float),
    ]


class moe_layer_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "expert_store", "shared_blob", "shared_gate", "router", "router_bias", "head", "head_bias",
        "hist_cur", "hist_prev", "lora_a", "lora_b", "norm_gamma", "head_fc1", "head_fc1_onehot", "head_fc1_bias",
        "head_fc2", "shared_lora_a", "shared_lora_b", "shared_lora_ad", "shared_lora_bd")]


class moe_io(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "x_in", "y_out", "route_idx", "route_w", "used_idx", "used_w", "pred_idx", "pred_w",
        "hist_cur", "hist_prev")] + [("reactive", ctypes.c_int), ("self_rows", ctypes.c_int)]


class MoeError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {moe_status_str(code)} ({code})"
                         + (f", hip error {moe_last_hip_error()}" if code == MOE_E_HIP else ""))


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python sparse_moe_decode_prerouter_amd/build.py` "
            "(or __graft_entry__.build()) first. There is no non-HIP path.")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    sig = {
        "moe_expert_blob_bytes": (Z, [I, I, I]),
        "moe_layer_workspace_bytes": (Z, [P]),
        "moe_layer_create": (I, [P, P, P, Z, ctypes.POINTER(P)]),
        "moe_stage_experts": (I, [P, P, I, P]),
        "moe_stage_experts_device": (I, [P, P, I, I, P]),
        "moe_layer_use_buffer": (I, [P, I]),
        "moe_stack_set_staging": (I, [P, P, I]),
        "moe_layer_slots": (I, [P, P, I, P]),
        "moe_decode_step": (I, [P, P, I, P]),
        "moe_decode_noalloc": (I, [P, P, P, I, P, P]),
        "moe_prefill": (I, [P, P, I, P]),
        "moe_layer_sync_status": (I, [P]),
        "moe_layer_destroy": (None, [P]),
        "moe_status_str": (ctypes.c_char_p, [I]),
        "moe_last_hip_error": (I, []),
        "moe_plan_slots": (I, [P, I, P, I, I, P, P, P]),
        "moe_stack_workspace_bytes": (Z, [P, I]),
        "moe_stack_create": (I, [P, I, P, Z, ctypes.POINTER(P)]),
        "moe_stack_set_trace": (I, [P, P, Z]),
        "moe_stack_decode": (I, [P, P, P, I, P, P, P, P, P, P, P, I, P]),
        "moe_stack_prefill": (I, [P, P, I, P, P, P, P, P]),
        "moe_stack_destroy": (None, [P]),
        "moe_stack_set_one_launch": (I, [P, I]),
        "moe_stack_set_wait_limit": (I, [P, ctypes.c_uint]),
        "moe_stack_set_profiling": (I, [P, I]),
        "moe_stack_kernel_ms": (I, [P, P, P]),
        "moe_layer_set_profiling": (I, [P, I]),
        "moe_layer_kernel_ms": (I, [P, P, P, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()
EXPORTED = ("moe_expert_blob_bytes", "moe_layer_workspace_bytes", "moe_layer_create", "moe_stage_experts",
            "moe_stage_experts_device", "moe_layer_use_buffer", "moe_stack_set_staging",
            "moe_layer_slots", "moe_decode_step", "moe_decode_noalloc", "moe_prefill", "moe_layer_sync_status", "moe_layer_destroy",
            "moe_status_str", "moe_last_hip_error", "moe_plan_slots", "moe_stack_workspace_bytes",
            "moe_stack_create", "moe_stack_set_trace", "moe_stack_decode",
            "moe_stack_prefill", "moe_stack_destroy", "moe_stack_set_one_launch", "moe_stack_set_wait_limit", "moe_stack_set_profiling",
            "moe_stack_kernel_ms", "moe_layer_set_profiling", "moe_layer_kernel_ms")


# ---------------------------------------------------------------------------
# C-ABI functions under their own names
# ---------------------------------------------------------------------------
def moe_expert_blob_bytes(d_model: int, d_ff: int, group_size: int = 64) -> int:
    return _lib.moe_expert_blob_bytes(d_model, d_ff, group_size)


def moe_layer_workspace_bytes(desc: moe_layer_desc) -> int:
    return _lib.moe_layer_workspace_bytes(ctypes.byref(desc))


def moe_layer_create(desc: moe_layer_desc, w: moe_layer_weights, ws_ptr: int, ws_bytes: int) -> int:
    h = ctypes.c_void_p()
    rc = _lib.moe_layer_create(ctypes.byref(desc), ctypes.byref(w), ctypes.c_void_p(ws_ptr), ws_bytes,
                               ctypes.byref(h))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_layer_create")
    return h.value


def moe_stage_experts(handle: int, ids: Sequence[int], copy_stream: int = 0) -> None:
    arr = (ctypes.c_int32 * max(1, len(ids)))(*[int(i) for i in ids])
    rc = _lib.moe_stage_experts(handle, arr, len(ids), ctypes.c_void_p(copy_stream))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_stage_experts")


def moe_stage_experts_device(handle: int, ids_ptr: int, n_ids: int, buffer: int, stream: int = 0) -> None:
    rc = _lib.moe_stage_experts_device(handle, ids_ptr, n_ids, buffer, ctypes.c_void_p(stream))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_stage_experts_device")


def moe_layer_use_buffer(handle: int, buffer: int) -> None:
    rc = _lib.moe_layer_use_buffer(handle, buffer)
    if rc != MOE_OK:
        raise MoeError(rc, "moe_layer_use_buffer")


def moe_stack_set_staging(stack: int, copy_stream: int, mode: int) -> None:
    rc = _lib.moe_stack_set_staging(stack, ctypes.c_void_p(copy_stream), mode)
    if rc != MOE_OK:
        raise MoeError(rc, "moe_stack_set_staging")


def moe_layer_slots(handle: int, n_slots: int):
    arr = (ctypes.c_int32 * max(1, n_slots))()
    nb = ctypes.c_uint64()
    rc = _lib.moe_layer_slots(handle, arr, n_slots, ctypes.byref(nb))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_layer_slots")
    return list(arr)[:n_slots], nb.value


def moe_decode_step(handle: int, io: moe_io, n_tok: int, stream: int = 0) -> None:
    rc = _lib.moe_decode_step(handle, ctypes.byref(io), n_tok, ctypes.c_void_p(stream))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_decode_step")


def moe_decode_noalloc(desc: moe_layer_desc, w: moe_layer_weights, io: moe_io, n_tok: int,
                       status_ptr: Optional[int] = None, stream: int = 0) -> None:
    rc = _lib.moe_decode_noalloc(ctypes.byref(desc), ctypes.byref(w), ctypes.byref(io), n_tok, status_ptr,
                                 ctypes.c_void_p(stream))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_decode_noalloc")


def moe_prefill(handle: int, io: moe_io, n_tok: int, stream: int = 0) -> None:
    rc = _lib.moe_prefill(handle, ctypes.byref(io), n_tok, ctypes.c_void_p(stream))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_prefill")


def moe_layer_sync_status(handle: int) -> int:
    return _lib.moe_layer_sync_status(handle)


def moe_layer_destroy(handle: int) -> None:
    _lib.moe_layer_destroy(handle)


def moe_status_str(code: int) -> str:
    return _lib.moe_status_str(code).decode()


def moe_last_hip_error() -> int:
    return _lib.moe_last_hip_error()


def moe_plan_slots(resident: Sequence[int], wanted: Sequence[int], n_experts: int):
    """Pure host: returns (new_resident, copies [(slot, expert)]) or raises MoeError."""
    n = len(resident)
    res = (ctypes.c_int32 * max(1, n))(*resident)
    wa = (ctypes.c_int32 * max(1, len(wanted)))(*[int(x) for x in wanted])
    cs = (ctypes.c_int32 * max(1, n))()
    ce = (ctypes.c_int32 * max(1, n))()
    nc = ctypes.c_int()
    rc = _lib.moe_plan_slots(res, n, wa, len(wanted), n_experts, cs, ce, ctypes.byref(nc))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_plan_slots")
    return list(res)[:n], [(cs[i], ce[i]) for i in range(nc.value)]


def moe_stack_workspace_bytes(handles: Sequence[int]) -> int:
    arr = (ctypes.c_void_p * len(handles))(*handles)
    return _lib.moe_stack_workspace_bytes(arr, len(handles))


def moe_stack_create(handles: Sequence[int], ws_ptr: int, ws_bytes: int) -> int:
    arr = (ctypes.c_void_p * len(handles))(*handles)
    h = ctypes.c_void_p()
    rc = _lib.moe_stack_create(arr, len(handles), ctypes.c_void_p(ws_ptr), ws_bytes, ctypes.byref(h))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_stack_create")
    return h.value


def moe_stack_set_trace(stack: int, trace_ptr: Optional[int], n_floats: int) -> None:
    rc = _lib.moe_stack_set_trace(stack, trace_ptr, n_floats)
    if rc != MOE_OK:
        raise MoeError(rc, "moe_stack_set_trace")


def moe_stack_decode(stack: int, x_in: int, x_out: int, n_tok: int, route_idx: Optional[int],
                     route_w: Optional[int], pred_idx: int, pred_w: int, used_idx: Optional[int],
                     used_w: Optional[int], hist_prev: Optional[int], first_step: bool, stream: int = 0) -> None:
    rc = _lib.moe_stack_decode(stack, x_in, x_out, n_tok, route_idx, route_w, pred_idx, pred_w, used_idx, used_w,
                               hist_prev, 1 if first_step else 0, ctypes.c_void_p(stream))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_stack_decode")


def moe_stack_prefill(stack: int, x: int, n_tok: int, used_idx: Optional[int], used_w: Optional[int],
                      pred_idx: Optional[int], pred_w: Optional[int], stream: int = 0) -> None:
    rc = _lib.moe_stack_prefill(stack, x, n_tok, used_idx, used_w, pred_idx, pred_w, ctypes.c_void_p(stream))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_stack_prefill")


def moe_stack_destroy(stack: int) -> None:
    _lib.moe_stack_destroy(stack)


def moe_stack_set_one_launch(stack: int, enable: bool) -> None:
    rc = _lib.moe_stack_set_one_launch(stack, 1 if enable else 0)
    if rc != MOE_OK:
        raise MoeError(rc, "moe_stack_set_one_launch")


def moe_stack_set_wait_limit(stack: int, polls: int) -> None:
    rc = _lib.moe_stack_set_wait_limit(stack, polls)
    if rc != MOE_OK:
        raise MoeError(rc, "moe_stack_set_wait_limit")


def moe_stack_set_profiling(stack: int, enable: bool) -> None:
    rc = _lib.moe_stack_set_profiling(stack, 1 if enable else 0)
    if rc != MOE_OK:
        raise MoeError(rc, "moe_stack_set_profiling")


def moe_stack_kernel_ms(stack: int):
    r, m = ctypes.c_float(), ctypes.c_float()
    rc = _lib.moe_stack_kernel_ms(stack, ctypes.byref(r), ctypes.byref(m))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_stack_kernel_ms")
    return r.value, m.value


def moe_layer_set_profiling(handle: int, enable: bool) -> None:
    rc = _lib.moe_layer_set_profiling(handle, 1 if enable else 0)
    if rc != MOE_OK:
        raise MoeError(rc, "moe_layer_set_profiling")


def moe_layer_kernel_ms(handle: int):
    r, a, b = ctypes.c_float(), ctypes.c_float(), ctypes.c_float()
    rc = _lib.moe_layer_kernel_ms(handle, ctypes.byref(r), ctypes.byref(a), ctypes.byref(b))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_layer_kernel_ms")
    return r.value, a.value, b.value


# ---------------------------------------------------------------------------
# convenience wrapper over torch tensors
# ---------------------------------------------------------------------------
def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream_ptr(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


class MoeLayer:
    """One MoE layer bound to tensors the caller keeps alive (kept here too)."""

    def __init__(self, *, d_model, n_experts, top_k, d_ff, d_ff_shared, lora_rank, lora_alpha, act_dtype,
                 max_tokens, expert_store, shared_blob=None, shared_gate=None, router=None, router_bias=None,
                 head=None, head_bias=None, next_n_experts=0, next_top_k=0, hist_cur=None, hist_prev=None,
                 lora_a=None, lora_b=None, norm_gamma=None, rms_eps=1e-6, fuse_norm_residual=False,
                 resident=True, slab_slots=0, head_fc1=None, head_fc1_onehot=None, head_fc1_bias=None,
                 head_fc2=None, shared_lora_a=None, shared_lora_b=None, shared_lora_ad=None, shared_lora_bd=None,
                 shared_lora_alpha=0.0, device_staging=False, double_slab=False, device="cuda"):
        import torch
        self._keep = [expert_store, shared_blob, shared_gate, router, router_bias, head, head_bias, hist_cur,
                      hist_prev, lora_a, lora_b, norm_gamma, head_fc1, head_fc1_onehot, head_fc1_bias, head_fc2,
                      shared_lora_a, shared_lora_b, shared_lora_ad, shared_lora_bd]
        shared_lora_rank = 0 if shared_lora_a is None else int(shared_lora_a.shape[0]) // 2
        flags = (MOE_FUSE_NORM_RESIDUAL if fuse_norm_residual else 0) | (MOE_RESIDENT_STORE if resident else 0) \
            | (MOE_DEVICE_STAGING if device_staging else 0) | (MOE_DOUBLE_SLAB if double_slab else 0)
        head_hidden = 0 if head_fc1 is None else int(head_fc1.shape[0])
        self.desc = moe_layer_desc(d_model, n_experts, top_k, d_ff, d_ff_shared, 64, lora_rank, float(lora_alpha),
                                   float(rms_eps), act_dtype, max_tokens, slab_slots, next_n_experts, next_top_k,
                                   flags, head_hidden, shared_lora_rank, float(shared_lora_alpha))
        self.weights = moe_layer_weights(*[_ptr(t) for t in self._keep])
        nbytes = moe_layer_workspace_bytes(self.desc)
        if nbytes == 0:
            raise MoeError(MOE_E_UNSUPPORTED, "moe_layer_workspace_bytes")
        self.workspace = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
        base = self.workspace.data_ptr()
        self._ws_ptr = (base + 255) // 256 * 256
        self.handle = moe_layer_create(self.desc, self.weights, self._ws_ptr, nbytes)
        self.top_k = top_k
        self.next_top_k = next_top_k
        self.d_model = d_model
        self.slab_slots = slab_slots

    def stage(self, ids, stream=None):
        moe_stage_experts(self.handle, list(ids), _stream_ptr(stream))

    def slots(self):
        return moe_layer_slots(self.handle, self.slab_slots)

    def stage_device(self, ids, buffer=0, stream=None):
        """ids: device int32 tensor of routing entries."""
        moe_stage_experts_device(self.handle, ids.data_ptr(), ids.numel(), buffer, _stream_ptr(stream))

    def use_buffer(self, buffer):
        moe_layer_use_buffer(self.handle, buffer)

    def _io(self, x, y, route_idx, route_w, used, pred, hist_cur, hist_prev, reactive, self_rows=0):
        import torch
        n = x.shape[0]
        dev = x.device
        out = {"y": y}
        if used:
            out["used_idx"] = torch.empty((n, self.top_k), dtype=torch.int32, device=dev)
            out["used_w"] = torch.empty((n, self.top_k), dtype=torch.float32, device=dev)
        if pred:
            out["pred_idx"] = torch.empty((n, self.next_top_k), dtype=torch.int32, device=dev)
            out["pred_w"] = torch.empty((n, self.next_top_k), dtype=torch.float32, device=dev)
        io = moe_io(_ptr(x), _ptr(y), _ptr(route_idx), _ptr(route_w), _ptr(out.get("used_idx")),
                    _ptr(out.get("used_w")), _ptr(out.get("pred_idx")), _ptr(out.get("pred_w")),
                    _ptr(hist_cur), _ptr(hist_prev), 1 if reactive else 0, 1 if self_rows else 0)
        return io, out

    def decode(self, x, route_idx=None, route_w=None, *, y=None, used=True, pred=True, hist_cur=None,
               hist_prev=None, reactive=False, self_rows=False, stream=None):
        import torch
        if y is None:
            y = torch.empty((x.shape[0], self.d_model), dtype=torch.float32, device=x.device)
        io, out = self._io(x, y, route_idx, route_w, used, pred, hist_cur, hist_prev, reactive, self_rows)
        moe_decode_step(self.handle, io, x.shape[0], _stream_ptr(stream))
        return out

    def prefill(self, x, route_idx=None, route_w=None, *, y=None, used=True, pred=True, hist_cur=None,
                hist_prev=None, stream=None):
        import torch
        if y is None:
            y = torch.empty((x.shape[0], self.d_model), dtype=torch.float32, device=x.device)
        io, out = self._io(x, y, route_idx, route_w, used, pred, hist_cur, hist_prev, False)
        moe_prefill(self.handle, io, x.shape[0], _stream_ptr(stream))
        return out

    def status(self) -> int:
        return moe_layer_sync_status(self.handle)

    def set_profiling(self, enable: bool = True):
        moe_layer_set_profiling(self.handle, enable)

    def kernel_ms(self):
        return moe_layer_kernel_ms(self.handle)

    def close(self):
        if getattr(self, "handle", None):
            moe_layer_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class MoeStack:
    """A stack of MoeLayer objects driven one decode step at a time
    (moe_stack_decode). Routing buffers are [L][n_tok][k] device tensors; the
    step's predictions feed the next step, so callers rotate two buffers."""

    def __init__(self, layers, device="cuda"):
        import torch
        self.layers = list(layers)
        hs = [L.handle for L in self.layers]
        nbytes = moe_stack_workspace_bytes(hs)
        if nbytes == 0:
            raise MoeError(MOE_E_INVALID, "moe_stack_workspace_bytes")
        self.workspace = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
        self.handle = moe_stack_create(hs, (self.workspace.data_ptr() + 255) // 256 * 256, nbytes)
        self.k = self.layers[0].top_k
        self.trace = None

    def set_staging(self, mode, copy_stream=None):
        """Device staging driven by the stack (MOE_STAGE_PREROUTED / _ON_DEMAND / _OFF)."""
        self.copy_stream = copy_stream
        moe_stack_set_staging(self.handle, 0 if copy_stream is None else copy_stream.cuda_stream, mode)

    def set_one_launch(self, enable=True):
        """One launch per qualifying decode step (moe_stack_set_one_launch)."""
        moe_stack_set_one_launch(self.handle, enable)

    def set_wait_limit(self, polls):
        """Bound of the one-launch step's device-side waits (0: default)."""
        moe_stack_set_wait_limit(self.handle, polls)

    def set_profiling(self, enable=True):
        moe_stack_set_profiling(self.handle, enable)

    def kernel_ms(self):
        """(router ms, step-kernel ms) of the most recent one-launch step."""
        return moe_stack_kernel_ms(self.handle)

    def set_trace(self, trace):
        """trace: device fp32 tensor [n_layers, n_tok, d] receiving each layer's
        input residual stream on later calls (None turns it off)."""
        self.trace = trace
        moe_stack_set_trace(self.handle, _ptr(trace), 0 if trace is None else trace.numel())

    def decode(self, x, route_idx, route_w, pred_idx, pred_w, *, x_out=None, used_idx=None, used_w=None,
               hist_prev=None, first_step=False, stream=None):
        xo = x if x_out is None else x_out
        moe_stack_decode(self.handle, x.data_ptr(), xo.data_ptr(), x.shape[0], _ptr(route_idx), _ptr(route_w),
                         pred_idx.data_ptr(), pred_w.data_ptr(), _ptr(used_idx), _ptr(used_w), _ptr(hist_prev),
                         first_step, _stream_ptr(stream))

    def prefill(self, x, *, used_idx=None, used_w=None, pred_idx=None, pred_w=None, stream=None):
        moe_stack_prefill(self.handle, x.data_ptr(), x.shape[0], _ptr(used_idx), _ptr(used_w), _ptr(pred_idx),
                          _ptr(pred_w), _stream_ptr(stream))

    def close(self):
        if getattr(self, "handle", None):
            moe_stack_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
