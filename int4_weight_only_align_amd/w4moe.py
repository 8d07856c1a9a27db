"""Python binding of libw4moe (include/w4moe.h): argument marshalling only.

Every step of the layer runs in the library's HIP kernels. PyTorch provides device memory and the
stream; tensors are passed by data pointer. If libw4moe.so is absent, loading raises: there is no
fallback path.

The functions named like the C entry points take and return the same things (torch tensors in place
of device pointers, the current torch stream when `stream` is None). `MoELayer` wraps a handle.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

__all__ = [
    "LIB_PATH", "W4MoEError", "load_library", "w4moe_create", "w4moe_destroy", "w4moe_prepack",
    "w4moe_prepack_act_order", "w4moe_forward", "w4moe_forward_noalloc",
    "w4moe_moe_align", "w4moe_align_block", "w4moe_packed_weights", "w4moe_set_plan", "w4moe_resolved_plan",
    "w4moe_set_expert_range", "w4moe_set_profiling",
    "w4moe_read_profile", "w4moe_read_profile_calls", "w4moe_device_error", "w4moe_set_wait_limit", "w4moe_route", "w4moe_forward_logits", "w4moe_status_string", "w4moe_last_error", "MoELayer",
    "EXPORTED_SYMBOLS",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libw4moe.so")

EXPORTED_SYMBOLS = (
    "w4moe_create", "w4moe_prepack", "w4moe_prepack_act_order", "w4moe_forward", "w4moe_forward_noalloc",
    "w4moe_moe_align",
    "w4moe_align_block",
    "w4moe_packed_weights", "w4moe_set_plan", "w4moe_resolved_plan", "w4moe_set_profiling", "w4moe_read_profile",
    "w4moe_read_profile_calls", "w4moe_route", "w4moe_forward_logits", "w4moe_set_expert_range",
    "w4moe_device_error", "w4moe_set_wait_limit", "w4moe_destroy", "w4moe_status_string", "w4moe_last_error",
)

STATUS = {0: "W4MOE_OK", 1: "W4MOE_ERR_INVALID_ARG", 2: "W4MOE_ERR_UNSUPPORTED", 3: "W4MOE_ERR_NOT_PREPACKED",
          4: "W4MOE_ERR_OUT_OF_MEMORY", 5: "W4MOE_ERR_HIP"}


class W4MoEError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status


class Config(C.Structure):
    _fields_ = [("num_experts", C.c_int32), ("hidden", C.c_int32), ("inter", C.c_int32), ("topk", C.c_int32),
                ("group_size", C.c_int32), ("max_tokens", C.c_int32), ("num_bits", C.c_int32),
                ("act_order", C.c_int32)]


_lib = None


def load_library():
    """Load libw4moe.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
    lib = C.CDLL(LIB_PATH)
    P, i32, i64 = C.c_void_p, C.c_int32, C.c_int64
    sig = {
        "w4moe_create": ([C.POINTER(Config), C.POINTER(P)], C.c_int),
        "w4moe_prepack": ([P, i32, i32, P, P, P, P, P], C.c_int),
        "w4moe_prepack_act_order": ([P, i32, i32, P, P, P, P, P, P, P], C.c_int),
        "w4moe_forward": ([P, P, i32, P, P, P, P], C.c_int),
        "w4moe_forward_noalloc": ([P, P, i32, P, P, P, P], C.c_int),
        "w4moe_forward_logits": ([P, P, i32, P, P, P, P, P], C.c_int),
        "w4moe_route": ([P, P, i32, P, P, P], C.c_int),
        "w4moe_moe_align": ([P, P, i32, i32, P, P, P, P, P, P, P], C.c_int),
        "w4moe_align_block": ([P], i32),
        "w4moe_packed_weights": ([P, i32, C.POINTER(P), C.POINTER(i64)], C.c_int),
        "w4moe_set_plan": ([P, i32], C.c_int),
        "w4moe_set_expert_range": ([P, i32, i32], C.c_int),
        "w4moe_resolved_plan": ([P, i32, C.POINTER(i32)], C.c_int),
        "w4moe_set_profiling": ([P, i32], C.c_int),
        "w4moe_read_profile": ([P, C.POINTER(C.c_double), C.POINTER(i64)], C.c_int),
        "w4moe_read_profile_calls": ([P, C.POINTER(C.c_double), i64, C.POINTER(i64)], C.c_int),
        "w4moe_device_error": ([P, C.POINTER(i32)], C.c_int),
        "w4moe_set_wait_limit": ([P, i64], C.c_int),
        "w4moe_destroy": ([P], None),
        "w4moe_status_string": ([C.c_int], C.c_char_p),
        "w4moe_last_error": ([], C.c_char_p),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes, fn.restype = args, res
    _lib = lib
    return lib


def _check(rc):
    if rc != 0:
        raise W4MoEError(rc, load_library().w4moe_last_error().decode())


def _stream(stream):
    if stream is None:
        return C.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return C.c_void_p(stream.cuda_stream)
    return C.c_void_p(stream)


def _dev(t, dtype, name, shape=None):
    """Data pointer of a contiguous device tensor of the given dtype (None passes NULL)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return C.c_void_p(t.data_ptr())


def w4moe_status_string(status: int) -> str:
    return load_library().w4moe_status_string(status).decode()


def w4moe_last_error() -> str:
    return load_library().w4moe_last_error().decode()


def w4moe_align_block(h) -> int:
    return int(load_library().w4moe_align_block(h))


def w4moe_create(num_experts, hidden, inter, topk, max_tokens, group_size=32, num_bits=4, act_order=False):
    cfg = Config(num_experts, hidden, inter, topk, group_size, max_tokens, num_bits, 1 if act_order else 0)
    h = C.c_void_p()
    _check(load_library().w4moe_create(C.byref(cfg), C.byref(h)))
    return h


def w4moe_destroy(h):
    load_library().w4moe_destroy(h)


def w4moe_prepack(h, first_expert, num_experts, w1_q, w1_scales, w2_q, w2_scales, stream=None):
    """Logical tensors of experts [first_expert, first_expert + num_experts): int32 codes and bf16
    scales (torch.int32 / torch.bfloat16 or int16 bit patterns)."""
    def sc(t, name):
        if t.dtype == torch.bfloat16 or t.dtype == torch.int16:
            return _dev(t, t.dtype, name)
        raise TypeError(f"{name} must be bfloat16 (or int16 bit patterns)")
    _check(load_library().w4moe_prepack(h, first_expert, num_experts, _dev(w1_q, torch.int32, "w1_q"),
                                        sc(w1_scales, "w1_scales"), _dev(w2_q, torch.int32, "w2_q"),
                                        sc(w2_scales, "w2_scales"), _stream(stream)))


def _scales(t, name):
    if t.dtype == torch.bfloat16 or t.dtype == torch.int16:
        return _dev(t, t.dtype, name)
    raise TypeError(f"{name} must be bfloat16 (or int16 bit patterns)")


def w4moe_prepack_act_order(h, first_expert, num_experts, w1_q, w1_scales, w1_perm, w2_q, w2_scales, w2_perm,
                            stream=None):
    """As w4moe_prepack, for activation-ordered experts: w1_perm int32 [n][K] and w2_perm int32 [n][N]
    list each expert's reduction rows in group order (row perm[i] belongs to group i // group_size)."""
    i32 = torch.int32
    _check(load_library().w4moe_prepack_act_order(
        h, first_expert, num_experts, _dev(w1_q, i32, "w1_q"), _scales(w1_scales, "w1_scales"),
        _dev(w1_perm, i32, "w1_perm"), _dev(w2_q, i32, "w2_q"), _scales(w2_scales, "w2_scales"),
        _dev(w2_perm, i32, "w2_perm"), _stream(stream)))


def w4moe_forward(h, hidden, M, topk_ids, topk_weights, out, stream=None):
    _check(load_library().w4moe_forward(h, _dev(hidden, torch.bfloat16, "hidden"), int(M),
                                        _dev(topk_ids, torch.int32, "topk_ids"),
                                        _dev(topk_weights, torch.float32, "topk_weights"),
                                        _dev(out, torch.bfloat16, "out"), _stream(stream)))


def w4moe_forward_noalloc(h, hidden, M, topk_ids, topk_weights, out, stream=None):
    _check(load_library().w4moe_forward_noalloc(h, _dev(hidden, torch.bfloat16, "hidden"), int(M),
                                                _dev(topk_ids, torch.int32, "topk_ids"),
                                                _dev(topk_weights, torch.float32, "topk_weights"),
                                                _dev(out, torch.bfloat16, "out"), _stream(stream)))


def w4moe_forward_logits(h, hidden, M, logits, topk_ids, topk_weights, out, stream=None):
    _check(load_library().w4moe_forward_logits(h, _dev(hidden, torch.bfloat16, "hidden"), int(M),
                                               _dev(logits, torch.float32, "logits"),
                                               _dev(topk_ids, torch.int32, "topk_ids"),
                                               _dev(topk_weights, torch.float32, "topk_weights"),
                                               _dev(out, torch.bfloat16, "out"), _stream(stream)))


def w4moe_route(h, logits, M, topk_ids, topk_weights, stream=None):
    _check(load_library().w4moe_route(h, _dev(logits, torch.float32, "logits"), int(M),
                                      _dev(topk_ids, torch.int32, "topk_ids"),
                                      _dev(topk_weights, torch.float32, "topk_weights"), _stream(stream)))


def w4moe_moe_align(h, topk_ids, M, block, counts, offsets, sorted_ids, block_expert, active=None, n_active=None,
                    stream=None):
    i32 = torch.int32
    _check(load_library().w4moe_moe_align(h, _dev(topk_ids, i32, "topk_ids"), int(M), int(block),
                                          _dev(counts, i32, "counts"), _dev(offsets, i32, "offsets"),
                                          _dev(sorted_ids, i32, "sorted_ids"), _dev(block_expert, i32, "block_expert"),
                                          _dev(active, i32, "active"), _dev(n_active, i32, "n_active"),
                                          _stream(stream)))


def w4moe_packed_weights(h, which):
    ptr, nbytes = C.c_void_p(), C.c_int64()
    _check(load_library().w4moe_packed_weights(h, int(which), C.byref(ptr), C.byref(nbytes)))
    return ptr.value, nbytes.value


def w4moe_set_plan(h, plan):
    _check(load_library().w4moe_set_plan(h, int(plan)))


def w4moe_set_expert_range(h, first_expert, global_experts):
    _check(load_library().w4moe_set_expert_range(h, int(first_expert), int(global_experts)))


def w4moe_resolved_plan(h, M):
    plan = C.c_int32(0)
    _check(load_library().w4moe_resolved_plan(h, int(M), C.byref(plan)))
    return plan.value


def w4moe_set_profiling(h, enable):
    _check(load_library().w4moe_set_profiling(h, 1 if enable else 0))


def w4moe_read_profile(h):
    ms = (C.c_double * 4)()
    calls = C.c_int64()
    _check(load_library().w4moe_read_profile(h, ms, C.byref(calls)))
    return list(ms), calls.value


def w4moe_read_profile_calls(h, capacity=1024):
    buf = (C.c_double * capacity)()
    calls = C.c_int64()
    _check(load_library().w4moe_read_profile_calls(h, buf, capacity, C.byref(calls)))
    return list(buf[:min(calls.value, capacity)])


def w4moe_device_error(h):
    flags = C.c_int32()
    _check(load_library().w4moe_device_error(h, C.byref(flags)))
    return flags.value


def w4moe_set_wait_limit(h, microseconds):
    _check(load_library().w4moe_set_wait_limit(h, int(microseconds)))


class _DevBuf:
    """A raw device range exposed through __cuda_array_interface__ (for reading packed buffers)."""

    def __init__(self, ptr, nbytes):
        self.__cuda_array_interface__ = {"shape": (nbytes,), "typestr": "|u1", "data": (ptr, False), "version": 2,
                                         "strides": None}


class MoELayer:
    """Owns one w4moe handle on the current device."""

    def __init__(self, num_experts, hidden, inter, topk, max_tokens, group_size=32, num_bits=4, act_order=False):
        self.E, self.K, self.N, self.topk, self.max_tokens = num_experts, hidden, inter, topk, max_tokens
        self.handle = w4moe_create(num_experts, hidden, inter, topk, max_tokens, group_size, num_bits, act_order)

    def close(self):
        if self.handle is not None and self.handle.value:
            w4moe_destroy(self.handle)
        self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def prepack(self, w1_q, w1_scales, w2_q, w2_scales, first_expert=0, stream=None):
        n = w1_q.shape[0]
        w4moe_prepack(self.handle, first_expert, n, w1_q, w1_scales, w2_q, w2_scales, stream)

    def prepack_act_order(self, w1_q, w1_scales, w1_perm, w2_q, w2_scales, w2_perm, first_expert=0, stream=None):
        n = w1_q.shape[0]
        w4moe_prepack_act_order(self.handle, first_expert, n, w1_q, w1_scales, w1_perm, w2_q, w2_scales, w2_perm,
                                stream)

    def forward(self, hidden, topk_ids, topk_weights, out=None, stream=None):
        M = hidden.shape[0]
        if out is None:
            out = torch.empty((M, self.K), dtype=torch.bfloat16, device=hidden.device)
        w4moe_forward(self.handle, hidden, M, topk_ids, topk_weights, out, stream)
        return out

    __call__ = forward

    def forward_noalloc(self, hidden, topk_ids, topk_weights, out, stream=None):
        """The layer with the workspace in the library's static per-GPU array (no allocation anywhere,
        `out` given by the caller): single-launch mode, M * topk <= 64."""
        w4moe_forward_noalloc(self.handle, hidden, hidden.shape[0], topk_ids, topk_weights, out, stream)
        return out

    def route(self, logits, stream=None):
        """Top-k route of logits fp32 [M, E]: (ids int32 [M, topk], weights fp32 [M, topk])."""
        M = logits.shape[0]
        ids = torch.empty((M, self.topk), dtype=torch.int32, device=logits.device)
        w = torch.empty((M, self.topk), dtype=torch.float32, device=logits.device)
        w4moe_route(self.handle, logits, M, ids, w, stream)
        return ids, w

    def forward_logits(self, hidden, logits, out=None, stream=None):
        """Route and run the layer: (out, ids, weights)."""
        M = hidden.shape[0]
        if out is None:
            out = torch.empty((M, self.K), dtype=torch.bfloat16, device=hidden.device)
        ids = torch.empty((M, self.topk), dtype=torch.int32, device=hidden.device)
        w = torch.empty((M, self.topk), dtype=torch.float32, device=hidden.device)
        w4moe_forward_logits(self.handle, hidden, M, logits, ids, w, out, stream)
        return out, ids, w

    def moe_align(self, topk_ids, block, stream=None):
        M = topk_ids.shape[0]
        T = M * self.topk
        cap = T + min(self.E, T) * (block - 1) + 1
        dev = topk_ids.device
        i32 = torch.int32
        r = dict(counts=torch.zeros(self.E, dtype=i32, device=dev), offsets=torch.zeros(self.E + 1, dtype=i32, device=dev),
                 sorted_ids=torch.full((cap,), -1, dtype=i32, device=dev),
                 block_expert=torch.full((cap // block + 1,), -1, dtype=i32, device=dev),
                 active=torch.full((self.E,), -1, dtype=i32, device=dev), n_active=torch.zeros(1, dtype=i32, device=dev))
        w4moe_moe_align(self.handle, topk_ids, M, block, r["counts"], r["offsets"], r["sorted_ids"], r["block_expert"],
                        r["active"], r["n_active"], stream)
        return r

    def align_block(self):
        """Rows per token tile of forward's alignment (w4moe_align_block)."""
        return w4moe_align_block(self.handle)

    def packed_weights(self, which):
        """(device pointer, bytes) of the packed W1 (1) or W2 (2) buffer."""
        return w4moe_packed_weights(self.handle, which)

    def packed_bytes(self, which):
        """A uint8 device tensor copy of the packed W1 (1) or W2 (2) buffer."""
        ptr, nbytes = self.packed_weights(which)
        view = torch.as_tensor(_DevBuf(ptr, nbytes), device="cuda")
        return view.clone()

    def set_plan(self, plan):
        w4moe_set_plan(self.handle, plan)

    def set_expert_range(self, first_expert, global_experts):
        """Expert parallelism: this layer's experts are [first_expert, first_expert + E) of a layer of
        global_experts; routing ids (and the router's logits) are global from here on."""
        w4moe_set_expert_range(self.handle, first_expert, global_experts)
        self.E_all = int(global_experts)

    def resolved_plan(self, M):
        return w4moe_resolved_plan(self.handle, M)

    def set_profiling(self, enable):
        w4moe_set_profiling(self.handle, enable)

    def read_profile(self):
        return w4moe_read_profile(self.handle)

    def read_profile_calls(self, capacity=1024):
        return w4moe_read_profile_calls(self.handle, capacity)

    def device_error(self):
        return w4moe_device_error(self.handle)

    def set_wait_limit(self, microseconds):
        """Bound of the single-launch pair mode's hand-off wait (negative: the default, 100 ms)."""
        w4moe_set_wait_limit(self.handle, microseconds)
