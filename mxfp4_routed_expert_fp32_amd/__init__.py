"""Python binding of libmoe_mxfp4.so (the routed MXFP4 MoE layer for gfx950).

Argument marshalling only: torch tensors are used for device memory and
streams, their addresses go to the C ABI declared in include/moe_mxfp4.h, and
every step of the layer runs in the library's HIP kernels.  There is no
fallback: if the library is missing, importing the binding's functions raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_mxfp4.so")

MOE_ABI_VERSION = 1
MOE_LAYOUT_ROWMAJOR_V1 = 1
MOE_LAYOUT_SCALE4_V1 = 2
MOE_DTYPE_F32, MOE_DTYPE_BF16 = 0, 1

STATUS = {
    0: "MOE_OK", -1: "MOE_ERR_NULL", -2: "MOE_ERR_SHAPE", -3: "MOE_ERR_DTYPE", -4: "MOE_ERR_ALIGN",
    -5: "MOE_ERR_WORKSPACE", -6: "MOE_ERR_LAYOUT", -7: "MOE_ERR_UNSUPPORTED", -8: "MOE_ERR_OVERFLOW",
    -9: "MOE_ERR_DEVICE", -10: "MOE_ERR_ABI", -11: "MOE_ERR_RANGE", -12: "MOE_ERR_SCRATCH_LIMIT",
    -13: "MOE_ERR_POISONED", -14: "MOE_ERR_STATE", -15: "MOE_ERR_IO",
}

EXPORTS = [
    "moe_abi_version", "moe_status_string", "moe_layer_check", "moe_mxfp4_packed_bytes",
    "moe_workspace_bytes", "moe_mxfp4_pack", "moe_mxfp4_forward", "moe_mxfp4_forward_noalloc", "moe_mxfp4_experts",
    "moe_mxfp4_gate_up", "moe_mxfp4_gate_up_select", "moe_mxfp4_down", "moe_combine",
    "moe_router_logits", "moe_topk_softmax", "moe_sort_workspace_bytes", "moe_sort_by_expert",
    "moe_max_expert_blocks", "moe_expert_blocks", "moe_mxfp4_grouped_gate_up", "moe_mxfp4_grouped_down",
    "moe_mxfp4_dequant", "moe_mxfp4_dequant_bf16", "moe_rmsnorm", "moe_residual_add", "moe_stack_workspace_bytes",
    "moe_mxfp4_stack_forward", "moe_stack_graph_create", "moe_stack_graph_launch",
    "moe_stack_graph_destroy", "moe_cache_create", "moe_cache_destroy", "moe_cache_slots", "moe_cache_get_stats",
    "moe_cache_plan", "moe_cache_finish", "moe_cache_cancel", "moe_cache_workspace_bytes", "moe_cache_layer_forward",
    "moe_route_hint_workspace_bytes", "moe_route_hint", "moe_trace_open", "moe_trace_record", "moe_trace_close",
    "moe_trace_count", "moe_int8_dequant", "moe_int8_gemv", "moe_mxfp4_scale4_encode", "moe_mfma_rate",
]
MOE_TRACE_BUFFERED, MOE_TRACE_SYNC = 0, 1
MOE_CACHE_PREFETCH = 1


class CacheStats(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("capacity", ctypes.c_int32), ("poisoned", ctypes.c_int32),
                ("alloc_retries", ctypes.c_int32), ("plans", ctypes.c_int64), ("hits", ctypes.c_int64),
                ("misses", ctypes.c_int64), ("prefetched", ctypes.c_int64), ("evictions", ctypes.c_int64),
                ("bytes_uploaded", ctypes.c_uint64)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_ if f != "struct_size"}


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__("%s failed: %s (%d)" % (fn, STATUS.get(status, "?"), status))


class LayerDesc(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_uint32), ("struct_size", ctypes.c_uint32),
                ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k_max", ctypes.c_int32), ("layout", ctypes.c_uint32), ("reserved", ctypes.c_uint32)]

    @classmethod
    def make(cls, hidden: int, inter: int, n_experts: int, top_k_max: int,
             layout: int = MOE_LAYOUT_ROWMAJOR_V1) -> "LayerDesc":
        return cls(MOE_ABI_VERSION, ctypes.sizeof(cls), hidden, inter, n_experts, top_k_max, layout, 0)


_lock = threading.Lock()
_lib = None


def lib():
    """Load libmoe_mxfp4.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise ImportError("libmoe_mxfp4.so is not built (run __graft_entry__.build() or "
                                  "python mxfp4_routed_expert_fp32_amd/build.py)")
            L = ctypes.CDLL(LIB_PATH)
            vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
            P = ctypes.POINTER
            D = P(LayerDesc)
            sig = {
                "moe_abi_version": ([], ctypes.c_uint32),
                "moe_status_string": ([ctypes.c_int], ctypes.c_char_p),
                "moe_layer_check": ([D], ctypes.c_int),
                "moe_mxfp4_packed_bytes": ([D, P(sz), P(sz)], ctypes.c_int),
                "moe_workspace_bytes": ([D, i32, i32, P(sz)], ctypes.c_int),
                "moe_mxfp4_pack": ([D, vp, vp, i64, i64, vp, vp, vp], ctypes.c_int),
                "moe_mxfp4_forward": ([D, vp, i32, vp, vp, vp, vp, i32, i32, vp, vp, vp, vp, vp, sz, vp],
                                      ctypes.c_int),
                "moe_mxfp4_forward_noalloc": ([D, vp, i32, vp, vp, vp, vp, i32, i32, vp, vp, vp, vp, vp],
                                              ctypes.c_int),
                "moe_mxfp4_experts": ([D, vp, i32, vp, vp, vp, vp, i32, i32, vp, vp, sz, vp], ctypes.c_int),
                "moe_mxfp4_gate_up": ([D, vp, i32, vp, i32, i32, vp, vp, vp, vp], ctypes.c_int),
                "moe_mxfp4_gate_up_select": ([D, vp, i32, vp, i32, i32, vp, vp, vp, vp, vp, vp], ctypes.c_int),
                "moe_mxfp4_down": ([D, vp, vp, i32, vp, vp, vp, vp], ctypes.c_int),
                "moe_combine": ([vp, vp, i32, i32, i32, vp, vp, vp], ctypes.c_int),
                "moe_router_logits": ([D, vp, i32, vp, vp, i32, vp, vp], ctypes.c_int),
                "moe_topk_softmax": ([vp, i32, i32, i32, vp, vp, vp], ctypes.c_int),
                "moe_sort_workspace_bytes": ([i32, i32, i32, P(sz)], ctypes.c_int),
                "moe_sort_by_expert": ([vp, i32, i32, i32, vp, vp, vp, sz, vp], ctypes.c_int),
                "moe_max_expert_blocks": ([i32, i32, P(i32)], ctypes.c_int),
                "moe_expert_blocks": ([vp, i32, i32, vp, i32, vp, vp], ctypes.c_int),
                "moe_mxfp4_grouped_gate_up": ([D, vp, i32, i32, vp, vp, vp, i32, vp, vp, vp, vp], ctypes.c_int),
                "moe_mxfp4_grouped_down": ([D, vp, i32, vp, vp, vp, i32, vp, vp, vp, vp], ctypes.c_int),
                "moe_mxfp4_dequant": ([D, vp, vp, i64, i32, vp, vp], ctypes.c_int),
                "moe_mxfp4_dequant_bf16": ([D, vp, vp, i64, i32, vp, vp], ctypes.c_int),
                "moe_rmsnorm": ([vp, vp, ctypes.c_float, i32, i32, vp, vp], ctypes.c_int),
                "moe_residual_add": ([vp, vp, i64, vp], ctypes.c_int),
                "moe_stack_workspace_bytes": ([D, i32, i32, P(sz)], ctypes.c_int),
                "moe_mxfp4_stack_forward": ([D, i32, vp, vp, vp, vp, vp, ctypes.c_float, vp, i32, i32, i32,
                                             vp, vp, sz, vp], ctypes.c_int),
                "moe_stack_graph_create": ([D, i32, vp, vp, vp, vp, vp, ctypes.c_float, vp, i32, i32, i32,
                                            vp, vp, sz, vp, P(vp)], ctypes.c_int),
                "moe_stack_graph_launch": ([vp, vp], ctypes.c_int),
                "moe_stack_graph_destroy": ([vp], ctypes.c_int),
                "moe_cache_create": ([D, i32, i32, i32, P(vp)], ctypes.c_int),
                "moe_cache_destroy": ([vp], ctypes.c_int),
                "moe_cache_slots": ([vp, P(vp), P(vp), P(i32)], ctypes.c_int),
                "moe_cache_get_stats": ([vp, P(CacheStats)], ctypes.c_int),
                "moe_cache_plan": ([vp, i32, vp, i32, i32, vp, vp, P(i32)], ctypes.c_int),
                "moe_cache_finish": ([vp, vp, vp, i32, vp], ctypes.c_int),
                "moe_cache_cancel": ([vp], ctypes.c_int),
                "moe_cache_workspace_bytes": ([vp, i32, i32, P(sz)], ctypes.c_int),
                "moe_cache_layer_forward": ([vp, i32, vp, i32, vp, vp, vp, vp, i32, i32, i32, vp, vp, vp, vp, sz,
                                             vp], ctypes.c_int),
                "moe_route_hint_workspace_bytes": ([D, i32, i32, P(sz)], ctypes.c_int),
                "moe_route_hint": ([D, vp, vp, ctypes.c_float, vp, vp, i32, i32, vp, vp, sz, vp], ctypes.c_int),
                "moe_trace_open": ([ctypes.c_char_p, i32, ctypes.c_uint64, P(vp)], ctypes.c_int),
                "moe_trace_record": ([vp, i32, i64, i32, i32, vp, vp], ctypes.c_int),
                "moe_trace_close": ([vp], ctypes.c_int),
                "moe_trace_count": ([ctypes.c_char_p, i32, i32, vp, P(i64)], ctypes.c_int),
                "moe_int8_dequant": ([vp, vp, i32, i32, vp, vp], ctypes.c_int),
                "moe_mxfp4_scale4_encode": ([D, vp, i64, i64, vp, vp, vp], ctypes.c_int),
                "moe_int8_gemv": ([vp, vp, i32, i32, vp, i32, i32, vp, i32, vp], ctypes.c_int),
                "moe_mfma_rate": ([i32, vp, i32, i32, vp, vp], ctypes.c_int),
            }
            for name, (args, res) in sig.items():
                f = getattr(L, name)
                f.argtypes = args
                f.restype = res
            if L.moe_abi_version() != MOE_ABI_VERSION:
                raise ImportError("libmoe_mxfp4.so ABI version mismatch")
            _lib = L
    return _lib


def _check(fn: str, rc: int) -> None:
    if rc != 0:
        raise MoeError(fn, rc)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _xdtype(x) -> int:
    import torch
    if x.dtype == torch.float32:
        return MOE_DTYPE_F32
    if x.dtype == torch.bfloat16:
        return MOE_DTYPE_BF16
    raise TypeError("x must be float32 or bfloat16")


def _ptr_array(ts):
    arr = (ctypes.c_void_p * len(ts))()
    for i, t in enumerate(ts):
        arr[i] = None if t is None else t.data_ptr()
    return arr


# --------------------------------------------------------------------------- sizes

def packed_bytes(desc: LayerDesc):
    c, s = ctypes.c_size_t(), ctypes.c_size_t()
    _check("moe_mxfp4_packed_bytes", lib().moe_mxfp4_packed_bytes(ctypes.byref(desc), ctypes.byref(c), ctypes.byref(s)))
    return c.value, s.value


def workspace_bytes(desc: LayerDesc, n_tokens: int, k: int) -> int:
    b = ctypes.c_size_t()
    _check("moe_workspace_bytes", lib().moe_workspace_bytes(ctypes.byref(desc), n_tokens, k, ctypes.byref(b)))
    return b.value


def stack_workspace_bytes(desc: LayerDesc, n_tokens: int, k: int) -> int:
    b = ctypes.c_size_t()
    _check("moe_stack_workspace_bytes",
           lib().moe_stack_workspace_bytes(ctypes.byref(desc), n_tokens, k, ctypes.byref(b)))
    return b.value


# --------------------------------------------------------------------------- calls

def moe_mxfp4_pack(desc, logical_codes, logical_scales, expert_begin, expert_count, packed_codes,
                   packed_scales, stream=None):
    _check("moe_mxfp4_pack", lib().moe_mxfp4_pack(
        ctypes.byref(desc), _ptr(logical_codes), _ptr(logical_scales), expert_begin, expert_count,
        _ptr(packed_codes), _ptr(packed_scales), _stream(stream)))


def moe_mxfp4_forward(desc, x, router_w, router_bias, packed_codes, packed_scales, k, out, workspace,
                      logits_out=None, topk_idx_out=None, topk_w_out=None, stream=None):
    _check("moe_mxfp4_forward", lib().moe_mxfp4_forward(
        ctypes.byref(desc), _ptr(x), _xdtype(x), _ptr(router_w), _ptr(router_bias), _ptr(packed_codes),
        _ptr(packed_scales), x.shape[0], k, _ptr(out), _ptr(logits_out), _ptr(topk_idx_out),
        _ptr(topk_w_out), _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))


def moe_mxfp4_forward_noalloc(desc, x, router_w, router_bias, packed_codes, packed_scales, k, out,
                              logits_out=None, topk_idx_out=None, topk_w_out=None, stream=None):
    _check("moe_mxfp4_forward_noalloc", lib().moe_mxfp4_forward_noalloc(
        ctypes.byref(desc), _ptr(x), _xdtype(x), _ptr(router_w), _ptr(router_bias), _ptr(packed_codes),
        _ptr(packed_scales), x.shape[0], k, _ptr(out), _ptr(logits_out), _ptr(topk_idx_out),
        _ptr(topk_w_out), _stream(stream)))


def moe_mxfp4_experts(desc, x, topk_idx, topk_w, packed_codes, packed_scales, k, out, workspace,
                      stream=None):
    _check("moe_mxfp4_experts", lib().moe_mxfp4_experts(
        ctypes.byref(desc), _ptr(x), _xdtype(x), _ptr(topk_idx), _ptr(topk_w), _ptr(packed_codes),
        _ptr(packed_scales), x.shape[0], k, _ptr(out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def moe_mxfp4_gate_up(desc, x, pair_expert, k, packed_codes, packed_scales, h, stream=None):
    _check("moe_mxfp4_gate_up", lib().moe_mxfp4_gate_up(
        ctypes.byref(desc), _ptr(x), _xdtype(x), _ptr(pair_expert), pair_expert.numel(), k,
        _ptr(packed_codes), _ptr(packed_scales), _ptr(h), _stream(stream)))


def moe_mxfp4_gate_up_select(desc, x, logits, k, packed_codes, packed_scales, topk_idx, topk_w, h, stream=None):
    _check("moe_mxfp4_gate_up_select", lib().moe_mxfp4_gate_up_select(
        ctypes.byref(desc), _ptr(x), _xdtype(x), _ptr(logits), x.shape[0], k, _ptr(packed_codes),
        _ptr(packed_scales), _ptr(topk_idx), _ptr(topk_w), _ptr(h), _stream(stream)))


def moe_mxfp4_down(desc, h, pair_expert, packed_codes, packed_scales, y, stream=None):
    _check("moe_mxfp4_down", lib().moe_mxfp4_down(
        ctypes.byref(desc), _ptr(h), _ptr(pair_expert), pair_expert.numel(), _ptr(packed_codes),
        _ptr(packed_scales), _ptr(y), _stream(stream)))


def moe_combine(y, w, out, resid=None, stream=None):
    T, k = w.shape
    _check("moe_combine", lib().moe_combine(_ptr(y), _ptr(w), T, k, out.shape[1], _ptr(resid), _ptr(out),
                                            _stream(stream)))


def moe_router_logits(desc, x, router_w, router_bias, logits, stream=None):
    _check("moe_router_logits", lib().moe_router_logits(
        ctypes.byref(desc), _ptr(x), _xdtype(x), _ptr(router_w), _ptr(router_bias), x.shape[0],
        _ptr(logits), _stream(stream)))


def moe_topk_softmax(logits, k, idx, w, stream=None):
    _check("moe_topk_softmax", lib().moe_topk_softmax(
        _ptr(logits), logits.shape[0], logits.shape[1], k, _ptr(idx), _ptr(w), _stream(stream)))


def sort_workspace_bytes(n_experts: int, n_tokens: int, k: int) -> int:
    b = ctypes.c_size_t()
    _check("moe_sort_workspace_bytes",
           lib().moe_sort_workspace_bytes(n_experts, n_tokens, k, ctypes.byref(b)))
    return b.value


def moe_sort_by_expert(topk_idx, n_experts, expert_offsets, pair_list, workspace=None, stream=None):
    nb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("moe_sort_by_expert", lib().moe_sort_by_expert(
        _ptr(topk_idx), topk_idx.shape[0], n_experts, topk_idx.shape[1], _ptr(expert_offsets),
        _ptr(pair_list), _ptr(workspace), nb, _stream(stream)))


def max_expert_blocks(n_experts: int, n_pairs: int) -> int:
    m = ctypes.c_int32()
    _check("moe_max_expert_blocks", lib().moe_max_expert_blocks(n_experts, n_pairs, ctypes.byref(m)))
    return m.value


def moe_expert_blocks(expert_offsets, n_pairs, blocks, n_blocks, stream=None):
    """blocks: int32 [max_blocks, 4]; n_blocks: int32 [1] (device)."""
    _check("moe_expert_blocks", lib().moe_expert_blocks(
        _ptr(expert_offsets), expert_offsets.numel() - 1, n_pairs, _ptr(blocks), blocks.shape[0], _ptr(n_blocks),
        _stream(stream)))


def moe_mxfp4_grouped_gate_up(desc, x, k, pair_list, blocks, n_blocks, packed_codes, packed_scales, hterm,
                              stream=None):
    """x: bf16 [T, H]; hterm: bf16 (or int16) [2, T*k, I]."""
    _check("moe_mxfp4_grouped_gate_up", lib().moe_mxfp4_grouped_gate_up(
        ctypes.byref(desc), _ptr(x), x.shape[0], k, _ptr(pair_list), _ptr(blocks), _ptr(n_blocks), blocks.shape[0],
        _ptr(packed_codes), _ptr(packed_scales), _ptr(hterm), _stream(stream)))


def moe_mxfp4_grouped_down(desc, hterm, pair_list, blocks, n_blocks, packed_codes, packed_scales, y, stream=None):
    """hterm: [2, P, I] bf16 terms; y: fp32 [P, H]."""
    _check("moe_mxfp4_grouped_down", lib().moe_mxfp4_grouped_down(
        ctypes.byref(desc), _ptr(hterm), pair_list.numel(), _ptr(pair_list), _ptr(blocks), _ptr(n_blocks),
        blocks.shape[0], _ptr(packed_codes), _ptr(packed_scales), _ptr(y), _stream(stream)))


def moe_mxfp4_dequant(desc, packed_codes, packed_scales, expert, matrix, out, stream=None):
    _check("moe_mxfp4_dequant", lib().moe_mxfp4_dequant(
        ctypes.byref(desc), _ptr(packed_codes), _ptr(packed_scales), expert, matrix, _ptr(out),
        _stream(stream)))


def moe_mxfp4_dequant_bf16(desc, packed_codes, packed_scales, expert, matrix, out, stream=None):
    _check("moe_mxfp4_dequant_bf16", lib().moe_mxfp4_dequant_bf16(
        ctypes.byref(desc), _ptr(packed_codes), _ptr(packed_scales), expert, matrix, _ptr(out),
        _stream(stream)))


def moe_rmsnorm(r, gamma, eps, out, stream=None):
    _check("moe_rmsnorm", lib().moe_rmsnorm(_ptr(r), _ptr(gamma), eps, r.shape[0], r.shape[1], _ptr(out),
                                            _stream(stream)))


def moe_residual_add(r, d, stream=None):
    _check("moe_residual_add", lib().moe_residual_add(_ptr(r), _ptr(d), r.numel(), _stream(stream)))


def moe_mxfp4_stack_forward(desc, packed_codes, packed_scales, router_w, router_bias, gamma, eps, x, k,
                            residual, workspace, stream=None):
    n = len(packed_codes)
    arrs = [_ptr_array(packed_codes), _ptr_array(packed_scales), _ptr_array(router_w),
            None if router_bias is None else _ptr_array(router_bias), _ptr_array(gamma)]
    _check("moe_mxfp4_stack_forward", lib().moe_mxfp4_stack_forward(
        ctypes.byref(desc), n, *[None if a is None else ctypes.cast(a, ctypes.c_void_p) for a in arrs],
        eps, _ptr(x), _xdtype(x), x.shape[0], k, _ptr(residual), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


class StackGraph:
    """moe_stack_graph_create / launch / destroy."""

    def __init__(self, desc, packed_codes, packed_scales, router_w, router_bias, gamma, eps, x, k,
                 residual, workspace, stream=None):
        n = len(packed_codes)
        arrs = [_ptr_array(packed_codes), _ptr_array(packed_scales), _ptr_array(router_w),
                None if router_bias is None else _ptr_array(router_bias), _ptr_array(gamma)]
        h = ctypes.c_void_p()
        _check("moe_stack_graph_create", lib().moe_stack_graph_create(
            ctypes.byref(desc), n, *[None if a is None else ctypes.cast(a, ctypes.c_void_p) for a in arrs],
            eps, _ptr(x), _xdtype(x), x.shape[0], k, _ptr(residual), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(stream), ctypes.byref(h)))
        self._h = h
        self._keep = (packed_codes, packed_scales, router_w, router_bias, gamma, x, residual, workspace)

    def launch(self, stream=None):
        _check("moe_stack_graph_launch", lib().moe_stack_graph_launch(self._h, _stream(stream)))

    def close(self):
        if self._h:
            _check("moe_stack_graph_destroy", lib().moe_stack_graph_destroy(self._h))
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class ExpertCache:
    """moe_cache_*: host-streamed experts with a device residency cache.

    Host spans are numpy arrays (or raw addresses) of one layer's experts in
    the logical layout, experts back to back; pinned=True when they live in
    pinned host memory (direct DMA, no staging)."""

    def __init__(self, desc, n_layers, capacity=0, max_retries=4):
        h = ctypes.c_void_p()
        _check("moe_cache_create", lib().moe_cache_create(ctypes.byref(desc), n_layers, capacity, max_retries,
                                                          ctypes.byref(h)))
        self._h = h
        self.desc = desc
        c, s, n = ctypes.c_void_p(), ctypes.c_void_p(), ctypes.c_int32()
        _check("moe_cache_slots", lib().moe_cache_slots(h, ctypes.byref(c), ctypes.byref(s), ctypes.byref(n)))
        self.slot_codes, self.slot_scales, self.capacity = c.value, s.value, n.value
        self.slot_desc = LayerDesc.make(desc.hidden, desc.inter, self.capacity, min(desc.top_k_max, self.capacity))

    def stats(self):
        st = CacheStats()
        st.struct_size = ctypes.sizeof(CacheStats)
        _check("moe_cache_get_stats", lib().moe_cache_get_stats(self._h, ctypes.byref(st)))
        return st.as_dict()

    def plan(self, layer, ids, prefetch=False):
        """ids: host int32 array.  Returns (slots [n] or None, ordered miss ids)."""
        import numpy as np
        ids = np.ascontiguousarray(ids, np.int32).reshape(-1)
        slots = None if prefetch else np.empty(ids.size, np.int32)
        miss = np.empty(ids.size, np.int32)
        nm = ctypes.c_int32()
        _check("moe_cache_plan", lib().moe_cache_plan(
            self._h, layer, ids.ctypes.data, ids.size, MOE_CACHE_PREFETCH if prefetch else 0,
            None if slots is None else slots.ctypes.data, miss.ctypes.data, ctypes.byref(nm)))
        return slots, miss[:nm.value].copy()

    def finish(self, miss_codes, miss_scales, pinned=False, stream=None):
        """miss_codes / miss_scales: per-miss host spans (numpy arrays or addresses), in miss order."""
        n = len(miss_codes)
        pc = (ctypes.c_void_p * max(n, 1))()
        ps = (ctypes.c_void_p * max(n, 1))()
        for i in range(n):
            pc[i] = _addr(miss_codes[i])
            ps[i] = _addr(miss_scales[i])
        _check("moe_cache_finish", lib().moe_cache_finish(self._h, pc, ps, 1 if pinned else 0, _stream(stream)))

    def cancel(self):
        _check("moe_cache_cancel", lib().moe_cache_cancel(self._h))

    def workspace_bytes(self, n_tokens, k):
        b = ctypes.c_size_t()
        _check("moe_cache_workspace_bytes", lib().moe_cache_workspace_bytes(self._h, n_tokens, k, ctypes.byref(b)))
        return b.value

    def layer_forward(self, layer, x, router_w, router_bias, host_codes, host_scales, k, out, workspace,
                      topk_idx_out=None, topk_w_out=None, pinned=False, stream=None):
        _check("moe_cache_layer_forward", lib().moe_cache_layer_forward(
            self._h, layer, _ptr(x), _xdtype(x), _ptr(router_w), _ptr(router_bias), _addr(host_codes),
            _addr(host_scales), 1 if pinned else 0, x.shape[0], k, _ptr(out), _ptr(topk_idx_out), _ptr(topk_w_out),
            _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))

    def close(self):
        if self._h:
            _check("moe_cache_destroy", lib().moe_cache_destroy(self._h))
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _addr(a):
    """Host address of a numpy array, a torch CPU tensor or a raw integer address."""
    if isinstance(a, int):
        return ctypes.c_void_p(a)
    if hasattr(a, "ctypes"):
        return ctypes.c_void_p(a.ctypes.data)
    return ctypes.c_void_p(a.data_ptr())


def route_hint_workspace_bytes(desc, n_tokens, k) -> int:
    b = ctypes.c_size_t()
    _check("moe_route_hint_workspace_bytes",
           lib().moe_route_hint_workspace_bytes(ctypes.byref(desc), n_tokens, k, ctypes.byref(b)))
    return b.value


def moe_route_hint(desc, r, gamma_next, eps, router_w_next, router_bias_next, k, hint_idx, workspace, stream=None):
    _check("moe_route_hint", lib().moe_route_hint(
        ctypes.byref(desc), _ptr(r), _ptr(gamma_next), eps, _ptr(router_w_next), _ptr(router_bias_next), r.shape[0], k,
        _ptr(hint_idx), _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))


class RouteTrace:
    """moe_trace_open / record / close (host arrays)."""

    def __init__(self, path, mode=MOE_TRACE_BUFFERED, max_bytes=0):
        h = ctypes.c_void_p()
        _check("moe_trace_open", lib().moe_trace_open(os.fsencode(path), mode, max_bytes, ctypes.byref(h)))
        self._h = h

    def record(self, layer, position, ids, w):
        import numpy as np
        ids = np.ascontiguousarray(ids, np.int32)
        w = np.ascontiguousarray(w, np.float32)
        T, k = ids.shape
        _check("moe_trace_record", lib().moe_trace_record(self._h, layer, position, T, k, ids.ctypes.data,
                                                          w.ctypes.data))

    def close(self):
        if self._h:
            h, self._h = self._h, ctypes.c_void_p()
            _check("moe_trace_close", lib().moe_trace_close(h))

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def trace_count(path, n_layers, n_experts):
    """(counts [n_layers, n_experts] int64, number of records) of a router trace."""
    import numpy as np
    counts = np.zeros((n_layers, n_experts), np.int64)
    n = ctypes.c_int64()
    _check("moe_trace_count", lib().moe_trace_count(os.fsencode(path), n_layers, n_experts, counts.ctypes.data,
                                                    ctypes.byref(n)))
    return counts, n.value


def moe_int8_dequant(q, scales_f16, out, stream=None):
    """q: int8 [N, K]; scales_f16: int16/float16 [N] (binary16 bits); out: fp32 [N, K]."""
    N, K = q.shape
    _check("moe_int8_dequant", lib().moe_int8_dequant(_ptr(q), _ptr(scales_f16), N, K, _ptr(out), _stream(stream)))


def moe_int8_gemv(q, scales_f16, x, y, rows_per_workgroup=0, stream=None):
    """y [T, N] = x [T, K] . (q * s)^T."""
    N, K = q.shape
    _check("moe_int8_gemv", lib().moe_int8_gemv(_ptr(q), _ptr(scales_f16), N, K, _ptr(x), _xdtype(x), x.shape[0],
                                                _ptr(y), rows_per_workgroup, _stream(stream)))


MFMA_RATE_KINDS = {0: ("bf16", 16384), 1: ("fp8_x_fp4", 65536), 2: ("fp4_x_fp4", 65536)}  # name, flops per MFMA


def moe_mfma_rate(kind, operands, n_workgroups, iters, sink, stream=None):
    """Enqueue n_workgroups x 512 threads x iters x 8 MFMAs of one kind on
    random operands (operands: 65536 bytes; sink: n_workgroups * 512 floats)."""
    _check("moe_mfma_rate", lib().moe_mfma_rate(kind, _ptr(operands), n_workgroups, iters, _ptr(sink),
                                                _stream(stream)))


def moe_mxfp4_scale4_encode(desc4, scales8, expert_begin, expert_count, scale4, escapes, stream=None):
    """desc4: a scale4 descriptor; scales8: the 8-bit table of the experts
    (device); scale4: the layer's scale4 buffer; escapes: int32 [1] (device,
    incremented per row that cannot be coded)."""
    _check("moe_mxfp4_scale4_encode", lib().moe_mxfp4_scale4_encode(
        ctypes.byref(desc4), _ptr(scales8), expert_begin, expert_count, _ptr(scale4), _ptr(escapes), _stream(stream)))


def encode_scale4_layer(desc8, scales8, stream=None):
    """The scale4 buffer of a whole layer from its 8-bit table (device tensors),
    or None when some row cannot be coded (the layer keeps the 8-bit table).
    Returns (desc4, scale4)."""
    import torch
    desc4 = LayerDesc.make(desc8.hidden, desc8.inter, desc8.n_experts, desc8.top_k_max, MOE_LAYOUT_SCALE4_V1)
    _, sb4 = packed_bytes(desc4)
    scale4 = torch.empty(sb4, dtype=torch.uint8, device=scales8.device)
    esc = torch.zeros(1, dtype=torch.int32, device=scales8.device)
    moe_mxfp4_scale4_encode(desc4, scales8, 0, desc8.n_experts, scale4, esc, stream)
    if int(esc.item()) != 0:
        return None
    return desc4, scale4
