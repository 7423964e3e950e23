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
MOE_DTYPE_F32, MOE_DTYPE_BF16 = 0, 1

STATUS = {
    0: "MOE_OK", -1: "MOE_ERR_NULL", -2: "MOE_ERR_SHAPE", -3: "MOE_ERR_DTYPE", -4: "MOE_ERR_ALIGN",
    -5: "MOE_ERR_WORKSPACE", -6: "MOE_ERR_LAYOUT", -7: "MOE_ERR_UNSUPPORTED", -8: "MOE_ERR_OVERFLOW",
    -9: "MOE_ERR_DEVICE", -10: "MOE_ERR_ABI", -11: "MOE_ERR_RANGE", -12: "MOE_ERR_SCRATCH_LIMIT",
}

EXPORTS = [
    "moe_abi_version", "moe_status_string", "moe_layer_check", "moe_mxfp4_packed_bytes",
    "moe_workspace_bytes", "moe_mxfp4_pack", "moe_mxfp4_forward", "moe_mxfp4_forward_noalloc", "moe_mxfp4_experts",
    "moe_mxfp4_gate_up", "moe_mxfp4_gate_up_select", "moe_mxfp4_down", "moe_combine",
    "moe_router_logits", "moe_topk_softmax", "moe_sort_workspace_bytes", "moe_sort_by_expert",
    "moe_max_expert_blocks", "moe_expert_blocks", "moe_mxfp4_grouped_gate_up", "moe_mxfp4_grouped_down",
    "moe_mxfp4_dequant", "moe_mxfp4_dequant_bf16", "moe_rmsnorm", "moe_residual_add", "moe_stack_workspace_bytes",
    "moe_mxfp4_stack_forward", "moe_stack_graph_create", "moe_stack_graph_launch",
    "moe_stack_graph_destroy",
]


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__("%s failed: %s (%d)" % (fn, STATUS.get(status, "?"), status))


class LayerDesc(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_uint32), ("struct_size", ctypes.c_uint32),
                ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k_max", ctypes.c_int32), ("layout", ctypes.c_uint32), ("reserved", ctypes.c_uint32)]

    @classmethod
    def make(cls, hidden: int, inter: int, n_experts: int, top_k_max: int) -> "LayerDesc":
        return cls(MOE_ABI_VERSION, ctypes.sizeof(cls), hidden, inter, n_experts, top_k_max,
                   MOE_LAYOUT_ROWMAJOR_V1, 0)


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
