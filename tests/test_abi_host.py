"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/moe_mxfp4.h declares, and rejects invalid arguments
before launching anything."""
import ctypes
import os
import re
import subprocess

import pytest

import mxfp4_routed_expert_fp32_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_mxfp4.h")

pytestmark = pytest.mark.skipif(not os.path.exists(moe.LIB_PATH), reason="libmoe_mxfp4.so not built")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s*(moe_[a-z0-9_]+)\s*\(", src, flags=re.M)
    return sorted(set(names))


PAGE_TITLES = ("Deltafin's custom compiled runtime", "How the native runtime works", "brain.bigb.es \"deltafin\"",
               "Tarfa EXACTNESS")


def test_every_entry_point_cites_its_passage():
    """Each declaration's comment (the nearest one above it) names the page and
    section that define the operation, or says the pages do not describe it."""
    src = open(HEADER).read()
    body = src[src.index("#ifdef __cplusplus"):]
    decl = re.compile(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s*(moe_[a-z0-9_]+)\s*\(", re.M)
    base = src.index("#ifdef __cplusplus")
    missing = []
    for m in decl.finditer(body):
        pos = base + m.start()
        end = src.rfind("*/", 0, pos)
        start = src.rfind("/*", 0, end)
        comment = " ".join(re.sub(r"\n\s*\*(?!/)", " ", src[start:end]).split())
        # the allocation-free forward names the callers it is for instead
        if not (any(t in comment for t in PAGE_TITLES) or "not on the pages" in comment.lower()
                or "callers that cannot allocate" in comment):
            missing.append(m.group(1))
    assert not missing, missing


def test_header_and_binding_agree():
    assert declared_functions() == sorted(moe.EXPORTS)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", moe.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if l.strip())
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing


def test_abi_version_and_strings():
    L = moe.lib()
    assert L.moe_abi_version() == moe.MOE_ABI_VERSION
    for code in moe.STATUS:
        assert L.moe_status_string(code)
    assert L.moe_status_string(12345) == b"unknown status"


def D(**kw):
    base = dict(hidden=7168, inter=1536, n_experts=896, top_k_max=16)
    base.update(kw)
    return moe.LayerDesc.make(**base)


def rc_check(desc):
    return moe.lib().moe_layer_check(ctypes.byref(desc) if desc is not None else None)


def test_descriptor_validation():
    assert rc_check(D()) == 0
    assert rc_check(None) == -1
    d = D(); d.abi_version = 2
    assert rc_check(d) == -10
    d = D(); d.struct_size = 16
    assert rc_check(d) == -10
    d = D(); d.layout = 7
    assert rc_check(d) == -6
    assert rc_check(D(hidden=7000)) == -2
    assert rc_check(D(inter=100)) == -2
    assert rc_check(D(top_k_max=0)) == -2
    assert rc_check(D(top_k_max=65, n_experts=896)) == -2
    assert rc_check(D(n_experts=8, top_k_max=9)) == -2
    assert rc_check(D(hidden=16384)) == -7
    assert rc_check(D(n_experts=5000)) == -7


def test_sizes():
    c, s = moe.packed_bytes(D())
    assert c == 896 * 3 * 7168 * 1536 // 2 and s == 896 * 3 * 7168 * 1536 // 32
    assert c + s == 896 * 17547264
    ws1 = moe.workspace_bytes(D(), 1, 16)
    ws64 = moe.workspace_bytes(D(), 64, 16)
    assert 0 < ws1 < ws64
    with pytest.raises(moe.MoeError) as e:
        moe.workspace_bytes(D(), 0, 16)
    assert e.value.status == -2
    with pytest.raises(moe.MoeError) as e:
        moe.workspace_bytes(D(), 1, 17)
    assert e.value.status == -2


def call_forward(desc, x=16, wr=16, codes=16, scales=16, T=1, k=2, out=16, ws=16, ws_bytes=1 << 30,
                 dtype=1):
    return moe.lib().moe_mxfp4_forward(ctypes.byref(desc), x, dtype, wr, None, codes, scales, T, k, out,
                                       None, None, None, ws, ws_bytes, None)


def test_forward_rejects_before_launch():
    d = D()
    assert call_forward(d, x=None) == -1
    assert call_forward(d, codes=None) == -1
    assert call_forward(d, wr=None) == -1
    assert call_forward(d, dtype=5) == -3
    assert call_forward(d, T=0) == -2
    assert call_forward(d, T=(1 << 20) + 1) == -2   # above the largest token count
    assert call_forward(d, k=0) == -2
    assert call_forward(d, k=17) == -2
    assert call_forward(d, x=8) == -4
    assert call_forward(d, out=24) == -4
    assert call_forward(d, ws=None) == -5
    assert call_forward(d, ws_bytes=100) == -5
    bad = D(); bad.abi_version = 9
    assert call_forward(bad) == -10


def test_noalloc_forward_rejects_before_launch():
    """The allocation-free forward checks like the forward and refuses a call
    whose workspace would not fit its 64 MiB static scratch (at the K3 shape,
    the largest token count that fits is found from moe_workspace_bytes; one
    more is refused) before touching the device."""
    L = moe.lib()
    d = D()

    def call(x=16, wr=16, T=1, k=16, out=16, dtype=1):
        return L.moe_mxfp4_forward_noalloc(ctypes.byref(d), x, dtype, wr, None, 16, 16, T, k, out, None, None,
                                           None, None)
    assert call(x=None) == -1 and call(wr=None) == -1 and call(dtype=4) == -3
    assert call(T=0) == -2 and call(k=17) == -2 and call(out=24) == -4
    fits = max(t for t in range(1, 400) if moe.workspace_bytes(d, t, 16) <= 64 << 20)
    assert 64 <= fits < 399 and moe.workspace_bytes(d, fits + 1, 16) > 64 << 20
    assert call(T=fits + 1) == -12 and call(T=4096) == -12


def test_other_entry_points_reject_before_launch():
    L = moe.lib()
    d = D()
    assert L.moe_mxfp4_pack(ctypes.byref(d), 16, 16, 0, 897, 16, 16, None) == -11
    assert L.moe_mxfp4_pack(ctypes.byref(d), 16, 16, -1, 1, 16, 16, None) == -11
    assert L.moe_mxfp4_pack(ctypes.byref(d), 8, 16, 0, 1, 16, 16, None) == -4
    assert L.moe_mxfp4_dequant(ctypes.byref(d), 16, 16, 896, 0, 16, None) == -11
    assert L.moe_mxfp4_dequant(ctypes.byref(d), 16, 16, 0, 3, 16, None) == -11
    assert L.moe_mxfp4_dequant_bf16(ctypes.byref(d), 16, 16, 896, 0, 16, None) == -11
    assert L.moe_mxfp4_dequant_bf16(ctypes.byref(d), 16, 16, 0, 0, 8, None) == -4
    assert L.moe_mxfp4_dequant_bf16(ctypes.byref(d), None, 16, 0, 0, 16, None) == -1
    assert L.moe_topk_softmax(16, 1, 896, 65, 16, 16, None) == -2
    assert L.moe_topk_softmax(16, 1, 8, 9, 16, 16, None) == -2
    assert L.moe_topk_softmax(16, 1, 5000, 4, 16, 16, None) == -7
    assert L.moe_topk_softmax(None, 1, 8, 2, 16, 16, None) == -1
    assert L.moe_sort_by_expert(16, 0, 8, 2, 16, 16, None, 0, None) == -2
    # from 1024 tokens the sort works in blocks of 256 tokens and needs per-block counts
    assert moe.sort_workspace_bytes(896, 1023, 16) == 0
    assert moe.sort_workspace_bytes(896, 1024, 16) == (4 + 1) * 896 * 4
    assert moe.sort_workspace_bytes(896, 4097, 16) == (17 + 1) * 896 * 4
    assert L.moe_sort_by_expert(16, 4096, 896, 16, 16, 16, None, 0, None) == -5
    assert L.moe_sort_by_expert(16, 4096, 896, 16, 16, 16, 16, 17 * 896 * 4 - 1, None) == -5
    assert L.moe_sort_by_expert(16, 4096, 896, 16, 16, 16, 8, 17 * 896 * 4, None) == -4
    assert L.moe_rmsnorm(16, 16, ctypes.c_float(1e-6), 1, 7, 16, None) == -2
    assert L.moe_residual_add(16, None, 4, None) == -1
    g = ctypes.c_void_p()
    assert L.moe_stack_graph_create(ctypes.byref(d), 0, 16, 16, 16, None, 16, ctypes.c_float(1e-6), 16, 1,
                                    1, 16, 16, 16, 1 << 30, None, ctypes.byref(g)) == -2
    assert L.moe_stack_graph_destroy(None) == 0


def test_grouped_stage_entry_points_reject_before_launch():
    L = moe.lib()
    d = D()
    m = ctypes.c_int32()
    assert L.moe_max_expert_blocks(896, 65536, ctypes.byref(m)) == 0
    assert m.value == 512 + 896
    assert L.moe_max_expert_blocks(8, 3, ctypes.byref(m)) == 0 and m.value == 1 + 3
    assert L.moe_max_expert_blocks(0, 3, ctypes.byref(m)) == -2
    assert L.moe_max_expert_blocks(8, 3, None) == -1
    # capacity below what the sort can produce
    assert L.moe_expert_blocks(16, 896, 65536, 16, 1407, 16, None) == -5
    assert L.moe_expert_blocks(16, 896, 65536, 8, 1408, 16, None) == -4
    assert L.moe_expert_blocks(None, 896, 65536, 16, 1408, 16, None) == -1
    args = (16, 4096, 16, 16, 16, 16, 1408, 16, 16, 16, None)
    assert L.moe_mxfp4_grouped_gate_up(ctypes.byref(d), None, *args[1:]) == -1
    assert L.moe_mxfp4_grouped_gate_up(ctypes.byref(d), 16, 4096, 17, *args[3:]) == -2
    odd = D(hidden=7168 + 32)
    assert L.moe_mxfp4_grouped_gate_up(ctypes.byref(odd), *args) == -7
    # y of 4096 x 16 pairs x 8192 fp32 reaches 2 GiB
    assert L.moe_mxfp4_grouped_gate_up(ctypes.byref(D(hidden=8192)), *args) == -7
    # x of 40000 x 7168 bf16 tokens reaches 1 GiB
    assert L.moe_mxfp4_grouped_gate_up(ctypes.byref(d), 16, 40000, 16, *args[3:]) == -7
    assert L.moe_mxfp4_grouped_gate_up(ctypes.byref(d), 16, 4096, 16, 16, 8, 16, 1408, 16, 16, 16, None) == -4
    dn = (16, 65536, 16, 16, 16, 1408, 16, 16, 16, None)
    assert L.moe_mxfp4_grouped_down(ctypes.byref(d), None, *dn[1:]) == -1
    assert L.moe_mxfp4_grouped_down(ctypes.byref(odd), *dn) == -7
    assert L.moe_mxfp4_grouped_down(ctypes.byref(d), 16, 0, *dn[2:]) == -2
    assert L.moe_mxfp4_grouped_down(ctypes.byref(d), 16, 65536, 16, 16, 16, 1408, 16, 16, 24, None) == -4


def test_mfma_rate_rejects_before_launch():
    """The matrix-core rate entry checks kind, pointers, sizes and alignment on
    the host (fake device addresses: nothing is launched)."""
    f = moe.lib().moe_mfma_rate
    assert f(3, 16, 1, 1, 16, None) == -7      # MOE_ERR_UNSUPPORTED
    assert f(-1, 16, 1, 1, 16, None) == -7
    assert f(0, None, 1, 1, 16, None) == -1    # MOE_ERR_NULL
    assert f(1, 16, 1, 1, None, None) == -1
    assert f(2, 16, 0, 1, 16, None) == -2      # MOE_ERR_SHAPE
    assert f(2, 16, 65537, 1, 16, None) == -2
    assert f(0, 16, 1, 0, 16, None) == -2
    assert f(0, 16, 1, 1000001, 16, None) == -2
    assert f(0, 8, 1, 1, 16, None) == -4       # MOE_ERR_ALIGN
    assert f(0, 16, 1, 1, 24, None) == -4
