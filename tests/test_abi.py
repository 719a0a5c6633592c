"""The C-ABI library on the host: it loads, exports every function that
include/q3moe.h declares, reports the page-printed byte counts, and rejects
bad arguments with a status code before any HIP call is made (so these
tests need no GPU)."""
import ctypes
import re
from pathlib import Path

import pytest

import sparse_moe_decode_q3moe_amd as q3
from sparse_moe_decode_q3moe_amd import _lib

ROOT = Path(__file__).resolve().parent.parent
HEADER = ROOT / "include" / "q3moe.h"

OK, E_NULL, E_SHAPE, E_QTYPE, E_ALIGN, E_WORKSPACE, E_HIP, E_ALIAS = range(8)


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", HEADER.read_text(), flags=re.S)
    return sorted(set(re.findall(r"\b(q3moe_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return q3.library()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) == 29, names
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(_lib.EXPORTS) == names


def test_persistent_path_query(lib):
    """Shapes the block rejects answer -1; T = 0 and shapes outside the
    persistent kernel's range (more than 4 tokens, H != 2048) answer 0 on
    any machine.  Whether a decode shape takes the persistent kernel depends
    on the device, so the GPU tests check that case."""
    f = lib.q3moe_persistent_path
    assert f(1, 2000, 768, 128, 8, q3.Q6_K, 1) == -1        # H % 256
    assert f(1, 2048, 768, 128, 8, 7, 1) == -1               # unknown down qtype
    assert f(1, 2048, 768, 128, 8, q3.Q6_K, 2) == -1
    assert f(-1, 2048, 768, 128, 8, q3.Q6_K, 1) == -1
    assert f(0, 2048, 768, 128, 8, q3.Q6_K, 1) == 0
    assert f(5, 2048, 768, 128, 8, q3.Q6_K, 1) == 0
    assert f(512, 2048, 768, 128, 8, q3.Q6_K, 0) == 0
    assert f(1, 4096, 768, 128, 8, q3.Q6_K, 1) == 0
    assert f(1, 2048, 768, 128, 9, q3.Q6_K, 1) == 0


def test_byte_counts(lib):
    assert lib.q3moe_qtype_block_bytes(q3.Q4_K) == 144
    assert lib.q3moe_qtype_block_bytes(q3.Q6_K) == 210
    assert lib.q3moe_qtype_block_bytes(7) == 0
    assert lib.q3moe_expert_matrix_bytes(q3.Q4_K, 768, 2048) == 884736
    assert lib.q3moe_expert_matrix_bytes(q3.Q6_K, 2048, 768) == 1290240
    assert lib.q3moe_expert_matrix_bytes(q3.Q4_K, 2048, 768) == 884736
    assert lib.q3moe_expert_matrix_bytes(q3.Q4_K, 2, 100) == -1
    assert lib.q3moe_route_workspace_bytes(3, 128) == 4096 + 3 * 128 * 8
    ws = lib.q3moe_expert_ffn_workspace_bytes(5, 2048, 768, 128, 8)
    assert ws >= 5 * 8 * 768 * 4 and ws % 256 == 0
    for s in range(8):
        assert lib.q3moe_status_string(s)


FAKE = ctypes.c_void_p(0x10000)          # aligned, never dereferenced: validation fails first
FAKE_MIS = ctypes.c_void_p(0x10004)


def _experts(base=FAKE, qtype=q3.Q4_K, stride=884736, reserved=0):
    return _lib._Experts(base.value if base else None, qtype, reserved, stride)


def _ffn(lib, T=1, H=2048, F=768, E=128, k=8, hidden=FAKE, idx=FAKE, w=FAKE,
         gate=None, up=None, down=None, out=ctypes.c_void_p(0x40000), acc=0, ws=FAKE,
         ws_bytes=1 << 30):
    gate = gate or _experts()
    up = up or _experts()
    down = down or _experts(qtype=q3.Q6_K, stride=1290240)
    return lib.q3moe_expert_ffn(hidden, T, H, F, E, k, idx, w, gate, up, down, out, acc, ws,
                                ws_bytes, None)


def test_expert_ffn_validation(lib):
    assert _ffn(lib, T=0) == OK                            # nothing to do, nothing enqueued
    assert _ffn(lib, H=2000) == E_SHAPE
    assert _ffn(lib, F=700) == E_SHAPE
    assert _ffn(lib, H=8192) == E_SHAPE
    assert _ffn(lib, k=0) == E_SHAPE
    assert _ffn(lib, k=33, E=64) == E_SHAPE
    assert _ffn(lib, k=9, E=8) == E_SHAPE
    assert _ffn(lib, acc=2) == E_SHAPE
    assert _ffn(lib, hidden=None) == E_NULL
    assert _ffn(lib, out=None) == E_NULL
    assert _ffn(lib, gate=_experts(base=None)) == E_NULL
    assert _ffn(lib, gate=_experts(qtype=q3.Q6_K, stride=1 << 21)) == E_QTYPE
    assert _ffn(lib, down=_experts(qtype=9, stride=1 << 21)) == E_QTYPE
    assert _ffn(lib, gate=_experts(base=FAKE_MIS)) == E_ALIGN
    assert _ffn(lib, gate=_experts(stride=884736 + 8)) == E_ALIGN
    assert _ffn(lib, gate=_experts(stride=884736 - 16)) == E_SHAPE
    assert _ffn(lib, down=_experts(qtype=q3.Q6_K, stride=884736)) == E_SHAPE
    assert _ffn(lib, gate=_experts(reserved=1)) == E_SHAPE
    assert _ffn(lib, hidden=FAKE_MIS) == E_ALIGN
    assert _ffn(lib, out=ctypes.c_void_p(0x10000 + 4096)) == E_ALIAS
    assert _ffn(lib, ws=None) == E_WORKSPACE
    assert _ffn(lib, ws_bytes=100) == E_WORKSPACE
    assert _ffn(lib, ws=FAKE_MIS) == E_ALIGN


def _moe(lib, T=1, H=2048, F=768, E=128, k=8, hidden=FAKE, router=ctypes.c_void_p(0x70000),
         idx=ctypes.c_void_p(0x50000), w=ctypes.c_void_p(0x60000), out=ctypes.c_void_p(0x40000),
         acc=0, ws=ctypes.c_void_p(0x80000), ws_bytes=1 << 30, gate=None, down=None):
    gate = gate or _experts()
    down = down or _experts(qtype=q3.Q6_K, stride=1290240)
    return lib.q3moe_moe_ffn(hidden, T, H, F, E, k, router, gate, _experts(), down, idx, w, out,
                             acc, ws, ws_bytes, None)


def test_moe_ffn_validation(lib):
    """The one-call route + expert FFN checks the union of both calls'
    arguments, and its routing outputs for aliasing."""
    assert _moe(lib, T=0) == OK
    assert _moe(lib, H=2000) == E_SHAPE
    assert _moe(lib, E=1025) == E_SHAPE
    assert _moe(lib, k=9, E=8) == E_SHAPE
    assert _moe(lib, acc=2) == E_SHAPE
    assert _moe(lib, router=None) == E_NULL
    assert _moe(lib, idx=None) == E_NULL
    assert _moe(lib, w=None) == E_NULL
    assert _moe(lib, gate=_experts(qtype=q3.Q6_K, stride=1 << 21)) == E_QTYPE
    assert _moe(lib, router=FAKE_MIS) == E_ALIGN
    assert _moe(lib, idx=ctypes.c_void_p(0x40000 + 64)) == E_ALIAS     # routing into out
    assert _moe(lib, w=ctypes.c_void_p(0x50000 + 16)) == E_ALIAS       # weights over indices
    assert _moe(lib, idx=ctypes.c_void_p(0x10000 + 32)) == E_ALIAS     # routing into hidden
    assert _moe(lib, ws=None) == E_WORKSPACE
    need = lib.q3moe_moe_ffn_workspace_bytes(1, 2048, 768, 128, 8)
    assert need >= lib.q3moe_expert_ffn_workspace_bytes(1, 2048, 768, 128, 8) + \
        lib.q3moe_route_workspace_bytes(1, 128)
    assert _moe(lib, ws_bytes=need - 1) == E_WORKSPACE
    assert _moe(lib, ws=FAKE_MIS) == E_ALIGN


def _moe_pre(lib, T=1, H=2048, F=768, E=128, k=8, hidden=FAKE, gain=ctypes.c_void_p(0x90000),
             eps=1e-6, router=ctypes.c_void_p(0x70000), idx=ctypes.c_void_p(0x50000),
             w=ctypes.c_void_p(0x60000), out=ctypes.c_void_p(0x40000), acc=1,
             ws=ctypes.c_void_p(0x80000), ws_bytes=1 << 30):
    down = _experts(qtype=q3.Q6_K, stride=1290240)
    return lib.q3moe_moe_ffn_prenorm(hidden, T, H, F, E, k, gain, eps, router, _experts(),
                                     _experts(), down, idx, w, out, acc, ws, ws_bytes, None)


def test_moe_ffn_prenorm_validation(lib):
    """The pre-norm MoE block checks what q3moe_moe_ffn checks, plus the gain
    and eps; out may be hidden itself, but no other overlap is accepted.
    (Calls that would pass validation are not made here: they would launch.)"""
    assert _moe_pre(lib, T=0) == OK
    assert _moe_pre(lib, gain=None) == E_NULL
    assert _moe_pre(lib, T=0, gain=None) == OK
    assert _moe_pre(lib, eps=-1e-6) == E_SHAPE
    assert _moe_pre(lib, eps=float("nan")) == E_SHAPE
    assert _moe_pre(lib, eps=float("inf")) == E_SHAPE
    assert _moe_pre(lib, H=2000) == E_SHAPE
    assert _moe_pre(lib, gain=ctypes.c_void_p(0x90004)) == E_ALIGN
    assert _moe_pre(lib, out=ctypes.c_void_p(0x10000 + 16)) == E_ALIAS     # out partly over hidden
    assert _moe_pre(lib, gain=ctypes.c_void_p(0x40000 + 256)) == E_ALIAS   # gain inside out
    assert _moe_pre(lib, out=FAKE, idx=ctypes.c_void_p(0x10000 + 32)) == E_ALIAS
    assert _moe_pre(lib, ws=None) == E_WORKSPACE
    need = lib.q3moe_moe_ffn_workspace_bytes(3, 2048, 768, 128, 8)
    assert _moe_pre(lib, T=3, ws_bytes=need - 1) == E_WORKSPACE
    # the workspace also holds the normalised rows of the multi-kernel path
    assert need >= lib.q3moe_expert_ffn_workspace_bytes(3, 2048, 768, 128, 8) + \
        lib.q3moe_route_workspace_bytes(3, 128) + 3 * 2048 * 4


def _stack(lib, T=1, H=2048, F=768, E=128, k=8, eps=1e-6, x=FAKE, layers=None, n=None,
           idx=ctypes.c_void_p(0x50000), w=ctypes.c_void_p(0x60000), ws=ctypes.c_void_p(0x80000),
           ws_bytes=1 << 30, **layer_kw):
    if layers is None:
        kw = dict(norm_gain=0x90000, router=0x70000, gate=_experts(), up=_experts(),
                  down=_experts(qtype=q3.Q6_K, stride=1290240))
        kw.update(layer_kw)
        one = _lib._MoeLayer(kw["norm_gain"], kw["router"], kw["gate"], kw["up"], kw["down"])
        layers = (_lib._MoeLayer * 2)(one, one)
        n = 2 if n is None else n
    ptr = None if layers is False else ctypes.cast(layers, ctypes.c_void_p)
    return lib.q3moe_moe_stack(x, T, H, F, E, k, eps, ptr, 0 if n is None else n, idx, w, ws,
                               ws_bytes, None)


def test_moe_stack_validation(lib):
    """The layer stack checks every layer's tensors as the pre-norm block
    does, the [layers, T, k] routing outputs for aliasing with x and each
    other, and its larger workspace (the block's plus the residual stream's
    words).  Calls that would pass validation are not made here."""
    assert _stack(lib, T=0) == OK
    assert _stack(lib, n=0) == OK
    assert _stack(lib, n=-1) == E_SHAPE
    assert _stack(lib, layers=False, n=2) == E_NULL
    assert _stack(lib, x=None) == E_NULL
    assert _stack(lib, idx=None) == E_NULL
    assert _stack(lib, norm_gain=None) == E_NULL
    assert _stack(lib, router=None) == E_NULL
    assert _stack(lib, eps=-1.0) == E_SHAPE
    assert _stack(lib, H=2000) == E_SHAPE
    assert _stack(lib, k=9, E=8) == E_SHAPE
    assert _stack(lib, gate=_experts(qtype=q3.Q6_K, stride=1 << 21)) == E_QTYPE
    assert _stack(lib, x=FAKE_MIS) == E_ALIGN
    assert _stack(lib, norm_gain=0x90004) == E_ALIGN
    assert _stack(lib, router=0x10000 + 64) == E_ALIAS                    # router over x
    assert _stack(lib, norm_gain=0x10000 + 256) == E_ALIAS                # gain inside x
    # the second layer's routing (offset T*k*4 = 32 bytes) reaches into the weights
    assert _stack(lib, w=ctypes.c_void_p(0x50000 + 48)) == E_ALIAS
    assert _stack(lib, idx=ctypes.c_void_p(0x10000 + 32)) == E_ALIAS      # routing into x
    assert _stack(lib, ws=None) == E_WORKSPACE
    need = lib.q3moe_moe_stack_workspace_bytes(3, 2048, 768, 128, 8)
    assert need >= lib.q3moe_moe_ffn_workspace_bytes(3, 2048, 768, 128, 8) + 3 * 2048 * 8
    assert _stack(lib, T=3, ws_bytes=need - 1) == E_WORKSPACE
    assert _stack(lib, ws=FAKE_MIS) == E_ALIGN


def _gemv3(lib, T=1, N0=64, N1=8, N2=8, K=64, W0=FAKE, W1=ctypes.c_void_p(0x20000),
           W2=ctypes.c_void_p(0x30000), x=ctypes.c_void_p(0x40000), gain=ctypes.c_void_p(0x50000),
           eps=1e-6, y0=ctypes.c_void_p(0x60000), y1=ctypes.c_void_p(0x70000),
           y2=ctypes.c_void_p(0x80000)):
    return lib.q3moe_bf16_gemv3(W0, N0, W1, N1, W2, N2, K, x, T, gain, eps, y0, y1, y2, None)


def test_bf16_gemv3_validation(lib):
    """The fused projections check every matrix and output; with the norm,
    K <= 16384 and a finite eps >= 0.  (Calls that would pass validation are
    not made here: they would launch.)"""
    assert _gemv3(lib, T=0) == OK
    assert _gemv3(lib, N0=0) == E_SHAPE
    assert _gemv3(lib, N1=-1) == E_SHAPE
    assert _gemv3(lib, K=60) == E_SHAPE
    assert _gemv3(lib, K=16392) == E_SHAPE                                # too long for the norm
    assert _gemv3(lib, eps=-1.0) == E_SHAPE
    assert _gemv3(lib, eps=float("nan")) == E_SHAPE
    assert _gemv3(lib, W1=None) == E_NULL
    assert _gemv3(lib, y2=None) == E_NULL
    assert _gemv3(lib, x=None) == E_NULL
    assert _gemv3(lib, W2=ctypes.c_void_p(0x30008)) == E_ALIGN
    assert _gemv3(lib, gain=ctypes.c_void_p(0x50004)) == E_ALIGN
    assert _gemv3(lib, y1=ctypes.c_void_p(0x70002)) == E_ALIGN
    assert _gemv3(lib, y1=ctypes.c_void_p(0x60000 + 128)) == E_ALIAS     # y1 inside y0
    assert _gemv3(lib, y2=ctypes.c_void_p(0x40000 + 64)) == E_ALIAS      # y2 over x
    assert _gemv3(lib, y0=ctypes.c_void_p(0x20000 + 32)) == E_ALIAS      # y0 over W1
    assert _gemv3(lib, y0=ctypes.c_void_p(0x50000 - 16)) == E_ALIAS      # y0 over the gain


def _pro_kv(lib, T=1, nq=8, nkv=2, D=64, q=FAKE, k=ctypes.c_void_p(0x20000),
            v=ctypes.c_void_p(0x30000), pos=ctypes.c_void_p(0x40000), kc=ctypes.c_void_p(0x100000),
            vc=ctypes.c_void_p(0x200000), S=16, eps=1e-6, base=1e6):
    g = ctypes.c_void_p(0x50000)
    return lib.q3moe_attn_prologue_kv(q, k, v, T, nq, nkv, D, g, g, pos, eps, base, kc, vc, S, None)


def test_attn_prologue_kv_validation(lib):
    """The fused prologue + KV write checks the union of both calls'
    arguments.  (Calls that would pass validation are not made here.)"""
    assert _pro_kv(lib, T=0) == OK
    assert _pro_kv(lib, nq=6, nkv=4) == E_SHAPE
    assert _pro_kv(lib, D=63) == E_SHAPE
    assert _pro_kv(lib, S=0) == E_SHAPE
    assert _pro_kv(lib, base=0.0) == E_SHAPE
    assert _pro_kv(lib, v=None) == E_NULL
    assert _pro_kv(lib, kc=None) == E_NULL
    assert _pro_kv(lib, v=ctypes.c_void_p(0x20000 + 64)) == E_ALIAS           # v over k
    assert _pro_kv(lib, vc=ctypes.c_void_p(0x100000 + 256)) == E_ALIAS        # caches overlap
    assert _pro_kv(lib, pos=ctypes.c_void_p(0x200000 + 8)) == E_ALIAS         # positions in a cache


def _route(lib, T=1, H=2048, E=128, k=8, hidden=FAKE, router=FAKE, idx=FAKE, w=FAKE, ws=FAKE,
           ws_bytes=1 << 20):
    return lib.q3moe_route(hidden, T, H, router, E, k, idx, w, ws, ws_bytes, None)


def test_route_validation(lib):
    assert _route(lib, T=0) == OK
    assert _route(lib, T=-1) == E_SHAPE
    assert _route(lib, k=0) == E_SHAPE
    assert _route(lib, k=33, E=64) == E_SHAPE
    assert _route(lib, E=1025, k=8) == E_SHAPE
    assert _route(lib, k=9, E=8) == E_SHAPE
    assert _route(lib, H=2046) == E_SHAPE
    assert _route(lib, router=None) == E_NULL
    assert _route(lib, idx=None) == E_NULL
    assert _route(lib, hidden=FAKE_MIS) == E_ALIGN
    assert _route(lib, ws=None) == E_WORKSPACE
    assert _route(lib, T=4, ws_bytes=4096 + 4 * 128 * 8 - 1) == E_WORKSPACE


def test_group_validation(lib):
    G = lib.q3moe_group_by_expert
    c, o, p = ctypes.c_void_p(0x20000), ctypes.c_void_p(0x30000), ctypes.c_void_p(0x40000)
    assert G(FAKE, -1, 8, 128, c, o, p, None) == E_SHAPE
    assert G(FAKE, 4, 0, 128, c, o, p, None) == E_SHAPE
    assert G(FAKE, 4, 33, 128, c, o, p, None) == E_SHAPE
    assert G(FAKE, 4, 8, 0, c, o, p, None) == E_SHAPE
    assert G(FAKE, 4, 8, 1025, c, o, p, None) == E_SHAPE
    assert G(FAKE, 1 << 28, 32, 128, c, o, p, None) == E_SHAPE
    assert G(None, 4, 8, 128, c, o, p, None) == E_NULL
    assert G(FAKE, 4, 8, 128, None, o, p, None) == E_NULL
    assert G(FAKE, 4, 8, 128, c, o, None, None) == E_NULL
    assert G(FAKE, 4, 8, 128, c, o, ctypes.c_void_p(0x10000 + 64), None) == E_ALIAS
    assert G(FAKE, 4, 8, 128, c, ctypes.c_void_p(0x20000 + 256), p, None) == E_ALIAS


def test_prologue_and_rmsnorm_validation(lib):
    P = lib.q3moe_attn_prologue
    q, k = FAKE, ctypes.c_void_p(0x10000 + (1 << 20))
    args = dict(T=1, nq=32, nkv=4, D=128)

    def pro(T=1, nq=32, nkv=4, D=128, qp=q, kp=k, qn=FAKE, kn=FAKE, pos=FAKE, eps=1e-6, base=1e7):
        return P(qp, kp, T, nq, nkv, D, qn, kn, pos, eps, base, None)

    assert pro(T=0) == OK
    assert pro(D=127) == E_SHAPE
    assert pro(D=514) == E_SHAPE
    assert pro(nq=30, nkv=4) == E_SHAPE
    assert pro(eps=-1.0) == E_SHAPE
    assert pro(base=0.0) == E_SHAPE
    assert pro(qn=None) == E_NULL
    assert pro(pos=None) == E_NULL
    assert pro(kp=ctypes.c_void_p(0x10000 + 1024)) == E_ALIAS
    R = lib.q3moe_rmsnorm
    assert R(FAKE, 0, 2048, FAKE, 1e-6, FAKE, None) == OK
    assert R(FAKE, 1, 0, FAKE, 1e-6, FAKE, None) == E_SHAPE
    assert R(FAKE, 1, 2048, None, 1e-6, FAKE, None) == E_NULL
    assert R(FAKE, 2, 2048, FAKE, 1e-6, ctypes.c_void_p(0x10000 + 64), None) == E_ALIAS


def test_gemv_validation(lib):
    G = lib.q3moe_bf16_gemv
    W, x, y = FAKE, ctypes.c_void_p(0x100000), ctypes.c_void_p(0x200000)
    assert G(W, 64, 64, x, 0, y, 0, None) == OK
    assert G(W, 64, 64, x, -1, y, 0, None) == E_SHAPE
    assert G(W, 0, 64, x, 1, y, 0, None) == E_SHAPE
    assert G(W, 64, 60, x, 1, y, 0, None) == E_SHAPE          # K % 8
    assert G(W, 64, 0, x, 1, y, 0, None) == E_SHAPE
    assert G(W, 64, 64, x, 1, y, 2, None) == E_SHAPE          # accumulate in {0, 1}
    assert G(None, 64, 64, x, 1, y, 0, None) == E_NULL
    assert G(W, 64, 64, None, 1, y, 0, None) == E_NULL
    assert G(W, 64, 64, x, 1, None, 0, None) == E_NULL
    assert G(FAKE_MIS, 64, 64, x, 1, y, 0, None) == E_ALIGN
    assert G(W, 64, 64, ctypes.c_void_p(0x100004), 1, y, 0, None) == E_ALIGN
    assert G(W, 64, 64, x, 1, ctypes.c_void_p(0x200002), 0, None) == E_ALIGN
    assert G(W, 64, 64, x, 1, ctypes.c_void_p(0x10000 + 512), 0, None) == E_ALIAS   # y inside W
    assert G(W, 64, 64, x, 4, ctypes.c_void_p(0x100000 + 256), 0, None) == E_ALIAS  # y inside x


def test_kv_write_validation(lib):
    K = lib.q3moe_kv_write
    kn, vn, pos = FAKE, ctypes.c_void_p(0x20000), ctypes.c_void_p(0x30000)
    kc, vc = ctypes.c_void_p(0x1000000), ctypes.c_void_p(0x2000000)

    def kv(B=1, nkv=4, D=128, S=4096, k_new=kn, v_new=vn, p=pos, k_c=kc, v_c=vc):
        return K(k_new, v_new, B, nkv, D, p, k_c, v_c, S, None)

    assert kv(B=0) == OK
    assert kv(B=-1) == E_SHAPE
    assert kv(nkv=0) == E_SHAPE
    assert kv(D=0) == E_SHAPE
    assert kv(S=0) == E_SHAPE
    assert kv(nkv=1024, D=128) == E_SHAPE
    assert kv(p=None) == E_NULL
    assert kv(k_c=None) == E_NULL
    assert kv(v_c=ctypes.c_void_p(0x1000000 + 4096)) == E_ALIAS     # caches overlap
    assert kv(k_c=ctypes.c_void_p(0x20000 - 64)) == E_ALIAS         # cache covers v_new


def test_attention_validation(lib):
    A = lib.q3moe_gqa_attention
    WS = lib.q3moe_gqa_attention_workspace_bytes
    assert WS(1, 32, 4, 128, 4096) == 32 * 64 * 130 * 4
    assert WS(16, 32, 4, 128, 4096) == 16 * 32 * 16 * 130 * 4      # 4 tiles per workgroup
    assert WS(1, 32, 4, 96, 4096) == 0                              # unsupported head_dim
    assert WS(1, 30, 4, 128, 4096) == 0
    q, kc, vc = FAKE, ctypes.c_void_p(0x1000000), ctypes.c_void_p(0x2000000)
    ln, out, ws = ctypes.c_void_p(0x30000), ctypes.c_void_p(0x40000), ctypes.c_void_p(0x4000000)
    need = WS(1, 32, 4, 128, 4096)

    def at(B=1, nq=32, nkv=4, D=128, S=4096, scale=0.088, qp=q, k_c=kc, v_c=vc, lens=ln, o=out,
           w=ws, nbytes=need):
        return A(qp, B, nq, nkv, D, k_c, v_c, S, lens, scale, o, w, nbytes, None)

    assert at(B=0) == OK
    assert at(D=96) == E_SHAPE
    assert at(nq=30) == E_SHAPE
    assert at(nq=128, nkv=4) == E_SHAPE                             # group 32 > 16
    assert at(S=0) == E_SHAPE
    assert at(scale=float("nan")) == E_SHAPE
    assert at(scale=float("inf")) == E_SHAPE
    assert at(lens=None) == E_NULL
    assert at(o=None) == E_NULL
    assert at(k_c=ctypes.c_void_p(0x1000008)) == E_ALIGN
    assert at(qp=FAKE_MIS) == E_ALIGN
    assert at(w=None) == E_WORKSPACE
    assert at(nbytes=need - 1) == E_WORKSPACE
    assert at(o=ctypes.c_void_p(0x10000 + 256)) == E_ALIAS          # out overlaps q
    assert at(w=ctypes.c_void_p(0x40000 + 512)) == E_ALIAS          # workspace overlaps out


def test_binding_refuses_host_tensors():
    import torch
    x = torch.zeros(1, 256)
    r = torch.zeros(8, 256)
    with pytest.raises(ValueError):
        q3.q3moe_route(x, r, 2)
