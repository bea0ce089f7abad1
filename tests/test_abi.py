"""The C-ABI boundary without a GPU: the library loads, exports every entry point the
header declares, and rejects bad arguments before anything is enqueued.  No call
here reaches a kernel launch: every argument set is invalid on purpose, and the
range logic is exercised through a host-only build of the validation code."""
import ctypes
import os
import re
import subprocess

import pytest

import gemm_affine_u4_amd as qmm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qmm.h")
CSRC = os.path.join(ROOT, "gemm_affine_u4_amd", "csrc")

A = 1 << 20  # a 16-byte aligned fake device address; never dereferenced (every call below fails validation)


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(qmm_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(["qmm_linear", "qmm_fused_qkv", "qmm_fused_qkv_rope", "qmm_fused_gate_up_swiglu",
                                           "qmm_linear_fmt", "qmm_fused_qkv_fmt", "qmm_fused_gate_up_swiglu_fmt",
                                           "qmm_moe_gather_fmt",
                                           "qmm_moe_gather", "qmm_moe_prefill_workspace_bytes",
                                           "qmm_moe_layer",
                                           "qmm_moe_route", "qmm_moe_prefill", "qmm_moe_prefill_noalloc",
                                           "qmm_step_plan_bytes", "qmm_step_plan", "qmm_step_run",
                                           "qmm_status_str",
                                           "qmm_abi_version"])


def test_library_exports_every_declared_symbol():
    lib = qmm.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", qmm.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (qmm_\w+)$", out, re.M))
    assert set(declared_functions()) <= exported


def test_version_and_status_strings():
    assert qmm.qmm_abi_version() == 2
    for name, code in qmm.STATUS.items():
        assert qmm.qmm_status_str(code).startswith(name)
    assert qmm.qmm_status_str(99) == "QMM_ERR_UNKNOWN"


def _linear(x=A, M=1, K=512, codes=A + (1 << 16), s=A + (1 << 18), b=A + (1 << 19), N=64, lb=None,
            y=A + (1 << 21), od=0):
    return qmm.load_library().qmm_linear(x, M, K, codes, s, b, N, lb, y, od, None)


def _qkv(x=A, M=1, K=512, codes=A + (1 << 16), s=A + (1 << 18), b=A + (1 << 19), qo=64, kvo=16, lb=None,
         q=A + (1 << 21), k=A + (1 << 21) + 4096, v=A + (1 << 21) + 8192, od=0):
    return qmm.load_library().qmm_fused_qkv(x, M, K, codes, s, b, qo, kvo, lb, q, k, v, od, None)


S = qmm.STATUS


def test_null_pointers():
    assert _linear(x=None) == S["QMM_ERR_NULL"]
    assert _linear(codes=None) == S["QMM_ERR_NULL"]
    assert _linear(y=None) == S["QMM_ERR_NULL"]
    assert _qkv(k=None) == S["QMM_ERR_NULL"]
    lib = qmm.load_library()
    assert lib.qmm_fused_gate_up_swiglu(A, 1, 512, A + 65536, None, A + 2 ** 19, 8, A + 2 ** 21, 0, None) == 1
    # stage 2 needs combine weights
    assert lib.qmm_moe_gather(1, A, 512, A + 65536, A + 2 ** 18, A + 2 ** 19, 4, 64, A + 2 ** 22, None, 2,
                              A + 2 ** 21, 0, None) == S["QMM_ERR_NULL"]


def test_noalloc_rejects_sizes_beyond_its_scratch_before_any_device_call():
    """qmm_moe_prefill_noalloc checks the workspace the call would need against its scratch
    size (QMM_NOALLOC_SCRATCH_BYTES) before it looks the scratch up or enqueues anything:
    stage 2 of 2048 tokens x top-8 into 2048 output rows needs 134 MB of products."""
    lib = qmm.load_library()
    need = lib.qmm_moe_prefill_workspace_bytes(2048, 8, 256, 2048)
    assert need > qmm.QMM_NOALLOC_SCRATCH_BYTES
    st = lib.qmm_moe_prefill_noalloc(1, A, 2048, 512, A + 2 ** 24, A + 2 ** 26, A + 2 ** 27, 256, 2048,
                                     A + 2 ** 28, A + 2 ** 29, 8, A + 2 ** 30, 1, None)
    assert st == S["QMM_ERR_SHAPE"]
    # bad stage and NULL pointers are reported as for qmm_moe_prefill
    assert lib.qmm_moe_prefill_noalloc(2, A, 4, 512, A + 2 ** 24, A + 2 ** 26, A + 2 ** 27, 8, 64,
                                       A + 2 ** 28, A + 2 ** 29, 2, A + 2 ** 30, 1, None) == S["QMM_ERR_ENUM"]
    assert lib.qmm_moe_prefill_noalloc(1, A, 4, 512, A + 2 ** 24, A + 2 ** 26, A + 2 ** 27, 8, 64,
                                       A + 2 ** 28, None, 2, A + 2 ** 30, 1, None) == S["QMM_ERR_NULL"]


@pytest.mark.parametrize("K", [0, 32, 100, 96, 65536 + 64, -64])
def test_bad_K(K):
    assert _linear(K=K) == S["QMM_ERR_SHAPE"]


def test_bad_sizes():
    assert _linear(M=0) == S["QMM_ERR_SHAPE"]
    assert _linear(N=0) == S["QMM_ERR_SHAPE"]
    assert _qkv(qo=0) == S["QMM_ERR_SHAPE"]
    assert _qkv(kvo=0) == S["QMM_ERR_SHAPE"]
    lib = qmm.load_library()
    # topk out of range, odd gate+up rows, stage-2 K too large
    assert lib.qmm_moe_gather(0, A, 512, A + 65536, A + 2 ** 18, A + 2 ** 19, 4, 64, A + 2 ** 22, None, 0,
                              A + 2 ** 21, 0, None) == S["QMM_ERR_SHAPE"]
    assert lib.qmm_moe_gather(0, A, 512, A + 65536, A + 2 ** 18, A + 2 ** 19, 4, 63, A + 2 ** 22, None, 2,
                              A + 2 ** 21, 0, None) == S["QMM_ERR_SHAPE"]
    assert lib.qmm_moe_gather(1, A, 8192, A + 65536, A + 2 ** 18, A + 2 ** 19, 4, 64, A + 2 ** 22,
                              A + 2 ** 23, 2, A + 2 ** 21, 0, None) == S["QMM_ERR_SHAPE"]


def test_bad_enums():
    assert _linear(od=2) == S["QMM_ERR_ENUM"]
    lib = qmm.load_library()
    assert lib.qmm_moe_gather(7, A, 512, A + 65536, A + 2 ** 18, A + 2 ** 19, 4, 64, A + 2 ** 22, None, 2,
                              A + 2 ** 21, 0, None) == S["QMM_ERR_ENUM"]


def test_misaligned():
    assert _linear(x=A + 2) == S["QMM_ERR_ALIGN"]
    assert _linear(codes=A + (1 << 16) + 4) == S["QMM_ERR_ALIGN"]
    assert _linear(s=A + (1 << 18) + 1) == S["QMM_ERR_ALIGN"]
    assert _linear(y=A + (1 << 21) + 1) == S["QMM_ERR_ALIGN"]
    assert _linear(y=A + (1 << 21) + 2, od=1) == S["QMM_ERR_ALIGN"]   # fp32 output needs 4 bytes
    assert _linear(lb=A + (1 << 20) + 1) == S["QMM_ERR_ALIGN"]


def test_overlapping_outputs_and_inputs_are_rejected():
    # the split-view trap: K and V inside one buffer, overlapping
    assert _qkv(k=A + (1 << 21) + 100, v=A + (1 << 21) + 128) == S["QMM_ERR_ALIAS"]
    # Q overlapping K
    assert _qkv(q=A + (1 << 21), k=A + (1 << 21) + 64) == S["QMM_ERR_ALIAS"]
    # output on top of the activations or the weight
    assert _linear(y=A) == S["QMM_ERR_ALIAS"]
    assert _linear(y=A + (1 << 16) + 512) == S["QMM_ERR_ALIAS"]
    assert _linear(y=A + (1 << 19) + 16) == S["QMM_ERR_ALIAS"]


# ---- other formats ---------------------------------------------------------------------

def _linear_fmt(bits=4, group=64, K=512, **kw):
    args = dict(x=A, M=1, codes=A + (1 << 16), s=A + (1 << 18), b=A + (1 << 19), N=64, lb=None, y=A + (1 << 21),
                od=0)
    args.update(kw)
    return qmm.load_library().qmm_linear_fmt(bits, group, args["x"], args["M"], K, args["codes"], args["s"],
                                             args["b"], args["N"], args["lb"], args["y"], args["od"], None)


def test_format_validation():
    for bits, group, K in [(5, 64, 512), (4, 16, 512), (4, 96, 576), (4, 256, 512), (4, 128, 320), (1, 64, 512),
                           (qmm.QMM_FP8_E4M3, 64, 49216), (8, 64, 49216), (0x107, 64, 512)]:
        assert _linear_fmt(bits, group, K) == S["QMM_ERR_SHAPE"], (bits, group, K)
    # the plain call is the (4, 64) format: the same validation result for a bad pointer
    assert _linear_fmt(4, 64, x=A + 2) == S["QMM_ERR_ALIGN"] == _linear(x=A + 2)
    # group 128 with K = 512, group 32: past the shape checks (fails only on the alias below)
    assert _linear_fmt(4, 128, 512, y=A) == S["QMM_ERR_ALIAS"]
    assert _linear_fmt(4, 32, 512, y=A) == S["QMM_ERR_ALIAS"]
    # the alias ranges follow the format's sizes: K=512, N=64 at group 32 -> scales 64 x 16 x 2 B
    assert _linear_fmt(4, 32, 512, y=A + (1 << 18) + 64 * 16 * 2 - 2) == S["QMM_ERR_ALIAS"]
    assert _linear_fmt(4, 128, 512, y=A + (1 << 18) + 64 * 4 * 2 - 2) == S["QMM_ERR_ALIAS"]


# ---- fused QKV with rotary embedding ------------------------------------------------

def _rope(x=A, M=1, K=512, codes=A + (1 << 16), s=A + (1 << 18), b=A + (1 << 19), nq=2, nkv=1, hd=64, qg=0,
          rot=64, pos=A + (1 << 22), cs=A + (1 << 23), maxpos=16, lb=None, q=A + (1 << 21), g=None,
          k=A + (1 << 21) + 4096, v=A + (1 << 21) + 8192, od=0):
    return qmm.load_library().qmm_fused_qkv_rope(x, M, K, codes, s, b, nq, nkv, hd, qg, rot, pos, cs, maxpos, lb,
                                                 q, g, k, v, od, None)


def test_rope_validation():
    assert _rope(pos=None) == S["QMM_ERR_NULL"]
    assert _rope(cs=None) == S["QMM_ERR_NULL"]
    assert _rope(qg=1, g=None) == S["QMM_ERR_NULL"]      # output gate heads need a gate buffer
    assert _rope(od=3) == S["QMM_ERR_ENUM"]
    assert _rope(hd=63, rot=62) == S["QMM_ERR_SHAPE"]     # odd head_dim
    assert _rope(rot=66) == S["QMM_ERR_SHAPE"]            # rot_dim > head_dim
    assert _rope(rot=31) == S["QMM_ERR_SHAPE"]            # odd rot_dim
    assert _rope(rot=0) == S["QMM_ERR_SHAPE"]
    assert _rope(nkv=0) == S["QMM_ERR_SHAPE"]
    assert _rope(qg=2, g=A + (1 << 24)) == S["QMM_ERR_SHAPE"]
    assert _rope(maxpos=0) == S["QMM_ERR_SHAPE"]
    assert _rope(pos=A + (1 << 22) + 2) == S["QMM_ERR_ALIGN"]
    assert _rope(cs=A + (1 << 23) + 1) == S["QMM_ERR_ALIGN"]
    assert _rope(k=A + (1 << 21) + 64) == S["QMM_ERR_ALIAS"]          # k overlaps q
    assert _rope(q=A + (1 << 22)) == S["QMM_ERR_ALIAS"]               # q on the positions
    assert _rope(v=A + (1 << 23) + 8) == S["QMM_ERR_ALIAS"]           # v on the table
    assert _rope(qg=1, g=A + (1 << 21) + 4096 + 32) == S["QMM_ERR_ALIAS"]   # gate overlaps k


# ---- routed experts over a batch (prefill) --------------------------------------

WS = A + (1 << 24)   # 256-byte aligned fake workspace


def _route(ids=A, M=16, topk=2, E=4, ws=WS, nbytes=None):
    if nbytes is None:
        nbytes = qmm.qmm_moe_prefill_workspace_bytes(M, topk, E, 0)
    return qmm.load_library().qmm_moe_route(ids, M, topk, E, ws, nbytes, None)


def _prefill(stage=0, inp=A, M=16, K=512, codes=A + (1 << 16), s=A + (1 << 18), b=A + (1 << 19), E=4,
             rows=64, ids=A + (1 << 22), ew=A + (1 << 23), topk=2, ws=WS, nbytes=None, out=A + (1 << 21), od=0):
    if nbytes is None:
        nbytes = qmm.qmm_moe_prefill_workspace_bytes(M, topk, E, 0 if stage == 0 else rows)
    return qmm.load_library().qmm_moe_prefill(stage, inp, M, K, codes, s, b, E, rows, ids, ew, topk, ws, nbytes,
                                              out, od, None)


def test_moe_workspace_bytes():
    wb = qmm.qmm_moe_prefill_workspace_bytes
    assert wb(0, 8, 256) == 0 and wb(65536, 8, 256) == 0
    assert wb(16, 0, 4) == 0 and wb(16, 65, 4) == 0
    assert wb(16, 2, 0) == 0 and wb(16, 2, 4097) == 0
    n0 = wb(2048, 8, 256, 0)
    assert n0 % 256 == 0 and n0 >= 2048 * 8 * 4            # at least the bucketed pair list
    # the stage-2 products are fp32 [M*topk][out_rows] on top of the routing
    assert wb(2048, 8, 256, 2048) - n0 == 2048 * 8 * 2048 * 4
    assert wb(1, 1, 1) > 0 and wb(65535, 64, 4096) > 0


def test_moe_route_validation():
    assert _route(ids=None) == S["QMM_ERR_NULL"]
    assert _route(ws=None) == S["QMM_ERR_NULL"]
    assert _route(M=0) == S["QMM_ERR_SHAPE"]
    assert _route(E=5000) == S["QMM_ERR_SHAPE"]
    assert _route(nbytes=qmm.qmm_moe_prefill_workspace_bytes(16, 2, 4) - 4) == S["QMM_ERR_SHAPE"]
    assert _route(ws=WS + 128) == S["QMM_ERR_ALIGN"]
    assert _route(ids=A + 2) == S["QMM_ERR_ALIGN"]
    assert _route(ids=WS + 64) == S["QMM_ERR_ALIAS"]


def test_moe_prefill_validation():
    assert _prefill(stage=3) == S["QMM_ERR_ENUM"]
    assert _prefill(od=4) == S["QMM_ERR_ENUM"]
    assert _prefill(stage=1, ew=None) == S["QMM_ERR_NULL"]
    assert _prefill(ws=None) == S["QMM_ERR_NULL"]
    assert _prefill(ids=None) == S["QMM_ERR_NULL"]
    assert _prefill(rows=63) == S["QMM_ERR_SHAPE"]                  # odd gate+up rows
    assert _prefill(K=96) == S["QMM_ERR_SHAPE"]
    assert _prefill(topk=65) == S["QMM_ERR_SHAPE"]
    # stage 2 needs room for its fp32 products: a stage-1-sized workspace is too small
    assert _prefill(stage=1, nbytes=qmm.qmm_moe_prefill_workspace_bytes(16, 2, 4, 0)) == S["QMM_ERR_SHAPE"]
    assert _prefill(ws=WS + 16) == S["QMM_ERR_ALIGN"]
    assert _prefill(inp=A + 8) == S["QMM_ERR_ALIGN"]
    assert _prefill(out=A + (1 << 21) + 2, od=1) == S["QMM_ERR_ALIGN"]
    assert _prefill(out=WS + 256) == S["QMM_ERR_ALIAS"]             # out inside the workspace
    assert _prefill(ws=A + (1 << 16)) == S["QMM_ERR_ALIAS"]         # workspace on the weights
    assert _prefill(out=A + (1 << 22)) == S["QMM_ERR_ALIAS"]        # out on the expert ids


def _layer(x=A, K=512, gc=A + (1 << 16), gs=A + (1 << 18), gb=A + (1 << 19), dc=A + (1 << 20), ds=A + (1 << 21),
           db=A + (1 << 22), E=4, I=128, ids=A + (1 << 23), ew=A + (1 << 24), topk=2, h=A + (1 << 25),
           y=A + (1 << 26), od=0):
    return qmm.load_library().qmm_moe_layer(x, K, gc, gs, gb, dc, ds, db, E, I, ids, ew, topk, h, y, od, None)


def test_moe_layer_validation():
    for kw in ("x", "gc", "dc", "db", "ids", "ew", "h", "y"):
        assert _layer(**{kw: None}) == S["QMM_ERR_NULL"], kw
    assert _layer(od=3) == S["QMM_ERR_ENUM"]
    assert _layer(K=96) == S["QMM_ERR_SHAPE"]
    assert _layer(I=5184) == S["QMM_ERR_SHAPE"]                   # stage 2 in one K slice only
    assert _layer(topk=0) == S["QMM_ERR_SHAPE"] and _layer(topk=65) == S["QMM_ERR_SHAPE"]
    assert _layer(E=0) == S["QMM_ERR_SHAPE"]
    assert _layer(h=A + (1 << 25) + 2) == S["QMM_ERR_ALIGN"]
    assert _layer(y=A + 8) == S["QMM_ERR_ALIAS"]                   # y on x
    assert _layer(h=A + (1 << 26) + 64) == S["QMM_ERR_ALIAS"]      # h over y


def _proj(kind=1, wait_for=-1, K=1024, rows=96, q_out=64, kv_out=16, x=A, codes=A + (1 << 16), s=A + (1 << 18),
          b=A + (1 << 19), lb=None, o0=A + (1 << 21), o1=A + (1 << 22), o2=A + (1 << 23), od=0, reserved=0):
    return qmm.StepProj(kind, wait_for, K, rows, q_out, kv_out, x, codes, s, b, lb, o0, o1, o2, od, reserved)


def _plan(projs, plan=A + (1 << 24), nbytes=1 << 20):
    arr = (qmm.StepProj * len(projs))(*projs)
    return qmm.load_library().qmm_step_plan(ctypes.cast(arr, ctypes.c_void_p), len(projs), plan, nbytes, None)


def _run(projs, plan=A + (1 << 24)):
    arr = (qmm.StepProj * len(projs))(*projs) if projs else None
    return qmm.load_library().qmm_step_run(ctypes.cast(arr, ctypes.c_void_p) if arr else None, len(projs), plan,
                                           None)


def test_step_validation_before_any_device_call():
    pb = qmm.qmm_step_plan_bytes
    assert pb([_proj(kind=7)]) == 0
    assert pb([_proj(K=512, rows=96)]) == 0 and pb([_proj(K=1000)]) == 0     # K > 512, a multiple of 64
    assert pb([_proj(), _proj(wait_for=1)]) == 0                             # waits for itself
    assert pb([_proj(wait_for=-2)]) == 0 and pb([_proj(rows=0)]) == 0
    assert _plan([]) == S["QMM_ERR_SHAPE"]
    assert _plan([_proj(kind=7)]) == S["QMM_ERR_ENUM"]
    assert _plan([_proj(x=None)]) == S["QMM_ERR_NULL"]
    assert _plan([_proj(o1=None)]) == S["QMM_ERR_NULL"]                        # QKV needs three outputs
    assert _plan([_proj(od=5)]) == S["QMM_ERR_ENUM"]
    assert _plan([_proj(reserved=1)]) == S["QMM_ERR_SHAPE"]
    assert _plan([_proj(), _proj(wait_for=1)]) == S["QMM_ERR_SHAPE"]
    assert _plan([_proj(q_out=60)]) == S["QMM_ERR_SHAPE"]                     # q + 2 kv != rows
    assert _plan([_proj(kind=2, rows=97)]) == S["QMM_ERR_SHAPE"]              # gate+up rows even
    assert _plan([_proj(kind=2, rows=96, lb=A + (1 << 20))]) == S["QMM_ERR_SHAPE"]  # no bias on gate+up
    assert _plan([_proj(K=65536 * 2)]) == S["QMM_ERR_SHAPE"]
    assert _plan([_proj(x=A + 8)]) == S["QMM_ERR_ALIGN"]
    assert _plan([_proj(od=1, o0=A + (1 << 21) + 2)]) == S["QMM_ERR_ALIGN"]
    assert _run([]) == S["QMM_ERR_NULL"]
    assert _run([_proj(kind=9)]) == S["QMM_ERR_SHAPE"]
    assert _run([_proj(), _proj(wait_for=3)]) == S["QMM_ERR_SHAPE"]
    assert _run([_proj(codes=None)]) == S["QMM_ERR_NULL"]
    assert _run([_proj()], plan=A + 64) == S["QMM_ERR_ALIGN"]


# ---- host-only build of the validation code ------------------------------------

@pytest.fixture(scope="module")
def shim(tmp_path_factory):
    d = tmp_path_factory.mktemp("shim")
    so = str(d / "libqmm_validate_host.so")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fsanitize=undefined", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include", "-I", CSRC,
           os.path.join(CSRC, "qmm_validate.cpp"), os.path.join(ROOT, "tests", "validate_shim.cpp"), "-o", so]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    lib = ctypes.CDLL(so)
    lib.shim_aligned.argtypes = [ctypes.c_void_p, ctypes.c_ulong]
    lib.shim_k_ok.argtypes = [ctypes.c_longlong]
    arr = ctypes.POINTER(ctypes.c_ulonglong)
    lib.shim_any_alias.argtypes = [arr, ctypes.c_int, arr, ctypes.c_int]
    return lib


def _ranges(pairs):
    flat = [v for p in pairs for v in p]
    return (ctypes.c_ulonglong * max(1, len(flat)))(*flat), len(pairs)


def _alias(shim, outs, ins):
    o, no = _ranges(outs)
    i, ni = _ranges(ins)
    return shim.shim_any_alias(o, no, i, ni)


def test_range_logic_touching_is_not_overlap(shim):
    assert _alias(shim, [(1000, 100), (1100, 50)], []) == 0          # adjacent outputs
    assert _alias(shim, [(1000, 100), (1099, 50)], []) == 1          # one byte shared
    assert _alias(shim, [(1000, 100)], [(900, 100)]) == 0            # input ends where output starts
    assert _alias(shim, [(1000, 100)], [(900, 101)]) == 1
    assert _alias(shim, [(1000, 100)], [(1050, 1)]) == 1             # input inside output
    assert _alias(shim, [(1000, 100)], [(0, 0), (5000, 10)]) == 0    # null / disjoint inputs
    assert _alias(shim, [(1000, 0)], [(1000, 10)]) == 0              # empty output range
    assert _alias(shim, [(1000, 10), (2000, 10), (1005, 1)], []) == 1


def test_alignment_and_k_rules(shim):
    assert shim.shim_aligned(4096, 16) == 1 and shim.shim_aligned(4104, 16) == 0 and shim.shim_aligned(4104, 8) == 1
    for K, ok in [(64, 1), (128, 1), (65536, 1), (65600, 0), (0, 0), (63, 0), (96, 0), (-64, 0)]:
        assert shim.shim_k_ok(K) == ok, K
