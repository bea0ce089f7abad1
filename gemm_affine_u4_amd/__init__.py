"""Python binding of libqmm.so, the MI355X group-wise affine u4 quantized matmul.

Argument marshalling only: every function here forwards device pointers, sizes
and the current HIP stream to the C ABI of the same name (include/qmm.h) and
raises QmmError on a non-zero status.  Tensors are PyTorch device tensors used
as plain memory: bf16 arrays may be torch.bfloat16 or 16-bit integer tensors
holding the bit patterns, codes any 32-bit integer tensor.  The library must be
built (gemm_affine_u4_amd.build); there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["QmmError", "qmm_linear", "qmm_fused_qkv", "qmm_fused_qkv_rope", "qmm_fused_gate_up_swiglu",
           "qmm_moe_gather", "qmm_linear_fmt", "qmm_fused_qkv_fmt", "qmm_fused_gate_up_swiglu_fmt",
           "qmm_moe_gather_fmt", "qmm_moe_layer",
           "qmm_moe_prefill_workspace_bytes", "qmm_moe_route", "qmm_moe_prefill", "qmm_moe_prefill_noalloc",
           "QMM_NOALLOC_SCRATCH_BYTES", "StepProj", "step_linear", "step_fused_qkv", "step_gate_up_swiglu",
           "qmm_step_plan_bytes", "qmm_step_plan", "qmm_step_run",
           "QMM_STEP_LINEAR", "QMM_STEP_QKV", "QMM_STEP_GATE_UP_SWIGLU", "qmm_status_str", "qmm_abi_version", "load_library", "LIB_PATH",
           "QMM_OUT_BF16", "QMM_OUT_F32", "QMM_FP8_E4M3", "QMM_MOE_GATE_UP_SWIGLU", "QMM_MOE_DOWN_COMBINE", "STATUS"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqmm.so")

QMM_OUT_BF16, QMM_OUT_F32 = 0, 1
QMM_MOE_GATE_UP_SWIGLU, QMM_MOE_DOWN_COMBINE = 0, 1
QMM_FP8_E4M3 = 0x108   # `bits` of the *_fmt calls for fp8 e4m3 codes
QMM_NOALLOC_SCRATCH_BYTES = 64 << 20   # the library's scratch array of qmm_moe_prefill_noalloc
QMM_STEP_LINEAR, QMM_STEP_QKV, QMM_STEP_GATE_UP_SWIGLU = 0, 1, 2
STATUS = {"QMM_OK": 0, "QMM_ERR_NULL": 1, "QMM_ERR_SHAPE": 2, "QMM_ERR_ALIGN": 3, "QMM_ERR_ALIAS": 4,
          "QMM_ERR_ENUM": 5, "QMM_ERR_LAUNCH": 6}

_LIB = None
_P = ctypes.c_void_p


class StepProj(ctypes.Structure):
    """qmm_step_proj of the C ABI (one projection of a decode step)."""
    _fields_ = [("kind", ctypes.c_int32), ("wait_for", ctypes.c_int32), ("K", ctypes.c_int64),
                ("rows", ctypes.c_int64), ("q_out", ctypes.c_int64), ("kv_out", ctypes.c_int64),
                ("x", ctypes.c_void_p), ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("biases", ctypes.c_void_p), ("lin_bias", ctypes.c_void_p), ("out0", ctypes.c_void_p),
                ("out1", ctypes.c_void_p), ("out2", ctypes.c_void_p), ("out_dtype", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]
_I64 = ctypes.c_int64
_INT = ctypes.c_int

_SIGNATURES = {
    "qmm_linear": [_P, _I64, _I64, _P, _P, _P, _I64, _P, _P, _INT, _P],
    "qmm_fused_qkv": [_P, _I64, _I64, _P, _P, _P, _I64, _I64, _P, _P, _P, _P, _INT, _P],
    "qmm_fused_gate_up_swiglu": [_P, _I64, _I64, _P, _P, _P, _I64, _P, _INT, _P],
    "qmm_fused_qkv_rope": [_P, _I64, _I64, _P, _P, _P, _I64, _I64, _I64, _INT, _I64, _P, _P, _I64, _P, _P, _P, _P, _P,
                           _INT, _P],
    "qmm_moe_gather": [_INT, _P, _I64, _P, _P, _P, _I64, _I64, _P, _P, _I64, _P, _INT, _P],
    "qmm_moe_prefill_workspace_bytes": [_I64, _I64, _I64, _I64],
    "qmm_moe_layer": [_P, _I64, _P, _P, _P, _P, _P, _P, _I64, _I64, _P, _P, _I64, _P, _P, _INT, _P],
    "qmm_moe_route": [_P, _I64, _I64, _I64, _P, ctypes.c_size_t, _P],
    "qmm_moe_prefill": [_INT, _P, _I64, _I64, _P, _P, _P, _I64, _I64, _P, _P, _I64, _P, ctypes.c_size_t, _P,
                        _INT, _P],
    "qmm_moe_prefill_noalloc": [_INT, _P, _I64, _I64, _P, _P, _P, _I64, _I64, _P, _P, _I64, _P, _INT, _P],
    "qmm_linear_fmt": [_INT, _I64, _P, _I64, _I64, _P, _P, _P, _I64, _P, _P, _INT, _P],
    "qmm_fused_qkv_fmt": [_INT, _I64, _P, _I64, _I64, _P, _P, _P, _I64, _I64, _P, _P, _P, _P, _INT, _P],
    "qmm_fused_gate_up_swiglu_fmt": [_INT, _I64, _P, _I64, _I64, _P, _P, _P, _I64, _P, _INT, _P],
    "qmm_moe_gather_fmt": [_INT, _I64, _INT, _P, _I64, _P, _P, _P, _I64, _I64, _P, _P, _I64, _P, _INT, _P],
    "qmm_step_plan_bytes": [_P, ctypes.c_int32],
    "qmm_step_plan": [_P, ctypes.c_int32, _P, ctypes.c_size_t, _P],
    "qmm_step_run": [_P, ctypes.c_int32, _P, _P],
    "qmm_status_str": [_INT],
    "qmm_abi_version": [],
}


class QmmError(RuntimeError):
    def __init__(self, status: int, fn: str):
        self.status = status
        super().__init__(f"{fn}: {qmm_status_str(status)} (status {status})")


def load_library():
    """Load libqmm.so (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m gemm_affine_u4_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGNATURES.items():
            f = getattr(lib, name)
            f.argtypes = args
            f.restype = {"qmm_status_str": ctypes.c_char_p,
                         "qmm_moe_prefill_workspace_bytes": ctypes.c_size_t,
                         "qmm_step_plan_bytes": ctypes.c_size_t}.get(name, ctypes.c_int)
        _LIB = lib
    return _LIB


def qmm_status_str(status: int) -> str:
    return load_library().qmm_status_str(int(status)).decode()


def qmm_abi_version() -> int:
    return load_library().qmm_abi_version()


def _ptr(t, what: str):
    """Device pointer of a contiguous CUDA/HIP tensor (None -> NULL); raw ints pass through."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError(f"{what} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return t.data_ptr()


def _out_dtype(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return QMM_OUT_F32
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return QMM_OUT_BF16
    raise ValueError(f"unsupported output dtype {t.dtype}")


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def _check(status: int, fn: str):
    if status != 0:
        raise QmmError(status, fn)


def _mk(x):
    """(M, K) of activations [M, K] or [K]."""
    if x.dim() == 1:
        return 1, x.shape[0]
    return x.shape[0], x.shape[1]


def _need(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _elems(t) -> int:
    return 0 if t is None else t.numel()


def _bytes(t) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def _check_weight(codes, scales, biases, rows: int, K: int, what: str = "weight", bits: int = 4, group: int = 64):
    """The tensors must hold exactly rows x K*bits/32 words and rows x K/group bf16
    scales/biases, so the kernels never read past the end of a caller's buffer."""
    _need(K % 64 == 0 and K > 0 and K % group == 0, f"K={K} must be a positive multiple of 64 and of {group}")
    words = K * (8 if bits == QMM_FP8_E4M3 else bits) // 32
    _need(_bytes(codes) == rows * words * 4, f"{what} codes must hold {rows} x {words} uint32")
    _need(_bytes(scales) == rows * (K // group) * 2, f"{what} scales must hold {rows} x {K // group} bf16")
    _need(_bytes(biases) == rows * (K // group) * 2, f"{what} biases must hold {rows} x {K // group} bf16")


def qmm_linear(x, codes, scales, biases, y, lin_bias=None, stream=None) -> None:
    """y[M, N] = x[M, K] . W^T (+ lin_bias); N = codes.shape[0], out dtype from y."""
    M, K = _mk(x)
    N = codes.shape[0]
    _check_weight(codes, scales, biases, N, K)
    _need(_bytes(x) == M * K * 2, "x must be bf16 [M, K]")
    _need(_elems(y) == M * N, "y must have M x N elements")
    _need(lin_bias is None or _bytes(lin_bias) == N * 2, "lin_bias must be bf16 [N]")
    _check(load_library().qmm_linear(_ptr(x, "x"), M, K, _ptr(codes, "codes"), _ptr(scales, "scales"),
                                     _ptr(biases, "biases"), codes.shape[0], _ptr(lin_bias, "lin_bias"),
                                     _ptr(y, "y"), _out_dtype(y), _stream(stream)), "qmm_linear")


def qmm_fused_qkv(x, codes, scales, biases, q, k, v, lin_bias=None, stream=None) -> None:
    """One matmul over [q_out + 2*kv_out] rows; q_out = q.shape[-1], kv_out = k.shape[-1]."""
    M, K = _mk(x)
    q_out, kv_out = q.shape[-1], k.shape[-1]
    rows = q_out + 2 * kv_out
    _check_weight(codes, scales, biases, rows, K)
    _need(_bytes(x) == M * K * 2, "x must be bf16 [M, K]")
    _need(_elems(q) == M * q_out and _elems(k) == M * kv_out and _elems(v) == M * kv_out,
          "q, k, v must be [M, q_out], [M, kv_out], [M, kv_out]")
    _need(q.dtype == k.dtype == v.dtype, "q, k, v must share a dtype")
    _need(lin_bias is None or _bytes(lin_bias) == rows * 2, "lin_bias must be bf16 [q_out + 2*kv_out]")
    _check(load_library().qmm_fused_qkv(_ptr(x, "x"), M, K, _ptr(codes, "codes"), _ptr(scales, "scales"),
                                        _ptr(biases, "biases"), q.shape[-1], k.shape[-1],
                                        _ptr(lin_bias, "lin_bias"), _ptr(q, "q"), _ptr(k, "k"), _ptr(v, "v"),
                                        _out_dtype(q), _stream(stream)), "qmm_fused_qkv")


def qmm_fused_qkv_rope(x, codes, scales, biases, q, k, v, positions, cos_sin, rot_dim: int, gate=None,
                       lin_bias=None, stream=None) -> None:
    """Fused QKV + split + rotary embedding.  q [M, n_q, head_dim], k/v [M, n_kv, head_dim],
    gate [M, n_q, head_dim] when the Q section carries output-gate heads (then the weight
    has (2*n_q + 2*n_kv)*head_dim rows); positions int32 [M]; cos_sin fp32 [max_pos, rot_dim]."""
    M, K = _mk(x)
    _need(q.dim() == 3 and k.dim() == 3 and v.dim() == 3, "q, k, v must be [M, heads, head_dim]")
    n_q, hd = q.shape[1], q.shape[2]
    n_kv = k.shape[1]
    q_gate = 1 if gate is not None else 0
    rows = (n_q * (1 + q_gate) + 2 * n_kv) * hd
    _check_weight(codes, scales, biases, rows, K)
    _need(_bytes(x) == M * K * 2, "x must be bf16 [M, K]")
    _need(tuple(q.shape) == (M, n_q, hd) and tuple(k.shape) == (M, n_kv, hd) and tuple(v.shape) == (M, n_kv, hd),
          "q, k, v shapes do not match")
    _need(gate is None or tuple(gate.shape) == (M, n_q, hd), "gate must be [M, n_q, head_dim]")
    _need(positions.numel() == M and positions.element_size() == 4, "positions must be int32 [M]")
    _need(cos_sin.dim() == 2 and cos_sin.shape[1] == rot_dim and cos_sin.element_size() == 4,
          "cos_sin must be fp32 [max_pos, rot_dim]")
    _need(lin_bias is None or _bytes(lin_bias) == rows * 2, "lin_bias must be bf16 [rows]")
    od = _out_dtype(q)
    _check(load_library().qmm_fused_qkv_rope(
        _ptr(x, "x"), M, K, _ptr(codes, "codes"), _ptr(scales, "scales"), _ptr(biases, "biases"), n_q, n_kv, hd,
        q_gate, rot_dim, _ptr(positions, "positions"), _ptr(cos_sin, "cos_sin"), cos_sin.shape[0],
        _ptr(lin_bias, "lin_bias"), _ptr(q, "q"), _ptr(gate, "gate"), _ptr(k, "k"), _ptr(v, "v"), od,
        _stream(stream)), "qmm_fused_qkv_rope")


def qmm_fused_gate_up_swiglu(x, codes, scales, biases, h, stream=None) -> None:
    """h[M, I] = silu(gate) * up over [gate; up] rows; I = h.shape[-1]."""
    M, K = _mk(x)
    I = h.shape[-1]
    _check_weight(codes, scales, biases, 2 * I, K)
    _need(_bytes(x) == M * K * 2, "x must be bf16 [M, K]")
    _need(_elems(h) == M * I, "h must be [M, I]")
    _check(load_library().qmm_fused_gate_up_swiglu(_ptr(x, "x"), M, K, _ptr(codes, "codes"),
                                                   _ptr(scales, "scales"), _ptr(biases, "biases"), h.shape[-1],
                                                   _ptr(h, "h"), _out_dtype(h), _stream(stream)),
           "qmm_fused_gate_up_swiglu")


def qmm_moe_gather(stage, inp, codes, scales, biases, expert_ids, out, expert_w=None, stream=None) -> None:
    """Routed experts gathered in place from the grid codes [E, rows, K/8]."""
    E, rows = codes.shape[0], codes.shape[1]
    K = inp.shape[-1]
    topk = expert_ids.shape[0]
    _check_weight(codes, scales, biases, E * rows, K, "expert grid")
    _need(expert_ids.numel() == topk and expert_ids.element_size() == 4, "expert_ids must be int32 [topk]")
    if int(stage) == QMM_MOE_GATE_UP_SWIGLU:
        _need(_bytes(inp) == K * 2, "x must be bf16 [K]")
        _need(_elems(out) == topk * (rows // 2), "out must be [topk, rows/2]")
    else:
        _need(_bytes(inp) == topk * K * 2, "h must be bf16 [topk, K]")
        _need(_elems(out) == rows, "out must be [rows]")
        _need(expert_w is not None and _bytes(expert_w) == topk * 4, "expert_w must be fp32 [topk]")
    _check(load_library().qmm_moe_gather(int(stage), _ptr(inp, "in"), K, _ptr(codes, "codes"),
                                         _ptr(scales, "scales"), _ptr(biases, "biases"), E, rows,
                                         _ptr(expert_ids, "expert_ids"), _ptr(expert_w, "expert_w"),
                                         expert_ids.shape[0], _ptr(out, "out"), _out_dtype(out),
                                         _stream(stream)), "qmm_moe_gather")


def qmm_moe_layer(x, gu_codes, gu_scales, gu_biases, dn_codes, dn_scales, dn_biases, expert_ids, expert_w, h, y,
                  stream=None) -> None:
    """Both stages of the routed experts for one decode token in one call: x [K] bf16,
    gate+up grid [E, 2I, K/8], down grid [E, K, I/8], h [topk, I] bf16 (written), y [K]
    (bf16 or fp32)."""
    E, rows1 = gu_codes.shape[0], gu_codes.shape[1]
    K = x.shape[-1]
    I = rows1 // 2
    topk = expert_ids.shape[0]
    _check_weight(gu_codes, gu_scales, gu_biases, E * rows1, K, "gate+up expert grid")
    _need(dn_codes.shape[0] == E and dn_codes.shape[1] == K, "down grid must be [E, K, I/8]")
    _check_weight(dn_codes, dn_scales, dn_biases, E * K, I, "down expert grid")
    _need(_bytes(x) == K * 2, "x must be bf16 [K]")
    _need(expert_ids.numel() == topk and expert_ids.element_size() == 4, "expert_ids must be int32 [topk]")
    _need(_bytes(expert_w) == topk * 4, "expert_w must be fp32 [topk]")
    _need(_bytes(h) == topk * I * 2, "h must be bf16 [topk, I]")
    _need(_elems(y) == K, "y must be [K]")
    _check(load_library().qmm_moe_layer(_ptr(x, "x"), K, _ptr(gu_codes, "gu_codes"), _ptr(gu_scales, "gu_scales"),
                                        _ptr(gu_biases, "gu_biases"), _ptr(dn_codes, "dn_codes"),
                                        _ptr(dn_scales, "dn_scales"), _ptr(dn_biases, "dn_biases"), E, I,
                                        _ptr(expert_ids, "expert_ids"), _ptr(expert_w, "expert_w"), topk,
                                        _ptr(h, "h"), _ptr(y, "y"), _out_dtype(y), _stream(stream)),
           "qmm_moe_layer")


def qmm_moe_prefill_workspace_bytes(M: int, topk: int, E: int, out_rows: int = 0) -> int:
    """Workspace bytes for M tokens x topk slots over E experts (0 = sizes out of range)."""
    return int(load_library().qmm_moe_prefill_workspace_bytes(M, topk, E, out_rows))


def qmm_moe_route(expert_ids, E: int, workspace, stream=None) -> None:
    """Bucket the (token, slot) pairs of expert_ids int32 [M, topk] by expert into workspace
    (a device uint8 tensor of qmm_moe_prefill_workspace_bytes bytes)."""
    _need(expert_ids.dim() == 2 and expert_ids.element_size() == 4, "expert_ids must be int32 [M, topk]")
    M, topk = expert_ids.shape
    _check(load_library().qmm_moe_route(_ptr(expert_ids, "expert_ids"), M, topk, E, _ptr(workspace, "workspace"),
                                        _bytes(workspace), _stream(stream)), "qmm_moe_route")


def qmm_moe_prefill(stage, inp, codes, scales, biases, expert_ids, workspace, out, expert_w=None,
                    stream=None) -> None:
    """One stage of the routed experts over a batch, on a workspace routed by qmm_moe_route
    with the same expert_ids; grid codes [E, rows, K/8].  Stage 1: inp x [M, K], out
    h [M, topk, rows/2].  Stage 2: inp h [M, topk, K], out y [M, rows], expert_w [M, topk]."""
    E, rows = codes.shape[0], codes.shape[1]
    K = inp.shape[-1]
    _need(expert_ids.dim() == 2 and expert_ids.element_size() == 4, "expert_ids must be int32 [M, topk]")
    M, topk = expert_ids.shape
    _check_weight(codes, scales, biases, E * rows, K, "expert grid")
    if int(stage) == QMM_MOE_GATE_UP_SWIGLU:
        _need(_bytes(inp) == M * K * 2, "x must be bf16 [M, K]")
        _need(_elems(out) == M * topk * (rows // 2), "out must be [M, topk, rows/2]")
    else:
        _need(_bytes(inp) == M * topk * K * 2, "h must be bf16 [M, topk, K]")
        _need(_elems(out) == M * rows, "out must be [M, rows]")
        _need(expert_w is not None and _bytes(expert_w) == M * topk * 4, "expert_w must be fp32 [M, topk]")
    _check(load_library().qmm_moe_prefill(int(stage), _ptr(inp, "in"), M, K, _ptr(codes, "codes"),
                                          _ptr(scales, "scales"), _ptr(biases, "biases"), E, rows,
                                          _ptr(expert_ids, "expert_ids"), _ptr(expert_w, "expert_w"), topk,
                                          _ptr(workspace, "workspace"), _bytes(workspace), _ptr(out, "out"),
                                          _out_dtype(out), _stream(stream)), "qmm_moe_prefill")


def qmm_moe_prefill_noalloc(stage, inp, codes, scales, biases, expert_ids, out, expert_w=None, stream=None) -> None:
    """qmm_moe_prefill without a workspace (the library's own scratch array; no
    qmm_moe_route call first): for callers that cannot allocate.  Same arguments otherwise."""
    E, rows = codes.shape[0], codes.shape[1]
    K = inp.shape[-1]
    _need(expert_ids.dim() == 2 and expert_ids.element_size() == 4, "expert_ids must be int32 [M, topk]")
    M, topk = expert_ids.shape
    _check_weight(codes, scales, biases, E * rows, K, "expert grid")
    if int(stage) == QMM_MOE_GATE_UP_SWIGLU:
        _need(_bytes(inp) == M * K * 2, "x must be bf16 [M, K]")
        _need(_elems(out) == M * topk * (rows // 2), "out must be [M, topk, rows/2]")
    else:
        _need(_bytes(inp) == M * topk * K * 2, "h must be bf16 [M, topk, K]")
        _need(_elems(out) == M * rows, "out must be [M, rows]")
        _need(expert_w is not None and _bytes(expert_w) == M * topk * 4, "expert_w must be fp32 [M, topk]")
    _check(load_library().qmm_moe_prefill_noalloc(int(stage), _ptr(inp, "in"), M, K, _ptr(codes, "codes"),
                                                  _ptr(scales, "scales"), _ptr(biases, "biases"), E, rows,
                                                  _ptr(expert_ids, "expert_ids"), _ptr(expert_w, "expert_w"), topk,
                                                  _ptr(out, "out"), _out_dtype(out), _stream(stream)),
           "qmm_moe_prefill_noalloc")


# ---- a decode step in one launch --------------------------------------------------------

def step_linear(x, codes, scales, biases, y, lin_bias=None, wait_for: int = -1) -> StepProj:
    """A projection y [N] = W x (+ lin_bias) of a decode step (x [K] bf16)."""
    K = x.numel()
    N = codes.shape[0]
    _check_weight(codes, scales, biases, N, K)
    _need(_bytes(x) == K * 2 and _elems(y) == N, "x must be bf16 [K], y [N]")
    _need(lin_bias is None or _bytes(lin_bias) == N * 2, "lin_bias must be bf16 [N]")
    return StepProj(QMM_STEP_LINEAR, wait_for, K, N, 0, 0, _ptr(x, "x"), _ptr(codes, "codes"),
                    _ptr(scales, "scales"), _ptr(biases, "biases"), _ptr(lin_bias, "lin_bias"), _ptr(y, "y"),
                    None, None, _out_dtype(y), 0)


def step_fused_qkv(x, codes, scales, biases, q, k, v, lin_bias=None, wait_for: int = -1) -> StepProj:
    """A fused QKV projection of a decode step: q [q_out], k and v [kv_out]."""
    K = x.numel()
    q_out, kv_out = q.numel(), k.numel()
    rows = q_out + 2 * kv_out
    _check_weight(codes, scales, biases, rows, K)
    _need(_bytes(x) == K * 2 and v.numel() == kv_out, "x must be bf16 [K], v as k")
    _need(lin_bias is None or _bytes(lin_bias) == rows * 2, "lin_bias must be bf16 [rows]")
    _need(_out_dtype(q) == _out_dtype(k) == _out_dtype(v), "q, k, v must share a dtype")
    return StepProj(QMM_STEP_QKV, wait_for, K, rows, q_out, kv_out, _ptr(x, "x"), _ptr(codes, "codes"),
                    _ptr(scales, "scales"), _ptr(biases, "biases"), _ptr(lin_bias, "lin_bias"), _ptr(q, "q"),
                    _ptr(k, "k"), _ptr(v, "v"), _out_dtype(q), 0)


def step_gate_up_swiglu(x, codes, scales, biases, h, wait_for: int = -1) -> StepProj:
    """A fused gate+up+SwiGLU projection of a decode step: h [I] over 2I weight rows."""
    K = x.numel()
    I = h.numel()
    _check_weight(codes, scales, biases, 2 * I, K)
    _need(_bytes(x) == K * 2, "x must be bf16 [K]")
    return StepProj(QMM_STEP_GATE_UP_SWIGLU, wait_for, K, 2 * I, 0, 0, _ptr(x, "x"), _ptr(codes, "codes"),
                    _ptr(scales, "scales"), _ptr(biases, "biases"), None, _ptr(h, "h"), None, None,
                    _out_dtype(h), 0)


def _step_array(projs):
    arr = (StepProj * len(projs))(*projs)
    return arr, len(projs)


def qmm_step_plan_bytes(projs) -> int:
    arr, n = _step_array(projs)
    return int(load_library().qmm_step_plan_bytes(ctypes.cast(arr, ctypes.c_void_p), n))


def qmm_step_plan(projs, plan, stream=None) -> None:
    """Write the plan of `projs` (StepProj list) into `plan` (a device uint8 tensor of at
    least qmm_step_plan_bytes(projs) bytes); synchronises the stream."""
    arr, n = _step_array(projs)
    _check(load_library().qmm_step_plan(ctypes.cast(arr, ctypes.c_void_p), n, _ptr(plan, "plan"), _bytes(plan),
                                        _stream(stream)), "qmm_step_plan")


def qmm_step_run(projs, plan, stream=None) -> None:
    """One run of a planned decode step (projs exactly as given to qmm_step_plan): one
    launch per dependency level and kind."""
    arr, n = _step_array(projs)
    _check(load_library().qmm_step_run(ctypes.cast(arr, ctypes.c_void_p), n, _ptr(plan, "plan"), _stream(stream)),
           "qmm_step_run")


# ---- other formats of the affine family (code width `bits`, group size `group`) ----------

def qmm_linear_fmt(bits: int, group: int, x, codes, scales, biases, y, lin_bias=None, stream=None) -> None:
    """qmm_linear for codes of `bits` bits (one bit stream per row) and `group`-wide groups."""
    M, K = _mk(x)
    N = codes.shape[0]
    _check_weight(codes, scales, biases, N, K, bits=bits, group=group)
    _need(_bytes(x) == M * K * 2, "x must be bf16 [M, K]")
    _need(_elems(y) == M * N, "y must have M x N elements")
    _need(lin_bias is None or _bytes(lin_bias) == N * 2, "lin_bias must be bf16 [N]")
    _check(load_library().qmm_linear_fmt(int(bits), int(group), _ptr(x, "x"), M, K, _ptr(codes, "codes"),
                                         _ptr(scales, "scales"), _ptr(biases, "biases"), N,
                                         _ptr(lin_bias, "lin_bias"), _ptr(y, "y"), _out_dtype(y), _stream(stream)),
           "qmm_linear_fmt")


def qmm_fused_qkv_fmt(bits: int, group: int, x, codes, scales, biases, q, k, v, lin_bias=None, stream=None) -> None:
    M, K = _mk(x)
    q_out, kv_out = q.shape[-1], k.shape[-1]
    rows = q_out + 2 * kv_out
    _check_weight(codes, scales, biases, rows, K, bits=bits, group=group)
    _need(_bytes(x) == M * K * 2, "x must be bf16 [M, K]")
    _need(_elems(q) == M * q_out and _elems(k) == M * kv_out and _elems(v) == M * kv_out, "q/k/v sizes")
    _need(lin_bias is None or _bytes(lin_bias) == rows * 2, "lin_bias must be bf16 [rows]")
    _check(load_library().qmm_fused_qkv_fmt(int(bits), int(group), _ptr(x, "x"), M, K, _ptr(codes, "codes"),
                                            _ptr(scales, "scales"), _ptr(biases, "biases"), q_out, kv_out,
                                            _ptr(lin_bias, "lin_bias"), _ptr(q, "q"), _ptr(k, "k"), _ptr(v, "v"),
                                            _out_dtype(q), _stream(stream)), "qmm_fused_qkv_fmt")


def qmm_fused_gate_up_swiglu_fmt(bits: int, group: int, x, codes, scales, biases, h, stream=None) -> None:
    M, K = _mk(x)
    I = h.shape[-1]
    _check_weight(codes, scales, biases, 2 * I, K, bits=bits, group=group)
    _need(_bytes(x) == M * K * 2, "x must be bf16 [M, K]")
    _need(_elems(h) == M * I, "h must have M x I elements")
    _check(load_library().qmm_fused_gate_up_swiglu_fmt(int(bits), int(group), _ptr(x, "x"), M, K,
                                                       _ptr(codes, "codes"), _ptr(scales, "scales"),
                                                       _ptr(biases, "biases"), I, _ptr(h, "h"), _out_dtype(h),
                                                       _stream(stream)), "qmm_fused_gate_up_swiglu_fmt")


def qmm_moe_gather_fmt(bits: int, group: int, stage, inp, codes, scales, biases, expert_ids, out, expert_w=None,
                       stream=None) -> None:
    E, rows = codes.shape[0], codes.shape[1]
    K = inp.shape[-1]
    topk = expert_ids.shape[0]
    _check_weight(codes, scales, biases, E * rows, K, "expert grid", bits=bits, group=group)
    _need(expert_ids.numel() == topk and expert_ids.element_size() == 4, "expert_ids must be int32 [topk]")
    if int(stage) == QMM_MOE_GATE_UP_SWIGLU:
        _need(_bytes(inp) == K * 2, "x must be bf16 [K]")
        _need(_elems(out) == topk * (rows // 2), "out must be [topk, rows/2]")
    else:
        _need(_bytes(inp) == topk * K * 2, "h must be bf16 [topk, K]")
        _need(_elems(out) == rows, "out must be [rows]")
        _need(expert_w is not None and _bytes(expert_w) == topk * 4, "expert_w must be fp32 [topk]")
    _check(load_library().qmm_moe_gather_fmt(int(bits), int(group), int(stage), _ptr(inp, "in"), K,
                                             _ptr(codes, "codes"), _ptr(scales, "scales"), _ptr(biases, "biases"),
                                             E, rows, _ptr(expert_ids, "expert_ids"), _ptr(expert_w, "expert_w"),
                                             topk, _ptr(out, "out"), _out_dtype(out), _stream(stream)),
           "qmm_moe_gather_fmt")
