"""ctypes binding of libqma (include/qma.h): argument marshalling only.

Functions keep the C names. Tensor arguments are torch tensors on the GPU
(their data_ptr() is passed through). ``stream`` defaults to torch's current
stream. A non-OK status raises :class:`QmaError` carrying the library's
detail text. Every computation happens in the HIP library. There is no
Python or CPU fallback: if libqma.so is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqma.so")

SCHEDULE_SEMI_STATIC, SCHEDULE_DYNAMIC, SCHEDULE_GANG, SCHEDULE_STREAM_K = 0, 1, 2, 3
LAYER_FUSE_SILU_MUL = 1
SCHEDULE_NAMES = {0: "semi_static", 1: "dynamic", 2: "gang", 3: "stream_k"}

QMA_OK, QMA_ERR_INVALID_ARG, QMA_ERR_UNSUPPORTED, QMA_ERR_ROUTING, \
    QMA_ERR_WORKSPACE, QMA_ERR_HIP = range(6)
PATH_INDEXED, PATH_GROUPED_CONTIGUOUS, PATH_GROUPED_MASKED = 0, 1, 2
DTYPE_BF16, DTYPE_FP16, DTYPE_FP32 = 1, 2, 3
PACK_INT32_K8 = 1
KERNEL_SMALL_M, KERNEL_LARGE_M, KERNEL_LARGE_M_PC = 1, 2, 3
LARGE_M_KERNELS = (KERNEL_LARGE_M, KERNEL_LARGE_M_PC)
PROFILES = {0: "generic", 1: "ep_gate_up", 2: "ep_down", 3: "tp_gate_up", 4: "tp_down"}

# Every symbol include/qma.h declares.
EXPORTS = (
    "qma_layer_create", "qma_layer_create_ex", "qma_layer_destroy", "qma_layer_info",
    "qma_packed_weight_bytes", "qma_prepack", "qma_plan_indexed",
    "qma_plan_grouped", "qma_workspace_bytes", "qma_align_sizes",
    "qma_moe_align", "qma_validate_routing", "qma_validate_contiguous",
    "qma_indexed_gemm", "qma_indexed_gemm_scratch", "qma_grouped_contiguous_gemm",
    "qma_grouped_masked_gemm", "qma_silu_and_mul", "qma_moe_combine", "qma_router_topk",
    "qma_status_str", "qma_last_error_detail", "qma_version",
)


class QmaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        self.detail = detail
        super().__init__(f"{_status_name(status)}: {detail}")


class QuantDesc(ctypes.Structure):
    _fields_ = [("weight_bits", ctypes.c_int32), ("zero_point", ctypes.c_int32),
                ("group_size", ctypes.c_int32), ("scale_dtype", ctypes.c_int32),
                ("act_dtype", ctypes.c_int32), ("pack_format", ctypes.c_int32)]


def w4a16_desc(**over) -> QuantDesc:
    d = dict(weight_bits=4, zero_point=8, group_size=32, scale_dtype=DTYPE_BF16,
             act_dtype=DTYPE_BF16, pack_format=PACK_INT32_K8)
    d.update(over)
    return QuantDesc(**d)


class Plan(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "path", "kernel", "block_m", "block_n", "split_k", "k_depth",
        "num_experts", "n", "k", "rows", "tok_e_x100", "est_tiles", "profile",
        "waves_k", "expected_m", "n_stream", "schedule")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


_lib = None


def lib():
    """Load libqma.so (built in-tree by quantized_moe_align_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: the HIP library is not built "
                              "(run __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        sig = {
            "qma_layer_create": (I32, [ctypes.POINTER(QuantDesc), I32, I32, I32, I32,
                                       ctypes.POINTER(P)]),
            "qma_layer_create_ex": (I32, [ctypes.POINTER(QuantDesc), I32, I32, I32, I32,
                                          ctypes.c_uint32, ctypes.POINTER(P)]),
            "qma_layer_destroy": (None, [P]),
            "qma_layer_info": (I32, [P] + [ctypes.POINTER(I32)] * 5),
            "qma_packed_weight_bytes": (SZ, [P]),
            "qma_prepack": (I32, [P, P, P, P, P]),
            "qma_plan_indexed": (I32, [P, I32, I32, I32, ctypes.POINTER(Plan)]),
            "qma_plan_grouped": (I32, [P, I32, I32, ctypes.POINTER(Plan)]),
            "qma_workspace_bytes": (SZ, [ctypes.POINTER(Plan)]),
            "qma_align_sizes": (I32, [I32, I32, I32, I32, ctypes.POINTER(I32),
                                      ctypes.POINTER(I32)]),
            "qma_moe_align": (I32, [P, I32, I32, I32, I32, P, P, P, I32, P]),
            "qma_validate_routing": (I32, [P, I32, I32, I32, I32, P, P, P, I32, P]),
            "qma_validate_contiguous": (I32, [P, I32, I32, P]),
            "qma_indexed_gemm": (I32, [P, ctypes.POINTER(Plan), P, I32, I32, P, P, P, P,
                                       I32, I32, P, P, P, SZ, P]),
            "qma_indexed_gemm_scratch": (I32, [P, ctypes.POINTER(Plan), P, I32, I32, P, P, P,
                                               P, I32, I32, P, P, P]),
            "qma_grouped_contiguous_gemm": (I32, [P, ctypes.POINTER(Plan), P, P, I32, P, P,
                                                  P, SZ, P]),
            "qma_grouped_masked_gemm": (I32, [P, ctypes.POINTER(Plan), P, P, I32, I32, P,
                                              P, P, SZ, P]),
            "qma_silu_and_mul": (I32, [P, P, I64, I32, P]),
            "qma_moe_combine": (I32, [P, P, P, I32, I32, I32, I32, P, P]),
            "qma_router_topk": (I32, [P, I32, I32, I32, P, P, P]),
            "qma_status_str": (ctypes.c_char_p, [I32]),
            "qma_last_error_detail": (ctypes.c_char_p, []),
            "qma_version": (ctypes.c_char_p, []),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _status_name(s: int) -> str:
    return lib().qma_status_str(s).decode()


def _check(status: int):
    if status != QMA_OK:
        raise QmaError(status, lib().qma_last_error_detail().decode())


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def qma_version() -> str:
    return lib().qma_version().decode()


def qma_layer_create(E: int, N: int, K: int, path: int = PATH_INDEXED,
                     desc: Optional[QuantDesc] = None, flags: int = 0) -> ctypes.c_void_p:
    out = ctypes.c_void_p()
    if flags:
        _check(lib().qma_layer_create_ex(ctypes.byref(desc or w4a16_desc()), E, N, K, path,
                                         flags, ctypes.byref(out)))
    else:
        _check(lib().qma_layer_create(ctypes.byref(desc or w4a16_desc()), E, N, K, path,
                                      ctypes.byref(out)))
    return out


def qma_layer_destroy(layer) -> None:
    lib().qma_layer_destroy(layer)


def qma_layer_info(layer) -> dict:
    v = [ctypes.c_int32() for _ in range(5)]
    _check(lib().qma_layer_info(layer, *[ctypes.byref(x) for x in v]))
    E, N, K, path, prof = (x.value for x in v)
    return {"E": E, "N": N, "K": K, "path": path, "profile": PROFILES.get(prof, prof)}


def qma_packed_weight_bytes(layer) -> int:
    return int(lib().qma_packed_weight_bytes(layer))


def qma_prepack(layer, qweight, scales, packed, stream=None) -> None:
    _check(lib().qma_prepack(layer, _ptr(qweight), _ptr(scales), _ptr(packed),
                             _stream(stream)))


def qma_plan_indexed(layer, T: int, topk: int, force_block_m: int = 0) -> Plan:
    p = Plan()
    _check(lib().qma_plan_indexed(layer, T, topk, force_block_m, ctypes.byref(p)))
    return p


def qma_plan_grouped(layer, m_rows_or_budget: int, expected_m: int = 0) -> Plan:
    p = Plan()
    _check(lib().qma_plan_grouped(layer, m_rows_or_budget, expected_m, ctypes.byref(p)))
    return p


def qma_workspace_bytes(plan: Plan) -> int:
    return int(lib().qma_workspace_bytes(ctypes.byref(plan)))


def qma_align_sizes(T: int, topk: int, E: int, block_m: int):
    a, b = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().qma_align_sizes(T, topk, E, block_m, ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def qma_moe_align(topk_ids, T, topk, E, block_m, sorted_ids, expert_ids,
                  num_tokens_padded, sorted_cap, stream=None) -> None:
    _check(lib().qma_moe_align(_ptr(topk_ids), T, topk, E, block_m, _ptr(sorted_ids),
                               _ptr(expert_ids), _ptr(num_tokens_padded), sorted_cap,
                               _stream(stream)))


def qma_validate_routing(topk_ids, T, topk, E, block_m, sorted_ids, expert_ids,
                         num_tokens_padded, sorted_cap, stream=None) -> None:
    _check(lib().qma_validate_routing(_ptr(topk_ids), T, topk, E, block_m,
                                      _ptr(sorted_ids), _ptr(expert_ids),
                                      _ptr(num_tokens_padded), sorted_cap, _stream(stream)))


def qma_validate_contiguous(m_indices, M, E, stream=None) -> None:
    _check(lib().qma_validate_contiguous(_ptr(m_indices), M, E, _stream(stream)))


def qma_indexed_gemm(layer, plan: Plan, a, a_rows, a_row_div, packed_w, sorted_ids,
                     expert_ids, num_tokens_padded, sorted_cap, num_slots, topk_weights,
                     c, ws=None, ws_bytes=0, stream=None) -> None:
    _check(lib().qma_indexed_gemm(layer, ctypes.byref(plan), _ptr(a), a_rows, a_row_div,
                                  _ptr(packed_w), _ptr(sorted_ids), _ptr(expert_ids),
                                  _ptr(num_tokens_padded), sorted_cap, num_slots,
                                  _ptr(topk_weights), _ptr(c), _ptr(ws), ws_bytes,
                                  _stream(stream)))


def qma_indexed_gemm_scratch(layer, plan: Plan, a, a_rows, a_row_div, packed_w, sorted_ids,
                             expert_ids, num_tokens_padded, sorted_cap, num_slots, topk_weights,
                             c, stream=None) -> None:
    _check(lib().qma_indexed_gemm_scratch(layer, ctypes.byref(plan), _ptr(a), a_rows,
                                          a_row_div, _ptr(packed_w), _ptr(sorted_ids),
                                          _ptr(expert_ids), _ptr(num_tokens_padded),
                                          sorted_cap, num_slots, _ptr(topk_weights), _ptr(c),
                                          _stream(stream)))


def qma_grouped_contiguous_gemm(layer, plan: Plan, a, m_indices, M, packed_w, c,
                                ws=None, ws_bytes=0, stream=None) -> None:
    _check(lib().qma_grouped_contiguous_gemm(layer, ctypes.byref(plan), _ptr(a),
                                             _ptr(m_indices), M, _ptr(packed_w), _ptr(c),
                                             _ptr(ws), ws_bytes, _stream(stream)))


def qma_grouped_masked_gemm(layer, plan: Plan, a, masked_m, Mb, expected_m, packed_w, c,
                            ws=None, ws_bytes=0, stream=None) -> None:
    _check(lib().qma_grouped_masked_gemm(layer, ctypes.byref(plan), _ptr(a), _ptr(masked_m),
                                         Mb, expected_m, _ptr(packed_w), _ptr(c), _ptr(ws),
                                         ws_bytes, _stream(stream)))


def qma_silu_and_mul(x, y, R, I, stream=None) -> None:
    _check(lib().qma_silu_and_mul(_ptr(x), _ptr(y), R, I, _stream(stream)))


def qma_router_topk(logits, T, E, topk, topk_ids, topk_weights=None, stream=None) -> None:
    _check(lib().qma_router_topk(_ptr(logits), T, E, topk, _ptr(topk_ids), _ptr(topk_weights),
                                 _stream(stream)))


def qma_moe_combine(c2, w, topk_ids, E, T, topk, N, out, stream=None) -> None:
    _check(lib().qma_moe_combine(_ptr(c2), _ptr(w), _ptr(topk_ids), E, T, topk, N, _ptr(out),
                                 _stream(stream)))
