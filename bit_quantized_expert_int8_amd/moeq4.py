"""ctypes binding of libmoeq4.so — one Python function per C entry point, same names, argument
marshalling only (every step of the decode path runs in the library's HIP kernels).

Pointers may be given as ints or as objects with ``data_ptr()`` (torch tensors); streams and events as
ints, ``torch.cuda.Stream``/``Event`` objects or None.  A non-OK status raises ``MoeError`` carrying the
library's message.  If the library is not built, importing this module raises ``ImportError``: there is
no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

# Load torch's HIP runtime first.  torch ships its own libamdhip64 (requested as "libamdhip64.so"), while
# this library asks for "libamdhip64.so.7"; if this library were loaded first, the process would map two
# HIP runtimes (and two HSA runtimes) once torch is imported.  With torch loaded first, the soname
# "libamdhip64.so.7" resolves to the runtime torch already mapped, so there is exactly one.
import torch  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoeq4.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_OUT_OF_RANGE, MOE_ERR_CACHE, MOE_ERR_HIP = range(6)
MOE_F32, MOE_BF16 = 0, 1
MOE_ACT_GELU_TANH, MOE_ACT_SILU = 0, 1
MOE_CACHE_HOST_ONLY = 1

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python -m bit_quantized_expert_int8_amd.build` "
                      "(or __graft_entry__.build())")
_lib = ctypes.CDLL(LIB_PATH)

_vp, _i32, _u32, _sz, _u64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_size_t, ctypes.c_uint64
_st = ctypes.c_int


class moe_q4_pool(ctypes.Structure):
    _fields_ = [("base_dev", _vp), ("record_bytes", _sz), ("n_records", _i32), ("d", _i32), ("F", _i32),
                ("sb_dtype", ctypes.c_int)]


class moe_stack_layer(ctypes.Structure):
    _fields_ = [("router_w_dev", _vp), ("router_scale_dev", _vp), ("gamma_dev", _vp), ("routed_base_dev", _vp),
                ("shared_base_dev", _vp), ("ids_dev", _vp), ("weights_dev", _vp), ("logits_dev", _vp),
                ("u_dev", _vp)]


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status}: {moe_last_error()}")


def _sig(name, restype, argtypes):
    f = getattr(_lib, name)
    f.restype = restype
    f.argtypes = argtypes
    return f


_c = {
    "moe_record_bytes": _sig("moe_record_bytes", _sz, [_i32, _i32, ctypes.c_int]),
    "moe_record_layout": _sig("moe_record_layout", _st, [_i32, _i32, ctypes.c_int, ctypes.POINTER(_sz)]),
    "q4_quantize": _sig("q4_quantize", _st, [_vp, _i32, _i32, ctypes.c_int, _vp, _vp, _vp]),
    "q4_pack_expert": _sig("q4_pack_expert", _st, [_vp, _vp, _i32, _i32, ctypes.c_int, _vp, _vp]),
    "q4_gemv": _sig("q4_gemv", _st, [_vp, ctypes.c_int, _i32, _vp, _vp, ctypes.c_int, _i32, _i32, _vp, _vp]),
    "moe_rmsnorm": _sig("moe_rmsnorm", _st, [_vp, ctypes.c_int, _vp, ctypes.c_float, _i32, _i32, _vp, ctypes.c_int, _vp]),
    "moe_router_workspace_bytes": _sig("moe_router_workspace_bytes", _sz, [_i32, _i32]),
    "moe_router_topk": _sig("moe_router_topk", _st, [_vp, ctypes.c_int, _i32, _i32, _vp, _vp, _i32, _i32, _vp, _vp, _vp,
                                                     _vp, _vp, _sz, _vp]),
    "moe_norm_router_topk": _sig("moe_norm_router_topk", _st, [_vp, ctypes.c_int, _vp, ctypes.c_float, _i32, _i32, _vp, _vp,
                                                               _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_group_pairs_max_groups": _sig("moe_group_pairs_max_groups", _i32, [_i32, _i32, _i32]),
    "moe_group_pairs": _sig("moe_group_pairs", _st, [_vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp]),
    "q4_expert_gemv_workspace_bytes": _sig("q4_expert_gemv_workspace_bytes", _sz,
                                           [ctypes.POINTER(moe_q4_pool), _i32, ctypes.POINTER(moe_q4_pool), _i32]),
    "q4_expert_gemv": _sig("q4_expert_gemv", _st, [ctypes.POINTER(moe_q4_pool), _vp, _i32, ctypes.POINTER(moe_q4_pool), _vp,
                                                   ctypes.c_int, _i32, ctypes.c_int, _vp, _vp, _vp, _sz, _vp]),
    "q4_expert_gate_up": _sig("q4_expert_gate_up", _st, [ctypes.POINTER(moe_q4_pool), _vp, _i32, ctypes.POINTER(moe_q4_pool),
                                                         _vp, ctypes.c_int, _i32, ctypes.c_int, _vp, _sz, _vp]),
    "q4_expert_down": _sig("q4_expert_down", _st, [ctypes.POINTER(moe_q4_pool), _vp, _i32, ctypes.POINTER(moe_q4_pool), _i32,
                                                   _vp, _vp, _vp, _sz, _vp]),
    "q4_expert_gemv_combine_workspace_bytes": _sig("q4_expert_gemv_combine_workspace_bytes", _sz,
                                                   [ctypes.POINTER(moe_q4_pool), _i32, ctypes.POINTER(moe_q4_pool), _i32]),
    "q4_expert_gemv_combine": _sig("q4_expert_gemv_combine", _st,
                                   [ctypes.POINTER(moe_q4_pool), _vp, _i32, ctypes.POINTER(moe_q4_pool), _vp, ctypes.c_int,
                                    _i32, ctypes.c_int, _vp, _vp, ctypes.c_int, _vp, ctypes.c_int, _vp, _sz, _vp]),
    "moe_decode_layer_workspace_bytes": _sig("moe_decode_layer_workspace_bytes", _sz, [_i32, _i32, _i32, _i32, _i32]),
    "moe_decode_layer_sync_bytes": _sig("moe_decode_layer_sync_bytes", _sz, [_i32, _i32]),
    "moe_decode_layer": _sig("moe_decode_layer", _st,
                             [_vp, ctypes.c_int, _vp, ctypes.c_float, _i32, _vp, _vp, _i32, _i32, _vp,
                              ctypes.POINTER(moe_q4_pool), _vp, ctypes.POINTER(moe_q4_pool), ctypes.c_int, _vp, _vp,
                              _vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_decode_layer_part": _sig("moe_decode_layer_part", _st,
                                  [_i32, _vp, ctypes.c_int, _vp, ctypes.c_float, _i32, _vp, _vp, _i32, _i32, _vp,
                                   ctypes.POINTER(moe_q4_pool), _vp, ctypes.POINTER(moe_q4_pool), ctypes.c_int, _vp, _vp,
                                   _vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_decode_layer_noalloc": _sig("moe_decode_layer_noalloc", _st,
                                     [_vp, ctypes.c_int, _vp, ctypes.c_float, _i32, _vp, _vp, _i32, _i32, _vp,
                                      ctypes.POINTER(moe_q4_pool), _vp, ctypes.POINTER(moe_q4_pool), ctypes.c_int, _vp,
                                      _vp, _vp, _vp, _vp, _vp, _vp]),
    "moe_decode_stack_workspace_bytes": _sig("moe_decode_stack_workspace_bytes", _sz,
                                             [_i32, _i32, _i32, _i32, _i32, _i32]),
    "moe_decode_stack": _sig("moe_decode_stack", _st,
                             [ctypes.POINTER(moe_stack_layer), _i32, _vp, ctypes.c_int, ctypes.c_float, _i32, _i32, _i32,
                              ctypes.POINTER(moe_q4_pool), ctypes.POINTER(moe_q4_pool), ctypes.c_int, _vp, _vp, _sz,
                              _vp]),
    "moe_combine": _sig("moe_combine", _st, [_vp, _vp, _vp, _vp, ctypes.c_int, _i32, _i32, _i32, _vp, ctypes.c_int, _vp]),
    "moe_expert_cache_create": _sig("moe_expert_cache_create", _st, [_i32, _i32, _i32, _sz, ctypes.POINTER(_vp),
                                                                     ctypes.POINTER(_vp), _u32, ctypes.POINTER(_vp)]),
    "moe_expert_cache_destroy": _sig("moe_expert_cache_destroy", None, [_vp]),
    "expert_cache_stage": _sig("expert_cache_stage", _st, [_vp, _i32, ctypes.POINTER(_i32), _i32, _vp, _vp, _vp, _vp]),
    "moe_expert_cache_stats": _sig("moe_expert_cache_stats", _st, [_vp, _i32, ctypes.POINTER(_u64), ctypes.POINTER(_u64),
                                                                   ctypes.POINTER(_u64)]),
    "moe_expert_cache_slots": _sig("moe_expert_cache_slots", _st, [_vp, _i32, ctypes.POINTER(_i32)]),
    "moe_expert_cache_inject_copy_failure": _sig("moe_expert_cache_inject_copy_failure", _st, [_vp, _i32]),
    "moe_hbm_read_probe": _sig("moe_hbm_read_probe", _st, [_vp, _sz, _vp, _vp]),
    "moe_last_error": _sig("moe_last_error", ctypes.c_char_p, []),
    "moe_version": _sig("moe_version", ctypes.c_char_p, []),
}


def _p(x) -> int | None:
    """Pointer value of an int, a tensor (data_ptr) or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    raise TypeError(f"cannot take a pointer from {type(x)!r}")


def _s(x) -> int | None:
    """Raw handle of a stream/event (int, torch.cuda.Stream/Event) or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "cuda_stream"):
        return x.cuda_stream
    if hasattr(x, "cuda_event"):
        return x.cuda_event
    raise TypeError(f"cannot take a stream/event handle from {type(x)!r}")


def _check(status: int, where: str) -> None:
    if status != MOE_OK:
        raise MoeError(status, where)


def pool(base, record_bytes: int, n_records: int, d: int, F: int, sb_dtype: int) -> moe_q4_pool:
    return moe_q4_pool(_p(base), record_bytes, n_records, d, F, sb_dtype)


def moe_last_error() -> str:
    return _c["moe_last_error"]().decode()


def moe_version() -> str:
    return _c["moe_version"]().decode()


def moe_record_bytes(d: int, F: int, sb_dtype: int) -> int:
    return _c["moe_record_bytes"](d, F, sb_dtype)


def moe_record_layout(d: int, F: int, sb_dtype: int) -> tuple:
    off = (_sz * 4)()
    _check(_c["moe_record_layout"](d, F, sb_dtype, off), "moe_record_layout")
    return tuple(off)


def q4_quantize(w, N, K, sb_dtype, codes, sb, stream=None) -> None:
    _check(_c["q4_quantize"](_p(w), N, K, sb_dtype, _p(codes), _p(sb), _s(stream)), "q4_quantize")


def q4_pack_expert(w_gate_up, w_down, d, F, sb_dtype, record, stream=None) -> None:
    _check(_c["q4_pack_expert"](_p(w_gate_up), _p(w_down), d, F, sb_dtype, _p(record), _s(stream)), "q4_pack_expert")


def q4_gemv(x, x_dtype, T, codes, sb, sb_dtype, N, K, y, stream=None) -> None:
    _check(_c["q4_gemv"](_p(x), x_dtype, T, _p(codes), _p(sb), sb_dtype, N, K, _p(y), _s(stream)), "q4_gemv")


def moe_rmsnorm(x, x_dtype, gamma, eps, T, d, out, out_dtype, stream=None) -> None:
    _check(_c["moe_rmsnorm"](_p(x), x_dtype, _p(gamma), eps, T, d, _p(out), out_dtype, _s(stream)), "moe_rmsnorm")


def moe_router_workspace_bytes(T: int, E: int) -> int:
    return _c["moe_router_workspace_bytes"](T, E)


def moe_router_topk(x, x_dtype, T, d, w, row_scale, E, k, forced_ids, ids, weights, logits, workspace, workspace_bytes,
                    stream=None) -> None:
    _check(_c["moe_router_topk"](_p(x), x_dtype, T, d, _p(w), _p(row_scale), E, k, _p(forced_ids), _p(ids), _p(weights),
                                 _p(logits), _p(workspace), workspace_bytes, _s(stream)), "moe_router_topk")


def moe_norm_router_topk(x, x_dtype, gamma, eps, T, d, w, row_scale, E, k, forced_ids, ids, weights, logits, u,
                         workspace, workspace_bytes, stream=None) -> None:
    _check(_c["moe_norm_router_topk"](_p(x), x_dtype, _p(gamma), eps, T, d, _p(w), _p(row_scale), E, k, _p(forced_ids),
                                      _p(ids), _p(weights), _p(logits), _p(u), _p(workspace), workspace_bytes,
                                      _s(stream)), "moe_norm_router_topk")


def moe_group_pairs_max_groups(T: int, k: int, n_valid: int) -> int:
    return _c["moe_group_pairs_max_groups"](T, k, n_valid)


def moe_group_pairs(ids, T, k, n_valid, n_groups, groups, perm, stream=None) -> None:
    _check(_c["moe_group_pairs"](_p(ids), T, k, n_valid, _p(n_groups), _p(groups), _p(perm), _s(stream)),
           "moe_group_pairs")


def _pp(p):
    return ctypes.byref(p) if p is not None else None


def q4_expert_gemv_workspace_bytes(routed, k, shared, T) -> int:
    return _c["q4_expert_gemv_workspace_bytes"](_pp(routed), k, _pp(shared), T)


def q4_expert_gemv(routed, ids, k, shared, x, x_dtype, T, act, y_routed, y_shared, workspace, workspace_bytes,
                   stream=None) -> None:
    _check(_c["q4_expert_gemv"](_pp(routed), _p(ids), k, _pp(shared), _p(x), x_dtype, T, act, _p(y_routed), _p(y_shared),
                                _p(workspace), workspace_bytes, _s(stream)), "q4_expert_gemv")


def q4_expert_gate_up(routed, ids, k, shared, x, x_dtype, T, act, workspace, workspace_bytes, stream=None) -> None:
    _check(_c["q4_expert_gate_up"](_pp(routed), _p(ids), k, _pp(shared), _p(x), x_dtype, T, act, _p(workspace),
                                   workspace_bytes, _s(stream)), "q4_expert_gate_up")


def q4_expert_down(routed, ids, k, shared, T, y_routed, y_shared, workspace, workspace_bytes, stream=None) -> None:
    _check(_c["q4_expert_down"](_pp(routed), _p(ids), k, _pp(shared), T, _p(y_routed), _p(y_shared), _p(workspace),
                                workspace_bytes, _s(stream)), "q4_expert_down")


def q4_expert_gemv_combine_workspace_bytes(routed, k, shared, T) -> int:
    return _c["q4_expert_gemv_combine_workspace_bytes"](_pp(routed), k, _pp(shared), T)


def q4_expert_gemv_combine(routed, ids, k, shared, x, x_dtype, T, act, weights, residual, residual_dtype, out, out_dtype,
                           workspace, workspace_bytes, stream=None) -> None:
    _check(_c["q4_expert_gemv_combine"](_pp(routed), _p(ids), k, _pp(shared), _p(x), x_dtype, T, act, _p(weights),
                                        _p(residual), residual_dtype, _p(out), out_dtype, _p(workspace), workspace_bytes,
                                        _s(stream)), "q4_expert_gemv_combine")


def moe_decode_layer_workspace_bytes(d, E, k, F, S) -> int:
    return _c["moe_decode_layer_workspace_bytes"](d, E, k, F, S)


def moe_decode_layer_sync_bytes(d, k) -> int:
    return _c["moe_decode_layer_sync_bytes"](d, k)


def moe_decode_layer(x, x_dtype, gamma, eps, residual, router_w, router_scale, E, k, forced_ids, routed, gemv_ids,
                     shared, act, ids, weights, logits, out, workspace, workspace_bytes, stream=None, u=None) -> None:
    _check(_c["moe_decode_layer"](_p(x), x_dtype, _p(gamma), eps, int(residual), _p(router_w), _p(router_scale), E, k,
                                  _p(forced_ids), _pp(routed), _p(gemv_ids), _pp(shared), act, _p(ids), _p(weights),
                                  _p(logits), _p(u), _p(out), _p(workspace), workspace_bytes, _s(stream)),
           "moe_decode_layer")


def moe_decode_layer_part(part, x, x_dtype, gamma, eps, residual, router_w, router_scale, E, k, forced_ids, routed,
                          gemv_ids, shared, act, ids, weights, logits, u, out, workspace, workspace_bytes,
                          stream=None) -> None:
    _check(_c["moe_decode_layer_part"](part, _p(x), x_dtype, _p(gamma), eps, int(residual), _p(router_w),
                                       _p(router_scale), E, k, _p(forced_ids), _pp(routed), _p(gemv_ids), _pp(shared),
                                       act, _p(ids), _p(weights), _p(logits), _p(u), _p(out), _p(workspace),
                                       workspace_bytes, _s(stream)), "moe_decode_layer_part")


MOE_DECODE_LAYER_NOALLOC_MAX_BYTES = 1 << 20


def moe_decode_layer_noalloc(x, x_dtype, gamma, eps, residual, router_w, router_scale, E, k, forced_ids, routed,
                             gemv_ids, shared, act, ids, weights, logits, u, out, status, stream=None) -> None:
    _check(_c["moe_decode_layer_noalloc"](_p(x), x_dtype, _p(gamma), eps, int(residual), _p(router_w), _p(router_scale),
                                          E, k, _p(forced_ids), _pp(routed), _p(gemv_ids), _pp(shared), act, _p(ids),
                                          _p(weights), _p(logits), _p(u), _p(out), _p(status), _s(stream)),
           "moe_decode_layer_noalloc")


def moe_decode_stack_workspace_bytes(n_layers, d, E, k, F, S) -> int:
    return _c["moe_decode_stack_workspace_bytes"](n_layers, d, E, k, F, S)


def stack_layers(descs) -> ctypes.Array:
    """ctypes array of moe_stack_layer from dicts with the field names (tensors or ints or None)."""
    arr = (moe_stack_layer * len(descs))()
    for i, d in enumerate(descs):
        for name, _ in moe_stack_layer._fields_:
            setattr(arr[i], name, _p(d.get(name)))
    return arr


def moe_decode_stack(layers, n_layers, x, x_dtype, eps, residual, E, k, routed, shared, act, out, workspace,
                     workspace_bytes, stream=None) -> None:
    """`layers`: a ctypes array from stack_layers()."""
    _check(_c["moe_decode_stack"](layers, n_layers, _p(x), x_dtype, eps, int(residual), E, k, _pp(routed), _pp(shared),
                                  act, _p(out), _p(workspace), workspace_bytes, _s(stream)), "moe_decode_stack")


def moe_combine(y_routed, weights, y_shared, residual, residual_dtype, T, k, d, out, out_dtype, stream=None) -> None:
    _check(_c["moe_combine"](_p(y_routed), _p(weights), _p(y_shared), _p(residual), residual_dtype, T, k, d, _p(out),
                             out_dtype, _s(stream)), "moe_combine")


def moe_expert_cache_create(n_layers, n_experts, n_slots, record_bytes, host_pools, slot_pools, flags=0) -> int:
    hp = (_vp * n_layers)(*[_p(x) for x in host_pools])
    sp = (_vp * n_layers)(*[_p(x) for x in slot_pools])
    out = _vp()
    _check(_c["moe_expert_cache_create"](n_layers, n_experts, n_slots, record_bytes, hp, sp, flags, ctypes.byref(out)),
           "moe_expert_cache_create")
    return out.value


def moe_expert_cache_destroy(cache: int) -> None:
    _c["moe_expert_cache_destroy"](cache)


def expert_cache_stage(cache, layer, ids_host, slot_ids, copy_stream=None, wait_event=None, ready_event=None) -> None:
    ids = (_i32 * len(ids_host))(*[int(v) for v in ids_host])
    _check(_c["expert_cache_stage"](cache, layer, ids, len(ids_host), _p(slot_ids), _s(copy_stream), _s(wait_event),
                                    _s(ready_event)), "expert_cache_stage")


def moe_expert_cache_stats(cache, layer=-1) -> tuple:
    h, m, b = _u64(), _u64(), _u64()
    _check(_c["moe_expert_cache_stats"](cache, layer, ctypes.byref(h), ctypes.byref(m), ctypes.byref(b)),
           "moe_expert_cache_stats")
    return h.value, m.value, b.value


def moe_expert_cache_slots(cache, layer, n_slots) -> list:
    out = (_i32 * n_slots)()
    _check(_c["moe_expert_cache_slots"](cache, layer, out), "moe_expert_cache_slots")
    return list(out)


def moe_expert_cache_inject_copy_failure(cache, after_n_copies) -> None:
    _check(_c["moe_expert_cache_inject_copy_failure"](cache, after_n_copies), "moe_expert_cache_inject_copy_failure")


def moe_hbm_read_probe(buf, nbytes, sink, stream=None) -> None:
    _check(_c["moe_hbm_read_probe"](_p(buf), nbytes, _p(sink), _s(stream)), "moe_hbm_read_probe")


def raw(name: str):
    """The raw ctypes function of a C entry point (for tests of status codes)."""
    return _c[name]


EXPORTED = tuple(_c)
