"""Python binding of liboccult, the collaboration-aware MoE layer step
(Occult) on one MI355X.

Each function has the name of its C entry point in include/occ.h and only
marshals arguments: tensors become device pointers, the current HIP stream is
passed along, and a non-zero status raises OccError.  PyTorch provides device
memory and streams; every step of the layer runs in the library's HIP kernels.
There is no fallback: importing this package fails if liboccult.so has not
been built.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboccult.so")

OCC_OK, OCC_EINVAL, OCC_EUNSUP, OCC_ENOSPC, OCC_EHIP = 0, -1, -2, -3, -4
OCC_F32, OCC_BF16 = 0, 1
DTYPE_CODE = {"f32": OCC_F32, "bf16": OCC_BF16}


class OccError(RuntimeError):
    def __init__(self, code: int, where: str, text: str):
        super().__init__(f"{where} failed with status {code}: {text}")
        self.code = code


class occ_layer_desc(C.Structure):
    _fields_ = [("T", C.c_int32), ("d", C.c_int32), ("E", C.c_int32), ("k", C.c_int32),
                ("D", C.c_int32), ("I", C.c_int32), ("n_shared", C.c_int32),
                ("I_shared", C.c_int32), ("dtype", C.c_int32), ("renorm", C.c_int32)]


class occ_brim(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("brim0", "brim1", "sfd_offset", "slot_offset",
                                          "sfd_token", "epd_token", "epd_sfd", "epd_w", "S")]


def _load(path: str = LIB_PATH):
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python expert_top_router_amd/build.py`")
    lib = C.CDLL(path)
    P, I32, SZ = C.c_void_p, C.c_int32, C.c_size_t
    DP, BP = C.POINTER(occ_layer_desc), C.POINTER(occ_brim)
    sig = {
        "occ_workspace_bytes": (SZ, [DP]),
        "occ_ffn_workspace_bytes": (SZ, [DP]),
        "occ_route_topk": (I32, [DP, P, P, P, P, P, P]),
        "occ_route_workspace_bytes": (SZ, [DP]),
        "occ_route_topk_ws": (I32, [DP, P, P, P, P, P, SZ, P]),
        "occ_build_brim": (I32, [DP, P, P, P, BP, P, SZ, P]),
        "occ_build_brim_pruned": (I32, [DP, P, P, P, I32, I32, BP, P, SZ, P]),
        "occ_build_brim_noalloc": (I32, [DP, P, P, P, BP, P]),
        "occ_dispatch": (I32, [DP, P, BP, P, P, P]),
        "occ_expert_ffn": (I32, [DP, P, BP, P, P, P, P, SZ, P, P, P, P, P, P]),
        "occ_expert_up": (I32, [DP, P, BP, P, P, P, SZ, P, P, P]),
        "occ_expert_down": (I32, [DP, BP, P, P, P, SZ, P, P, P, P]),
        "occ_combine": (I32, [DP, P, BP, P, P, P, P]),
        "occ_dispatch_direct": (I32, [DP, P, BP, P, P]),
        "occ_combine_direct": (I32, [DP, P, BP, P, P, P]),
        "occ_coactivation": (I32, [DP, P, P, I32, P]),
        "occ_backward_workspace_bytes": (SZ, [DP]),
        "occ_grad_combine": (I32, [DP, P, BP, P, P, P, P, P]),
        "occ_expert_backward": (I32, [DP, P, BP, P, P, P, P, SZ, P, P, SZ, P, P, P, P]),
        "occ_expert_ffn_keep": (I32, [DP, P, BP, P, P, P, P, SZ, P, P, P]),
        "occ_expert_backward_kept": (I32, [DP, P, BP, P, P, P, P, SZ, P, P, P, SZ, P, P, P, P]),
        "occ_router_backward": (I32, [DP, P, P, P, P, P, P, BP, P, P, P, P, P, SZ, P]),
        "occ_grad_dispatch": (I32, [DP, P, BP, P, P, P, P, P]),
        "occ_shared_backward": (I32, [DP, P, P, P, P, SZ, P, P, SZ, P, P, P, P]),
        "occ_cross_coactivation": (I32, [I32, I32, I32, P, I32, I32, P, P, I32, P]),
        "occ_home_device": (I32, [I32, I32, I32, P, I32, I32, P, P, P, P]),
        "occ_local_hits": (I32, [I32, I32, I32, P, I32, P, P, P, I32, P]),
        "occ_place_greedy": (I32, [I32, I32, P, P]),
        "occ_last_error": (C.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib = _load()

# Every symbol the C header declares (checked by the tests).
EXPORTED = ("occ_workspace_bytes", "occ_ffn_workspace_bytes", "occ_route_topk",
            "occ_route_workspace_bytes", "occ_route_topk_ws", "occ_build_brim",
            "occ_build_brim_pruned", "occ_build_brim_noalloc",
            "occ_dispatch", "occ_expert_ffn", "occ_expert_up", "occ_expert_down", "occ_combine",
            "occ_dispatch_direct", "occ_combine_direct", "occ_backward_workspace_bytes",
            "occ_grad_combine", "occ_expert_backward", "occ_router_backward",
            "occ_grad_dispatch", "occ_shared_backward", "occ_expert_ffn_keep", "occ_expert_backward_kept",
            "occ_coactivation",
            "occ_cross_coactivation", "occ_home_device", "occ_local_hits", "occ_place_greedy",
            "occ_last_error")


def lib():
    return _lib


def _ptr(t) -> Optional[int]:
    """Device (or host) address of a tensor / numpy array / int, None for None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if hasattr(t, "data_ptr"):
        return t.data_ptr()
    if hasattr(t, "ctypes"):
        return t.ctypes.data
    raise TypeError(f"cannot take the address of {type(t)}")


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int, where: str) -> None:
    if rc != OCC_OK:
        raise OccError(rc, where, _lib.occ_last_error().decode())


def last_error() -> str:
    return _lib.occ_last_error().decode()


def make_desc(T, d, E, k, D, I, n_shared=0, I_shared=0, dtype="bf16", renorm=0) -> occ_layer_desc:
    return occ_layer_desc(T, d, E, k, D, I, n_shared, I_shared,
                          DTYPE_CODE.get(dtype, dtype), renorm)


def desc_of(cfg) -> occ_layer_desc:
    """Descriptor of a layer configuration object (T, d, E, k, D, I, ...)."""
    return make_desc(cfg.T, cfg.d, cfg.E, cfg.k, cfg.D, cfg.I, cfg.n_shared, cfg.I_shared,
                     cfg.dtype, cfg.renorm)


def make_brim(**arrays) -> occ_brim:
    return occ_brim(*[_ptr(arrays.get(n)) for n, _ in occ_brim._fields_])


# ---- the entry points (same names as the C ABI) ---------------------------
def occ_workspace_bytes(desc: occ_layer_desc) -> int:
    return _lib.occ_workspace_bytes(C.byref(desc))


def occ_ffn_workspace_bytes(desc: occ_layer_desc) -> int:
    return _lib.occ_ffn_workspace_bytes(C.byref(desc))


def occ_route_topk(desc, x, w_router, topk_idx, topk_w, logits=None, stream=None):
    _check(_lib.occ_route_topk(C.byref(desc), _ptr(x), _ptr(w_router), _ptr(topk_idx),
                               _ptr(topk_w), _ptr(logits), _stream(stream)), "occ_route_topk")


def occ_route_workspace_bytes(desc: occ_layer_desc) -> int:
    return int(_lib.occ_route_workspace_bytes(C.byref(desc)))


def occ_route_topk_ws(desc, x, w_router, topk_idx, topk_w, ws, ws_bytes, stream=None):
    _check(_lib.occ_route_topk_ws(C.byref(desc), _ptr(x), _ptr(w_router), _ptr(topk_idx),
                                  _ptr(topk_w), _ptr(ws), int(ws_bytes), _stream(stream)),
           "occ_route_topk_ws")


def occ_build_brim(desc, topk_idx, topk_w, slot_expert_host, brim: occ_brim, ws, ws_bytes,
                   stream=None):
    import numpy as np
    se = np.ascontiguousarray(slot_expert_host, dtype=np.int32)
    _check(_lib.occ_build_brim(C.byref(desc), _ptr(topk_idx), _ptr(topk_w), se.ctypes.data,
                               C.byref(brim), _ptr(ws), ws_bytes, _stream(stream)),
           "occ_build_brim")


def occ_build_brim_noalloc(desc, topk_idx, topk_w, slot_expert_host, brim: occ_brim,
                           stream=None):
    import numpy as np
    se = np.ascontiguousarray(slot_expert_host, dtype=np.int32)
    _check(_lib.occ_build_brim_noalloc(C.byref(desc), _ptr(topk_idx), _ptr(topk_w),
                                       se.ctypes.data, C.byref(brim), _stream(stream)),
           "occ_build_brim_noalloc")


def occ_build_brim_pruned(desc, topk_idx, topk_w, slot_expert_host, budget, rescale,
                          brim: occ_brim, ws, ws_bytes, stream=None):
    import numpy as np
    se = np.ascontiguousarray(slot_expert_host, dtype=np.int32)
    _check(_lib.occ_build_brim_pruned(C.byref(desc), _ptr(topk_idx), _ptr(topk_w),
                                      se.ctypes.data, int(budget), int(rescale), C.byref(brim),
                                      _ptr(ws), ws_bytes, _stream(stream)),
           "occ_build_brim_pruned")


def occ_dispatch(desc, x, brim: occ_brim, sfd, epd, stream=None):
    _check(_lib.occ_dispatch(C.byref(desc), _ptr(x), C.byref(brim), _ptr(sfd), _ptr(epd),
                             _stream(stream)), "occ_dispatch")


def occ_expert_ffn(desc, epd, brim: occ_brim, slot_expert_host, w_gate_up, w_down, h_ws,
                   h_ws_bytes, out_epd, x=None, w_gate_up_sh=None, w_down_sh=None,
                   shared_out=None, stream=None):
    import numpy as np
    se = np.ascontiguousarray(slot_expert_host, dtype=np.int32)
    _check(_lib.occ_expert_ffn(C.byref(desc), _ptr(epd), C.byref(brim), se.ctypes.data,
                               _ptr(w_gate_up), _ptr(w_down), _ptr(h_ws), h_ws_bytes,
                               _ptr(out_epd), _ptr(x), _ptr(w_gate_up_sh), _ptr(w_down_sh),
                               _ptr(shared_out), _stream(stream)), "occ_expert_ffn")


def occ_expert_up(desc, epd, brim: occ_brim, slot_expert_host, w_gate_up, h_ws, h_ws_bytes,
                  x=None, w_gate_up_sh=None, stream=None):
    import numpy as np
    se = np.ascontiguousarray(slot_expert_host, dtype=np.int32)
    _check(_lib.occ_expert_up(C.byref(desc), _ptr(epd), C.byref(brim), se.ctypes.data,
                              _ptr(w_gate_up), _ptr(h_ws), h_ws_bytes, _ptr(x),
                              _ptr(w_gate_up_sh), _stream(stream)), "occ_expert_up")


def occ_expert_down(desc, brim: occ_brim, slot_expert_host, w_down, h_ws, h_ws_bytes, out_epd,
                    w_down_sh=None, shared_out=None, stream=None):
    import numpy as np
    se = np.ascontiguousarray(slot_expert_host, dtype=np.int32)
    _check(_lib.occ_expert_down(C.byref(desc), C.byref(brim), se.ctypes.data, _ptr(w_down),
                                _ptr(h_ws), h_ws_bytes, _ptr(out_epd), _ptr(w_down_sh),
                                _ptr(shared_out), _stream(stream)), "occ_expert_down")


def occ_combine(desc, out_epd, brim: occ_brim, shared_out, out_sfd, y, stream=None):
    _check(_lib.occ_combine(C.byref(desc), _ptr(out_epd), C.byref(brim), _ptr(shared_out),
                            _ptr(out_sfd), _ptr(y), _stream(stream)), "occ_combine")


def occ_dispatch_direct(desc, x, brim: occ_brim, epd, stream=None):
    _check(_lib.occ_dispatch_direct(C.byref(desc), _ptr(x), C.byref(brim), _ptr(epd),
                                    _stream(stream)), "occ_dispatch_direct")


def occ_combine_direct(desc, out_epd, brim: occ_brim, shared_out, y, stream=None):
    _check(_lib.occ_combine_direct(C.byref(desc), _ptr(out_epd), C.byref(brim), _ptr(shared_out),
                                   _ptr(y), _stream(stream)), "occ_combine_direct")


def occ_coactivation(desc, topk_idx, counts, accumulate=0, stream=None):
    _check(_lib.occ_coactivation(C.byref(desc), _ptr(topk_idx), _ptr(counts), int(accumulate),
                                 _stream(stream)), "occ_coactivation")


def occ_backward_workspace_bytes(desc: occ_layer_desc) -> int:
    return _lib.occ_backward_workspace_bytes(C.byref(desc))


def occ_grad_combine(desc, dy, brim: occ_brim, out_epd, d_out_sfd, d_out_epd, dw_epd,
                     stream=None):
    _check(_lib.occ_grad_combine(C.byref(desc), _ptr(dy), C.byref(brim), _ptr(out_epd),
                                 _ptr(d_out_sfd), _ptr(d_out_epd), _ptr(dw_epd), _stream(stream)),
           "occ_grad_combine")


def occ_expert_backward(desc, epd, brim: occ_brim, slot_expert_host, w_gate_up, w_down, h_ws,
                        h_ws_bytes, d_out_epd, bwd_ws, bwd_ws_bytes, d_epd, dw_gate_up, dw_down,
                        stream=None):
    import numpy as np
    se = np.ascontiguousarray(slot_expert_host, dtype=np.int32)
    _check(_lib.occ_expert_backward(C.byref(desc), _ptr(epd), C.byref(brim), se.ctypes.data,
                                    _ptr(w_gate_up), _ptr(w_down), _ptr(h_ws), h_ws_bytes,
                                    _ptr(d_out_epd), _ptr(bwd_ws), bwd_ws_bytes, _ptr(d_epd),
                                    _ptr(dw_gate_up), _ptr(dw_down), _stream(stream)),
           "occ_expert_backward")


def occ_expert_ffn_keep(desc, epd, brim: occ_brim, slot_expert_host, w_gate_up, w_down, h_ws,
                        h_ws_bytes, gu, out_epd, stream=None):
    import numpy as np
    se = np.ascontiguousarray(slot_expert_host, dtype=np.int32)
    _check(_lib.occ_expert_ffn_keep(C.byref(desc), _ptr(epd), C.byref(brim), se.ctypes.data,
                                    _ptr(w_gate_up), _ptr(w_down), _ptr(h_ws), h_ws_bytes,
                                    _ptr(gu), _ptr(out_epd), _stream(stream)),
           "occ_expert_ffn_keep")


def occ_expert_backward_kept(desc, epd, brim: occ_brim, slot_expert_host, w_gate_up, w_down,
                             h_ws, h_ws_bytes, gu, d_out_epd, bwd_ws, bwd_ws_bytes, d_epd,
                             dw_gate_up, dw_down, stream=None):
    import numpy as np
    se = np.ascontiguousarray(slot_expert_host, dtype=np.int32)
    _check(_lib.occ_expert_backward_kept(C.byref(desc), _ptr(epd), C.byref(brim),
                                         se.ctypes.data, _ptr(w_gate_up), _ptr(w_down),
                                         _ptr(h_ws), h_ws_bytes, _ptr(gu), _ptr(d_out_epd),
                                         _ptr(bwd_ws), bwd_ws_bytes, _ptr(d_epd),
                                         _ptr(dw_gate_up), _ptr(dw_down), _stream(stream)),
           "occ_expert_backward_kept")


def occ_router_backward(desc, x, w_router, logits, topk_idx, topk_w, slot_expert_host,
                        brim: occ_brim, dw_epd, dlogits, dx_router, dw_router, bwd_ws,
                        bwd_ws_bytes, stream=None):
    import numpy as np
    se = np.ascontiguousarray(slot_expert_host, dtype=np.int32)
    _check(_lib.occ_router_backward(C.byref(desc), _ptr(x), _ptr(w_router), _ptr(logits),
                                    _ptr(topk_idx), _ptr(topk_w), se.ctypes.data, C.byref(brim),
                                    _ptr(dw_epd), _ptr(dlogits), _ptr(dx_router),
                                    _ptr(dw_router), _ptr(bwd_ws), bwd_ws_bytes,
                                    _stream(stream)), "occ_router_backward")


def occ_grad_dispatch(desc, d_epd, brim: occ_brim, dx_router, d_sfd, dx, stream=None,
                      dx_shared=None):
    _check(_lib.occ_grad_dispatch(C.byref(desc), _ptr(d_epd), C.byref(brim), _ptr(dx_router),
                                  _ptr(dx_shared), _ptr(d_sfd), _ptr(dx), _stream(stream)),
           "occ_grad_dispatch")


def occ_shared_backward(desc, x, w_gate_up_sh, w_down_sh, h_ws, h_ws_bytes, dy, bwd_ws,
                        bwd_ws_bytes, dx_shared, dw_gate_up_sh, dw_down_sh, stream=None):
    _check(_lib.occ_shared_backward(C.byref(desc), _ptr(x), _ptr(w_gate_up_sh), _ptr(w_down_sh),
                                    _ptr(h_ws), h_ws_bytes, _ptr(dy), _ptr(bwd_ws), bwd_ws_bytes,
                                    _ptr(dx_shared), _ptr(dw_gate_up_sh), _ptr(dw_down_sh),
                                    _stream(stream)), "occ_shared_backward")


def occ_cross_coactivation(T, k1, E1, idx1, k2, E2, idx2, counts, accumulate=0, stream=None):
    _check(_lib.occ_cross_coactivation(T, k1, E1, _ptr(idx1), k2, E2, _ptr(idx2), _ptr(counts),
                                       int(accumulate), _stream(stream)),
           "occ_cross_coactivation")


def occ_home_device(T, k1, E1, idx1, E2, D, slot_expert2_host, affinity, home, stream=None):
    import numpy as np
    se = np.ascontiguousarray(slot_expert2_host, dtype=np.int32)
    _check(_lib.occ_home_device(T, k1, E1, _ptr(idx1), E2, D, se.ctypes.data, _ptr(affinity),
                                _ptr(home), _stream(stream)), "occ_home_device")


def occ_local_hits(T, k2, E2, idx2, D, slot_expert2_host, home, hits, accumulate=0,
                   stream=None):
    import numpy as np
    se = np.ascontiguousarray(slot_expert2_host, dtype=np.int32)
    _check(_lib.occ_local_hits(T, k2, E2, _ptr(idx2), D, se.ctypes.data, _ptr(home), _ptr(hits),
                               int(accumulate), _stream(stream)), "occ_local_hits")


def occ_place_greedy(E: int, D: int, counts_host):
    """Host greedy placement: returns slot_expert (numpy int32 [E])."""
    import numpy as np
    c = np.ascontiguousarray(counts_host, dtype=np.int32)
    out = np.empty(E, dtype=np.int32)
    _check(_lib.occ_place_greedy(E, D, c.ctypes.data, out.ctypes.data), "occ_place_greedy")
    return out


from .layer import MoELayer  # noqa: E402  (buffers + the call sequence)

__all__ = ["MoELayer", "OccError", "occ_layer_desc", "occ_brim", "make_desc", "desc_of",
           "make_brim", "occ_workspace_bytes", "occ_ffn_workspace_bytes", "occ_route_topk",
           "occ_route_workspace_bytes", "occ_route_topk_ws",
           "occ_build_brim", "occ_build_brim_noalloc", "occ_build_brim_pruned", "occ_dispatch", "occ_expert_ffn", "occ_expert_up",
           "occ_expert_down", "occ_combine", "occ_dispatch_direct", "occ_combine_direct",
           "occ_backward_workspace_bytes", "occ_grad_combine", "occ_expert_backward",
           "occ_router_backward", "occ_grad_dispatch", "occ_shared_backward", "occ_expert_ffn_keep",
           "occ_expert_backward_kept", "occ_coactivation", "occ_cross_coactivation", "occ_home_device", "occ_local_hits",
           "occ_place_greedy", "last_error"]
