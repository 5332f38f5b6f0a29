"""ctypes binding for libjolt (argument marshalling only).

Every function here has the name of the C entry point it calls and forwards
plain pointers and sizes; all computation runs inside libjolt.so.  PyTorch is
used by the helpers at the bottom only to own device memory and to supply the
current HIP stream.  Importing fails loudly if the library is not built.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import List, Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libjolt.so")

JOLT_OK, JOLT_E_INVALID, JOLT_E_UNSUPPORTED, JOLT_E_WORKSPACE = 0, 1, 2, 3
JOLT_E_INFEASIBLE, JOLT_E_NOCONV, JOLT_E_DEVICE, JOLT_E_CORRUPT = 4, 5, 6, 7
JOLT_BF16, JOLT_F32 = 0, 1
JOLT_TOKEN_EXACT, JOLT_TOKEN_RANDOMIZED = 0, 1


class JoltError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("libjolt status %d: %s" % (status, msg))
        self.status = status


class jolt_item(C.Structure):
    _fields_ = [("L", C.c_int32), ("H", C.c_int32), ("T", C.c_int32), ("d", C.c_int32),
                ("dtype", C.c_int32), ("item_id", C.c_uint32), ("seed", C.c_uint64)]


class jolt_config(C.Structure):
    _fields_ = [("mode", C.c_int32), ("oversample", C.c_int32), ("power_iters", C.c_int32),
                ("rank_step", C.c_int32), ("rt_max", C.c_int32), ("rf_max", C.c_int32),
                ("bits_mask", C.c_uint32), ("group_size", C.c_int32), ("budget_bytes", C.c_int64),
                ("fixed_rt", C.c_int32), ("fixed_rf", C.c_int32), ("fixed_bits", C.c_int32),
                ("max_sweeps", C.c_int32), ("delta_b", C.c_double * 9)]


class jolt_alloc(C.Structure):
    _fields_ = [("rt", C.c_int32), ("rf", C.c_int32), ("bits", C.c_int32), ("reserved", C.c_int32),
                ("bytes", C.c_int64), ("distortion", C.c_double)]


class jolt_attn_group(C.Structure):
    _fields_ = [("k_item", jolt_item), ("v_item", jolt_item), ("k_alloc", jolt_alloc), ("v_alloc", jolt_alloc),
                ("k_payload", C.c_void_p), ("v_payload", C.c_void_p), ("q", C.c_void_p), ("out", C.c_void_p),
                ("lse", C.c_void_p)]


class jolt_factor_view(C.Structure):
    _fields_ = [("ut", C.c_void_p), ("uf", C.c_void_p), ("lam_t", C.c_void_p), ("lam_f", C.c_void_p),
                ("core", C.c_void_p), ("energy", C.c_void_p), ("normx2", C.c_void_p),
                ("rt_max", C.c_int32), ("rf_max", C.c_int32)]


EXPORTED = [
    "jolt_create", "jolt_destroy", "jolt_status_str", "jolt_last_error", "jolt_workspace_size",
    "jolt_item_bytes", "jolt_payload_size", "jolt_payload_layout", "jolt_payload_header",
    "jolt_payload_validate", "jolt_plan", "jolt_replan", "jolt_compress", "jolt_encode_residual",
    "jolt_decompress", "jolt_decompress_noalloc", "jolt_attention_workspace_size", "jolt_decode_attention",
    "jolt_plan_factors", "jolt_plan_from_tables", "jolt_rotate", "jolt_quantize_pack",
    "jolt_unpack_dequant", "jolt_rademacher", "jolt_eigh", "jolt_eigh_workspace_size", "jolt_kernel_timer",
    "jolt_kernel_time",
]

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libjolt.so is not built (run python -m kv_cache_compression_jolt_amd.build)")
        L = C.CDLL(LIB_PATH)
        P, I32, U32, I64, U64, SZ, D = (C.c_void_p, C.c_int32, C.c_uint32, C.c_int64, C.c_uint64,
                                         C.c_size_t, C.c_double)
        sig = {
            "jolt_create": (I32, [C.c_int, C.POINTER(P)]),
            "jolt_destroy": (None, [P]),
            "jolt_status_str": (C.c_char_p, [I32]),
            "jolt_last_error": (C.c_char_p, [P]),
            "jolt_workspace_size": (I32, [C.POINTER(jolt_config), C.POINTER(jolt_item), I32,
                                          C.POINTER(SZ), C.POINTER(SZ)]),
            "jolt_item_bytes": (I64, [C.POINTER(jolt_item), I32, I32, I32]),
            "jolt_payload_size": (I32, [C.POINTER(jolt_item), C.POINTER(jolt_alloc), C.POINTER(SZ)]),
            "jolt_payload_layout": (I32, [C.POINTER(jolt_item), C.POINTER(jolt_alloc), C.POINTER(SZ),
                                          C.POINTER(SZ)]),
            "jolt_payload_header": (I32, [C.POINTER(jolt_item), C.POINTER(jolt_alloc), P]),
            "jolt_payload_validate": (I32, [P, C.POINTER(jolt_item), C.POINTER(jolt_alloc)]),
            "jolt_plan": (I32, [P, C.POINTER(jolt_config), C.POINTER(jolt_item), I32, C.POINTER(P), P, SZ, P,
                                C.POINTER(jolt_alloc), C.POINTER(D)]),
            "jolt_replan": (I32, [P, C.POINTER(jolt_config), C.POINTER(jolt_item), I32, P, SZ, P,
                                  C.POINTER(jolt_alloc), C.POINTER(D)]),
            "jolt_compress": (I32, [P, C.POINTER(jolt_config), C.POINTER(jolt_item), I32, C.POINTER(P),
                                    C.POINTER(jolt_alloc), P, SZ, P, SZ, C.POINTER(P), P]),
            "jolt_encode_residual": (I32, [P, C.POINTER(jolt_item), I32, C.POINTER(P), C.POINTER(jolt_alloc),
                                           P, SZ, C.POINTER(P), P]),
            "jolt_decompress": (I32, [P, C.POINTER(jolt_item), I32, C.POINTER(jolt_alloc), C.POINTER(P), P, SZ,
                                      C.POINTER(P), P]),
            "jolt_decompress_noalloc": (I32, [P, C.POINTER(jolt_item), I32, C.POINTER(jolt_alloc), C.POINTER(P),
                                              C.POINTER(P), P]),
            "jolt_attention_workspace_size": (I32, [C.POINTER(jolt_attn_group), I32, I32, C.POINTER(SZ)]),
            "jolt_decode_attention": (I32, [P, C.POINTER(jolt_attn_group), I32, I32, C.c_float, P, SZ, P]),
            "jolt_plan_factors": (I32, [C.POINTER(jolt_config), C.POINTER(jolt_item), I32, P, I32,
                                        C.POINTER(jolt_factor_view)]),
            "jolt_plan_from_tables": (I32, [I32, C.POINTER(I32), C.POINTER(C.POINTER(I32)),
                                            C.POINTER(C.POINTER(D)), C.POINTER(C.POINTER(I64)), I64,
                                            C.POINTER(jolt_alloc), C.POINTER(D)]),
            "jolt_rotate": (I32, [P, P, P, I64, I32, U64, U32, I32, P]),
            "jolt_quantize_pack": (I32, [P, P, I64, I32, I32, P, P, P]),
            "jolt_unpack_dequant": (I32, [P, P, P, I64, I32, I32, P, P]),
            "jolt_rademacher": (I32, [P, U64, U32, U32, U64, I64, P, P]),
            "jolt_eigh": (I32, [P, I32, I32, P, I32, I64, P, P, P, I32, P, SZ, P]),
            "jolt_eigh_workspace_size": (SZ, [I32, I32, I32]),
            "jolt_kernel_timer": (I32, [P, C.c_char_p, I32]),
            "jolt_kernel_time": (I32, [P, C.c_char_p, C.POINTER(D), C.POINTER(I64)]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(status: int, handle=None):
    if status != JOLT_OK:
        msg = ""
        if handle is not None:
            msg = (lib().jolt_last_error(handle) or b"").decode()
        raise JoltError(status, msg or lib().jolt_status_str(status).decode())


def _items(items: Sequence[jolt_item]):
    arr = (jolt_item * max(1, len(items)))(*items)
    return arr


def _ptrs(ptrs: Sequence[int]):
    return (C.c_void_p * max(1, len(ptrs)))(*[C.c_void_p(int(p)) for p in ptrs])


# ------------------------------------------------------------------ C entry points
def jolt_create(device: int = 0):
    h = C.c_void_p()
    _check(lib().jolt_create(device, C.byref(h)))
    return h


def jolt_destroy(h):
    lib().jolt_destroy(h)


def jolt_workspace_size(cfg: jolt_config, items: Sequence[jolt_item]):
    a, b = C.c_size_t(), C.c_size_t()
    _check(lib().jolt_workspace_size(C.byref(cfg), _items(items), len(items), C.byref(a), C.byref(b)))
    return a.value, b.value


def jolt_item_bytes(item: jolt_item, rt: int, rf: int, bits: int) -> int:
    return int(lib().jolt_item_bytes(C.byref(item), rt, rf, bits))


def jolt_payload_size(item: jolt_item, a: jolt_alloc) -> int:
    s = C.c_size_t()
    _check(lib().jolt_payload_size(C.byref(item), C.byref(a), C.byref(s)))
    return s.value


def jolt_payload_layout(item: jolt_item, a: jolt_alloc):
    off = (C.c_size_t * 5)()
    tot = C.c_size_t()
    _check(lib().jolt_payload_layout(C.byref(item), C.byref(a), off, C.byref(tot)))
    return list(off), tot.value


def jolt_payload_header(item: jolt_item, a: jolt_alloc) -> bytes:
    buf = (C.c_uint8 * 64)()
    _check(lib().jolt_payload_header(C.byref(item), C.byref(a), buf))
    return bytes(buf)


def jolt_payload_validate(header: bytes, item: jolt_item, a: jolt_alloc) -> int:
    buf = (C.c_uint8 * 64).from_buffer_copy(header[:64])
    return int(lib().jolt_payload_validate(buf, C.byref(item), C.byref(a)))


def jolt_plan(h, cfg, items, x_ptrs, ws_ptr, ws_bytes, stream):
    n = len(items)
    allocs = (jolt_alloc * max(1, n))()
    lam = C.c_double()
    st = lib().jolt_plan(h, C.byref(cfg), _items(items), n, _ptrs(x_ptrs), C.c_void_p(ws_ptr), ws_bytes,
                         C.c_void_p(stream), allocs, C.byref(lam))
    return st, [allocs[i] for i in range(n)], lam.value


def jolt_replan(h, cfg, items, ws_ptr, ws_bytes, stream):
    n = len(items)
    allocs = (jolt_alloc * max(1, n))()
    lam = C.c_double()
    st = lib().jolt_replan(h, C.byref(cfg), _items(items), n, C.c_void_p(ws_ptr), ws_bytes, C.c_void_p(stream),
                           allocs, C.byref(lam))
    return st, [allocs[i] for i in range(n)], lam.value


def jolt_compress(h, cfg, items, x_ptrs, allocs, plan_ptr, plan_bytes, codec_ptr, codec_bytes, pay_ptrs, stream):
    n = len(items)
    arr = (jolt_alloc * max(1, n))(*allocs)
    _check(lib().jolt_compress(h, C.byref(cfg), _items(items), n, _ptrs(x_ptrs), arr, C.c_void_p(plan_ptr),
                               plan_bytes, C.c_void_p(codec_ptr), codec_bytes, _ptrs(pay_ptrs),
                               C.c_void_p(stream)), h)


def jolt_encode_residual(h, items, x_ptrs, allocs, codec_ptr, codec_bytes, pay_ptrs, stream):
    n = len(items)
    arr = (jolt_alloc * max(1, n))(*allocs)
    _check(lib().jolt_encode_residual(h, _items(items), n, _ptrs(x_ptrs), arr, C.c_void_p(codec_ptr), codec_bytes,
                                      _ptrs(pay_ptrs), C.c_void_p(stream)), h)


def jolt_decompress(h, items, allocs, pay_ptrs, codec_ptr, codec_bytes, out_ptrs, stream):
    n = len(items)
    arr = (jolt_alloc * max(1, n))(*allocs)
    _check(lib().jolt_decompress(h, _items(items), n, arr, _ptrs(pay_ptrs), C.c_void_p(codec_ptr), codec_bytes,
                                 _ptrs(out_ptrs), C.c_void_p(stream)), h)


def jolt_decompress_noalloc(h, items, allocs, pay_ptrs, out_ptrs, stream):
    n = len(items)
    arr = (jolt_alloc * max(1, n))(*allocs)
    _check(lib().jolt_decompress_noalloc(h, _items(items), n, arr, _ptrs(pay_ptrs), _ptrs(out_ptrs),
                                         C.c_void_p(stream)), h)


def jolt_attention_workspace_size(groups: Sequence[jolt_attn_group], q_heads: int) -> int:
    arr = (jolt_attn_group * max(1, len(groups)))(*groups)
    b = C.c_size_t()
    _check(lib().jolt_attention_workspace_size(arr, len(groups), q_heads, C.byref(b)))
    return b.value


def jolt_decode_attention(h, groups: Sequence[jolt_attn_group], q_heads: int, scale: float, ws_ptr, ws_bytes, stream):
    arr = (jolt_attn_group * max(1, len(groups)))(*groups)
    _check(lib().jolt_decode_attention(h, arr, len(groups), q_heads, C.c_float(scale), C.c_void_p(ws_ptr), ws_bytes,
                                       C.c_void_p(stream)), h)


def jolt_plan_factors(cfg, items, plan_ptr, i) -> jolt_factor_view:
    v = jolt_factor_view()
    _check(lib().jolt_plan_factors(C.byref(cfg), _items(items), len(items), C.c_void_p(plan_ptr), i, C.byref(v)))
    return v


def jolt_plan_from_tables(cands: List, Ds: List, Bs: List, budget: int):
    """cands[i]: int32 (C_i, 3) array, Ds[i]: float64 (C_i,), Bs[i]: int64 (C_i,)."""
    import numpy as np
    n = len(cands)
    cands = [np.ascontiguousarray(c, dtype=np.int32) for c in cands]
    Ds = [np.ascontiguousarray(x, dtype=np.float64) for x in Ds]
    Bs = [np.ascontiguousarray(x, dtype=np.int64) for x in Bs]
    ncand = (C.c_int32 * n)(*[len(c) for c in cands])
    cp = (C.POINTER(C.c_int32) * n)(*[c.ctypes.data_as(C.POINTER(C.c_int32)) for c in cands])
    dp = (C.POINTER(C.c_double) * n)(*[x.ctypes.data_as(C.POINTER(C.c_double)) for x in Ds])
    bp = (C.POINTER(C.c_int64) * n)(*[x.ctypes.data_as(C.POINTER(C.c_int64)) for x in Bs])
    out = (jolt_alloc * n)()
    lam = C.c_double()
    st = lib().jolt_plan_from_tables(n, ncand, cp, dp, bp, int(budget), out, C.byref(lam))
    return st, [out[i] for i in range(n)], lam.value


def jolt_rotate(h, in_ptr, out_ptr, rows, d, seed, item_id, inverse, stream):
    _check(lib().jolt_rotate(h, C.c_void_p(in_ptr), C.c_void_p(out_ptr), rows, d, seed, item_id, inverse,
                             C.c_void_p(stream)), h)


def jolt_quantize_pack(h, rot_ptr, rows, d, bits, codes_ptr, scales_ptr, stream):
    _check(lib().jolt_quantize_pack(h, C.c_void_p(rot_ptr), rows, d, bits, C.c_void_p(codes_ptr),
                                    C.c_void_p(scales_ptr), C.c_void_p(stream)), h)


def jolt_unpack_dequant(h, codes_ptr, scales_ptr, rows, d, bits, out_ptr, stream):
    _check(lib().jolt_unpack_dequant(h, C.c_void_p(codes_ptr), C.c_void_p(scales_ptr), rows, d, bits,
                                     C.c_void_p(out_ptr), C.c_void_p(stream)), h)


def jolt_rademacher(h, seed, item_id, stream_id, first, count, out_ptr, stream):
    _check(lib().jolt_rademacher(h, seed, item_id, stream_id, first, count, C.c_void_p(out_ptr),
                                 C.c_void_p(stream)), h)


def jolt_eigh_workspace_size(n, count, force_jacobi=False) -> int:
    return int(lib().jolt_eigh_workspace_size(n, count, int(bool(force_jacobi))))


def jolt_eigh(h, n, count, a_ptr, lda, mat_stride, vec_ptr, lam_ptr, info_ptr, force_jacobi, ws_ptr, ws_bytes,
              stream):
    _check(lib().jolt_eigh(h, n, count, C.c_void_p(a_ptr), lda, mat_stride, C.c_void_p(vec_ptr),
                           C.c_void_p(lam_ptr), C.c_void_p(info_ptr), int(force_jacobi), C.c_void_p(ws_ptr),
                           ws_bytes, C.c_void_p(stream)), h)


def jolt_kernel_timer(h, kernel: str, enable: bool):
    _check(lib().jolt_kernel_timer(h, kernel.encode(), int(bool(enable))), h)


def jolt_kernel_time(h, kernel: str):
    """(total device ms, launches) of a kernel since its timer was turned on."""
    ms, n = C.c_double(0.0), C.c_int64(0)
    _check(lib().jolt_kernel_time(h, kernel.encode(), C.byref(ms), C.byref(n)), h)
    return ms.value, n.value


# ------------------------------------------------------------------ helpers
def make_item(L, H, T, d, dtype="bf16", item_id=0, seed=0) -> jolt_item:
    return jolt_item(L, H, T, d, JOLT_F32 if dtype == "f32" else JOLT_BF16, item_id, seed)


def make_config(mode="randomized", rt_max=128, rf_max=0, oversample=10, power_iters=1, rank_step=8,
                bits=(0, 2, 3, 4), budget=-1, fixed=(0, 0, 0), delta=None, max_sweeps=0) -> jolt_config:
    c = jolt_config()
    c.mode = JOLT_TOKEN_RANDOMIZED if mode == "randomized" else JOLT_TOKEN_EXACT
    c.oversample, c.power_iters, c.rank_step = oversample, power_iters, rank_step
    c.rt_max, c.rf_max = rt_max, rf_max
    c.bits_mask = sum(1 << b for b in bits)
    c.group_size = 64
    c.budget_bytes = int(budget)
    c.fixed_rt, c.fixed_rf, c.fixed_bits = fixed
    c.max_sweeps = max_sweeps
    dl = list(delta) if delta is not None else [1.0] + [0.0] * 8
    for b in range(9):
        v = dl[b] if b < len(dl) else 0.0
        c.delta_b[b] = float(v) if v is not None else 0.0
    return c


def stream_ptr() -> int:
    import torch
    return torch.cuda.current_stream().cuda_stream


class Jolt:
    """Owns a handle and the workspaces for one (config, item list)."""

    def __init__(self, cfg: jolt_config, items: Sequence[jolt_item], device: int = 0):
        import torch
        self.torch = torch
        self.cfg = cfg
        self.items = list(items)
        self.h = jolt_create(device)
        self.plan_bytes, self.codec_bytes = jolt_workspace_size(cfg, self.items)
        dev = torch.device("cuda", device)
        self.plan_ws = torch.empty(max(256, self.plan_bytes), dtype=torch.uint8, device=dev)
        self.codec_ws = torch.empty(max(256, self.codec_bytes), dtype=torch.uint8, device=dev)
        self.device = dev
        self.allocs: Optional[List[jolt_alloc]] = None
        self.lam = None
        self.status = None

    def plan(self, xs):
        st, allocs, lam = jolt_plan(self.h, self.cfg, self.items, [x.data_ptr() for x in xs],
                                    self.plan_ws.data_ptr(), self.plan_ws.numel(), stream_ptr())
        if st not in (JOLT_OK, JOLT_E_INFEASIBLE, JOLT_E_NOCONV):
            _check(st, self.h)
        self.status, self.allocs, self.lam = st, allocs, lam
        return allocs, lam

    def replan(self, budget):
        """The dual alone under a new budget, on this object's last plan."""
        self.cfg.budget_bytes = int(budget)
        st, allocs, lam = jolt_replan(self.h, self.cfg, self.items, self.plan_ws.data_ptr(), self.plan_ws.numel(),
                                      stream_ptr())
        if st not in (JOLT_OK, JOLT_E_INFEASIBLE, JOLT_E_NOCONV):
            _check(st, self.h)
        self.status, self.allocs, self.lam = st, allocs, lam
        return allocs, lam

    def alloc_payloads(self, allocs=None):
        allocs = allocs or self.allocs
        return [self.torch.zeros(jolt_payload_size(it, a), dtype=self.torch.uint8, device=self.device)
                for it, a in zip(self.items, allocs)]

    def compress(self, xs, payloads, allocs=None):
        allocs = allocs or self.allocs
        jolt_compress(self.h, self.cfg, self.items, [x.data_ptr() for x in xs], allocs, self.plan_ws.data_ptr(),
                      self.plan_ws.numel(), self.codec_ws.data_ptr(), self.codec_ws.numel(),
                      [p.data_ptr() for p in payloads], stream_ptr())

    def encode_residual(self, xs, payloads, allocs=None):
        allocs = allocs or self.allocs
        jolt_encode_residual(self.h, self.items, [x.data_ptr() for x in xs], allocs, self.codec_ws.data_ptr(),
                             self.codec_ws.numel(), [p.data_ptr() for p in payloads], stream_ptr())

    def decompress(self, payloads, outs, allocs=None):
        allocs = allocs or self.allocs
        jolt_decompress(self.h, self.items, allocs, [p.data_ptr() for p in payloads], self.codec_ws.data_ptr(),
                        self.codec_ws.numel(), [o.data_ptr() for o in outs], stream_ptr())

    def factors(self, i: int) -> jolt_factor_view:
        return jolt_plan_factors(self.cfg, self.items, self.plan_ws.data_ptr(), i)

    def close(self):
        if self.h is not None:
            jolt_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
