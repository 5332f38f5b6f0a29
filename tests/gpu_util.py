"""Helpers for the GPU tests: device tensors from synthetic items and payload
assembly from oracle-stored parameters (plain byte plumbing, no method math)."""
import numpy as np
import pytest


def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def jolt_binding():
    from kv_cache_compression_jolt_amd import binding as jb
    jb.lib()                      # raises if the library is not built
    return jb


def to_device(item, torch):
    if item.raw.dtype == np.uint16:
        return torch.from_numpy(item.raw.view(np.int16).copy()).cuda()
    return torch.from_numpy(item.raw.copy()).cuda()


def f64_to_param_bytes(v, dtype):
    if dtype == "f32":
        return np.ascontiguousarray(v, dtype=np.float32).tobytes()
    f = np.ascontiguousarray(v, dtype=np.float32)
    u = f.view(np.uint32)
    assert not np.any(u & 0xFFFF), "parameter values must already be bf16"
    return (u >> 16).astype(np.uint16).tobytes()


def payload_bytes(jb, jitem, alloc, params, dtype, words=None, scale_bits=None):
    """Host bytes of a payload: header + stored parameters (+ optional codes)."""
    off, total = jb.jolt_payload_layout(jitem, alloc)
    buf = bytearray(total)
    buf[:64] = jb.jolt_payload_header(jitem, alloc)
    if alloc.rt and alloc.rf:
        for o, arr in zip(off[:3], (params.Ut, params.Uf, params.C)):
            b = f64_to_param_bytes(arr, dtype)
            buf[o:o + len(b)] = b
    if words is not None:
        sb = np.ascontiguousarray(scale_bits, dtype="<u2").tobytes()
        buf[off[3]:off[3] + len(sb)] = sb
        wb = np.ascontiguousarray(words, dtype="<u8").tobytes()
        buf[off[4]:off[4] + len(wb)] = wb
    return bytes(buf)


def to_dev_bytes(b, torch):
    return torch.frombuffer(bytearray(b), dtype=torch.uint8).cuda()


def section(payload_host: bytes, off, total, idx):
    ends = list(off[1:]) + [total]
    return payload_host[off[idx]:ends[idx]]


def out_values(t, dtype):
    a = t.cpu().numpy()
    if dtype == "f32":
        return a.astype(np.float64)
    return (a.view(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rel(a, b):
    return float(np.linalg.norm((a - b).ravel()) / max(np.linalg.norm(b.ravel()), 1e-300))
