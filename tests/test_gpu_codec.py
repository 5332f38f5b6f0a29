"""GPU parity of the residual codec against the oracle.

Bit-exact where the pages' method makes an integer decision from the same fp32
input (rotation signs, sketch signs, quantized codes, scales, packing); within
fp32 rounding for the rotation; and for the fused encoder / decoder:
  * fed the oracle's stored parameters, the fused encoder's codes and scales
    may differ from the oracle's only at rounding boundaries: each differing
    code by one step, with the oracle's scaled value within the bound on the
    two residuals' difference of the midpoint (tests/parity_util.py); the
    fused decoder's output of
    those codes is the oracle's decode of the same codes to 1e-3 relative
    Frobenius (and, with no residual, the oracle's reconstruction itself); the
    reconstruction error is at most 1.05 x the oracle's + 1e-4;
  * decoding the oracle's own payload matches the oracle's decode to 1e-3.
Both sides' outputs are compared after the same final rounding to the cache dtype.
"""
import numpy as np
import pytest

import synth
from oracle import codec as ocodec, quant as oquant, rng as orng, tucker, wht
from tests.gpu_util import (jolt_binding, out_values, payload_bytes, rel, section, to_dev_bytes, to_device,
                            torch_cuda)
from tests.parity_util import check_codes, row_tolerance

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    torch = torch_cuda()
    jb = jolt_binding()
    h = jb.jolt_create(0)
    yield torch, jb, h
    jb.jolt_destroy(h)


def test_rademacher_streams_bit_exact(env):
    torch, jb, h = env
    for seed, iid, stream, first in [(0, 0, 0, 0), (7, 3, 1, 12345), (2 ** 63 + 5, 4000000000, 1, 2 ** 40)]:
        out = torch.empty(5000, dtype=torch.float32, device="cuda")
        print("rademacher", seed, iid, stream, flush=True)
        jb.jolt_rademacher(h, seed, iid, stream, first, 5000, out.data_ptr(), 0)
        torch.cuda.synchronize()
        ref = orng.rademacher(seed, iid, stream, np.arange(first, first + 5000, dtype=np.uint64))
        assert np.array_equal(out.cpu().numpy().astype(np.float64), ref)


@pytest.mark.parametrize("d", [64, 128])
def test_rotation(env, d):
    torch, jb, h = env
    rows = 1000
    x = np.random.default_rng(d).standard_normal((rows, d)).astype(np.float32)
    xin = torch.from_numpy(x).cuda()
    out = torch.empty_like(xin)
    back = torch.empty_like(xin)
    print("rotate d", d, flush=True)
    jb.jolt_rotate(h, xin.data_ptr(), out.data_ptr(), rows, d, 11, 2, 0, 0)
    jb.jolt_rotate(h, out.data_ptr(), back.data_ptr(), rows, d, 11, 2, 1, 0)
    torch.cuda.synchronize()
    s = orng.rotation_signs(11, 2, d)
    ref = wht.rotate(x.astype(np.float64), s)
    assert np.max(np.abs(out.cpu().numpy() - ref)) <= 1e-5 * np.max(np.abs(ref))
    assert np.max(np.abs(back.cpu().numpy() - x)) <= 1e-5 * np.max(np.abs(x))


def _tie_groups(bits, n):
    """Groups whose scaled values land exactly on .5 (scale 2^-3, exact in bf16,
    so x * inv is exact): half-to-even decides every element but the absmax."""
    qm = (1 << (bits - 1)) - 1
    s = np.float32(0.125)
    rg = np.random.default_rng(bits)
    g = np.empty((n, 64), dtype=np.float32)
    for i in range(n):
        k = rg.integers(-qm, qm, size=64)                 # k + 0.5 in [-qm + 0.5, qm - 0.5]
        g[i] = ((k + 0.5) * s).astype(np.float32)
        g[i, rg.integers(64)] = (qm if i % 2 else -qm) * s
    return g


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
def test_quantize_pack_bit_exact(env, bits, d):
    """The encoder's own quantize / pack / store code (the test hook runs it on
    rows read from memory) against the oracle on the oracle's fp32 rotated
    residual, with all-zero groups, exact .5 ties and a wide magnitude range:
    scales, code words and dequantized values identical."""
    torch, jb, h = env
    cfg = synth.config("mistral7b_gqa_1k", T=128, L=2, H=2, d=d)
    it = synth.make_item(cfg, synth.item_specs(cfg)[0])
    X = it.x
    lam_t, U_t = tucker.token_factor_exact(X, 16)
    lam_f, U_f = tucker.feature_factor(X)
    sp = ocodec.stored_params(U_t, U_f, tucker.core_full(X, U_t, U_f), 16, 24, "bf16")
    enc = ocodec.encode(X, sp, bits, it.seed, it.item_id, "bf16")
    rot = enc.rotated.copy()                                # (G, 64), row-major groups of the rows
    rot[3] = 0.0                                            # all-zero groups
    rot[-1] = 0.0
    rot[8:8 + 24] = _tie_groups(bits, 24)
    mag = np.exp(np.random.default_rng(7).uniform(-40, 40, (rot.shape[0], 1))).astype(np.float32)
    rot[40:] = (rot[40:] * mag[40:]).astype(np.float32)      # scales over many binades
    G = rot.shape[0]
    rows = G * 64 // d
    q_ref, s_ref = oquant.quantize_groups(rot, bits)
    w_ref = oquant.pack_codes(oquant.codes_from_q(q_ref, bits), bits)
    assert np.any((np.abs(rot[8:32] / 0.125) % 1) == 0.5)   # the tie groups do tie
    rin = torch.from_numpy(rot.reshape(rows, d).copy()).cuda()
    codes = torch.zeros(G * bits, dtype=torch.int64, device="cuda")
    scales = torch.zeros(G, dtype=torch.int16, device="cuda")
    print("quantize_pack bits", bits, "d", d, flush=True)
    jb.jolt_quantize_pack(h, rin.data_ptr(), rows, d, bits, codes.data_ptr(), scales.data_ptr(), 0)
    back = torch.empty_like(rin)
    jb.jolt_unpack_dequant(h, codes.data_ptr(), scales.data_ptr(), rows, d, bits, back.data_ptr(), 0)
    torch.cuda.synchronize()
    assert np.array_equal(scales.cpu().numpy().view(np.uint16), s_ref)
    assert np.array_equal(codes.cpu().numpy().view(np.uint64).reshape(G, bits), w_ref)
    assert np.array_equal(back.cpu().numpy().reshape(G, 64).astype(np.float64),
                          oquant.dequantize_groups(q_ref, s_ref))


CASES = [
    # dtype, L, H, T, d, rt, rf, bits
    ("bf16", 2, 3, 256, 128, 16, 24, 4),
    ("bf16", 2, 3, 200, 128, 24, 16, 2),     # ragged token tail
    ("bf16", 1, 2, 136, 128, 32, 128, 3),
    ("bf16", 2, 2, 130, 128, 8, 8, 8),
    ("bf16", 2, 3, 256, 128, 0, 0, 4),       # residual only
    ("bf16", 2, 3, 256, 128, 16, 24, 0),     # Tucker only
    ("bf16", 2, 3, 160, 64, 16, 16, 4),
    ("f32", 2, 4, 256, 64, 16, 12, 4),       # the fp32 exact configuration's shape
    ("f32", 1, 3, 96, 64, 8, 64, 5),
    ("f32", 1, 2, 128, 128, 16, 16, 4),
]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_fused_codec_parity(env, case):
    torch, jb, h = env
    dtype, L, H, T, d, rt, rf, bits = case
    base = "tiny_exact_f32" if dtype == "f32" else "mistral7b_gqa_1k"
    cfg = synth.config(base, L=L, H=H, T=T, d=d, rank_t=min(16, T), rank_f=min(12, d), dtype=dtype)
    it = synth.make_item(cfg, synth.item_specs(cfg)[1 if dtype == "bf16" else 0])
    X = it.x
    rtm = max(rt, 8)
    lam_t, U_t = tucker.token_factor_exact(X, rtm)
    lam_f, U_f = tucker.feature_factor(X)
    sp = ocodec.stored_params(U_t, U_f, tucker.core_full(X, U_t, U_f), rt, rf, dtype)
    enc = ocodec.encode(X, sp, bits, it.seed, it.item_id, dtype)
    ref = ocodec.decode(enc, L, H, T, d, it.seed, it.item_id, dtype)
    jit = jb.make_item(L, H, T, d, dtype, it.item_id, it.seed)
    al = jb.jolt_alloc(rt, rf, bits, 0, 0, 0.0)
    off, total = jb.jolt_payload_layout(jit, al)
    xdev = to_device(it, torch)
    codec_bytes = max(256, L * H * d * ((rt + 15) // 16 * 16) * 4 + 256)     # W~: fp32, or bf16 hi + lo
    ws = torch.empty(codec_bytes, dtype=torch.uint8, device="cuda")
    # (a) GPU encode of the oracle's stored parameters
    pay = to_dev_bytes(payload_bytes(jb, jit, al, sp, dtype), torch)
    print("fused codec", case, flush=True)
    jb.jolt_encode_residual(h, [jit], [xdev.data_ptr()], [al], ws.data_ptr(), ws.numel(), [pay.data_ptr()], 0)
    out = torch.empty_like(xdev)
    jb.jolt_decompress(h, [jit], [al], [pay.data_ptr()], ws.data_ptr(), ws.numel(), [out.data_ptr()], 0)
    torch.cuda.synchronize()
    host = pay.cpu().numpy().tobytes()
    assert host[:64] == jb.jolt_payload_header(jit, al)
    if bits:
        G = L * H * T * d // 64
        sc = np.frombuffer(section(host, off, total, 3)[:2 * G], dtype="<u2")
        wd = np.frombuffer(section(host, off, total, 4)[:8 * bits * G], dtype="<u8").reshape(G, bits)
        u_gpu = oquant.unpack_codes(wd, bits)
        u_ref = oquant.unpack_codes(enc.words, bits)
        # every differing code or scale is a rounding-boundary case within the
        # bound on the two residuals' difference (tests/parity_util.py)
        R = X - ocodec.low_rank(sp, L, H, T, d, dtype)
        nc, ns = check_codes(u_gpu, u_ref, sc, enc.scale_bits, enc.rotated,
                             row_tolerance(sp.Ut, sp.Uf, sp.C, R), bits, d)
        print("boundary cases: codes", nc, "scales", ns, flush=True)
    got = out_values(out, dtype)
    if bits:
        # the decode of the GPU's own codes and scales is the oracle's decode of them
        # (a residual value at a rounding boundary may take the neighbouring code
        # on either side: the encoders form it in fp32 and fp64 respectively;
        # those cases are bounded by the fractions above)
        own = ocodec.Encoded(rt, rf, bits, sp, wd, sc, None)
        assert rel(got, ocodec.decode(own, L, H, T, d, it.seed, it.item_id, dtype)) <= 1e-3
    else:
        assert rel(got, ref) <= 1e-3
    # the reconstruction error is the oracle's, up to the same tolerance
    err_gpu, err_ref = rel(got, X), rel(ref, X)
    assert err_gpu <= 1.05 * err_ref + 1e-4
    # (b) decoding the oracle's own payload
    pay2 = to_dev_bytes(payload_bytes(jb, jit, al, sp, dtype, enc.words, enc.scale_bits), torch)
    out2 = torch.empty_like(xdev)
    jb.jolt_decompress(h, [jit], [al], [pay2.data_ptr()], ws.data_ptr(), ws.numel(), [out2.data_ptr()], 0)
    torch.cuda.synchronize()
    assert rel(out_values(out2, dtype), ref) <= 1e-3
    # deterministic: a second encode writes the same bytes
    pay3 = to_dev_bytes(payload_bytes(jb, jit, al, sp, dtype), torch)
    jb.jolt_encode_residual(h, [jit], [xdev.data_ptr()], [al], ws.data_ptr(), ws.numel(), [pay3.data_ptr()], 0)
    torch.cuda.synchronize()
    assert torch.equal(pay3, pay)


def test_batched_items_mixed_bits(env):
    """Several items with different bits in one call (one launch per bit width)."""
    torch, jb, h = env
    cfg = synth.config("mistral7b_gqa_1k", T=192, L=2, H=2)
    specs = synth.item_specs(cfg)[:4]
    items = [synth.make_item(cfg, s) for s in specs]
    allocs_t = [(16, 16, 4), (8, 24, 2), (0, 0, 3), (24, 8, 0)]
    jits, als, pays, outs, refs, xs = [], [], [], [], [], []
    for it, (rt, rf, b) in zip(items, allocs_t):
        X = it.x
        U_t = tucker.token_factor_exact(X, 24)[1]
        U_f = tucker.feature_factor(X)[1]
        sp = ocodec.stored_params(U_t, U_f, tucker.core_full(X, U_t, U_f), rt, rf, "bf16")
        enc = ocodec.encode(X, sp, b, it.seed, it.item_id, "bf16")
        refs.append(ocodec.decode(enc, it.L, it.H, it.T, it.d, it.seed, it.item_id, "bf16"))
        jit = jb.make_item(it.L, it.H, it.T, it.d, "bf16", it.item_id, it.seed)
        al = jb.jolt_alloc(rt, rf, b, 0, 0, 0.0)
        jits.append(jit); als.append(al)
        pays.append(to_dev_bytes(payload_bytes(jb, jit, al, sp, "bf16"), torch))
        xs.append(to_device(it, torch))
        outs.append(torch.empty_like(xs[-1]))
    ws = torch.empty(1 << 22, dtype=torch.uint8, device="cuda")
    print("batched mixed bits", flush=True)
    jb.jolt_encode_residual(h, jits, [x.data_ptr() for x in xs], als, ws.data_ptr(), ws.numel(),
                            [p.data_ptr() for p in pays], 0)
    jb.jolt_decompress(h, jits, als, [p.data_ptr() for p in pays], ws.data_ptr(), ws.numel(),
                       [o.data_ptr() for o in outs], 0)
    torch.cuda.synchronize()
    for o, r in zip(outs, refs):
        assert rel(out_values(o, "bf16"), r) <= 1e-3


def test_workspace_too_small_is_rejected(env):
    torch, jb, h = env
    jit = jb.make_item(2, 2, 128, 128, "bf16", 0, 0)
    al = jb.jolt_alloc(16, 16, 4, 0, 0, 0.0)
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    pay = torch.zeros(jb.jolt_payload_size(jit, al), dtype=torch.uint8, device="cuda")
    x = torch.zeros(2 * 2 * 128 * 128, dtype=torch.int16, device="cuda")
    with pytest.raises(jb.JoltError) as e:
        jb.jolt_encode_residual(h, [jit], [x.data_ptr()], [al], ws.data_ptr(), ws.numel(), [pay.data_ptr()], 0)
    assert e.value.status == jb.JOLT_E_WORKSPACE
