"""GPU parity of decode attention over the stored factors (jolt_decode_attention)
with the oracle's fp64 softmax attention over the oracle's own decode of the
same payloads (oracle/attention.py).

Both sides read the same payload bytes; the GPU never forms K or V.  The GPU
forms scores and sums in fp32 from bf16 (or fp32) parameters: a score of
r_t + d products carries a relative error of a few 1e-6 of its magnitude, which
moves softmax weights and the output by about that much, so
    ||o_gpu - o_ref|| <= 1e-4 ||o_ref||  per layer,   |lse_gpu - lse_ref| <= 1e-4 (1 + |lse_ref|).
"""
import numpy as np
import pytest

import synth
from oracle import attention as oatt, codec as ocodec, tucker
from tests.gpu_util import jolt_binding, payload_bytes, to_dev_bytes, to_device, torch_cuda

pytestmark = pytest.mark.gpu


def _bits_to_f64(u16):
    return (u16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _payload_encoded(pay_host, jb, jit, a, dtype):
    """The oracle's view of a payload: stored parameters, codes and scales."""
    off, total = jb.jolt_payload_layout(jit, a)
    L, H, T, d = jit.L, jit.H, jit.T, jit.d
    rt, rf = (a.rt, a.rf) if a.rt and a.rf else (0, 0)
    N = L * H * T * d

    def arr(k, count):
        if dtype == "f32":
            return np.frombuffer(pay_host[off[k]:off[k] + 4 * count], dtype="<f4").astype(np.float64)
        return _bits_to_f64(np.frombuffer(pay_host[off[k]:off[k] + 2 * count], dtype="<u2"))
    sp = ocodec.StoredParams(Ut=arr(0, T * rt).reshape(T, rt), Uf=arr(1, d * rf).reshape(d, rf),
                             C=arr(2, L * H * rt * rf).reshape(L, H, rt, rf))
    words = sc = None
    if a.bits:
        G = N // 64
        sc = np.frombuffer(pay_host[off[3]:off[3] + 2 * G], dtype="<u2")
        words = np.frombuffer(pay_host[off[4]:off[4] + 8 * a.bits * G], dtype="<u8").reshape(G, a.bits)
    return ocodec.Encoded(rt, rf, a.bits, sp, words, sc, None)


def _attend(torch, jb, h, pairs, q_heads, scale):
    """pairs: (k_item, k_alloc, k_payload_dev, v_item, v_alloc, v_payload_dev, q_dev)."""
    groups, outs, lses = [], [], []
    for (ki, ka, kp, vi, va, vp, q) in pairs:
        out = torch.full((ki.L, q_heads, ki.d), float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.full((ki.L, q_heads), float("nan"), dtype=torch.float32, device="cuda")
        groups.append(jb.jolt_attn_group(ki, vi, ka, va, kp.data_ptr(), vp.data_ptr(), q.data_ptr(),
                                         out.data_ptr(), lse.data_ptr()))
        outs.append(out)
        lses.append(lse)
    wsb = jb.jolt_attention_workspace_size(groups, q_heads)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    jb.jolt_decode_attention(h, groups, q_heads, scale, ws.data_ptr(), wsb, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return [o.cpu().numpy().astype(np.float64) for o in outs], [l.cpu().numpy().astype(np.float64) for l in lses]


def _check(o_gpu, l_gpu, K, V, q, scale):
    o_ref, l_ref = oatt.decode_attention(q, K, V, scale)
    for l in range(q.shape[0]):
        err = np.linalg.norm(o_gpu[l] - o_ref[l]) / np.linalg.norm(o_ref[l])
        assert err <= 1e-4, (l, err)
    assert np.max(np.abs(l_gpu - l_ref) / (1.0 + np.abs(l_ref))) <= 1e-4


CASES = [
    # dtype, L, H, T, d, G, K (rt, rf, bits), V (rt, rf, bits)
    ("bf16", 2, 4, 704, 128, 4, (16, 24, 4), (24, 16, 3)),      # ragged last chunk
    ("bf16", 2, 2, 512, 128, 2, (0, 0, 4), (8, 8, 2)),          # K residual only
    ("bf16", 1, 2, 320, 128, 8, (32, 128, 0), (16, 16, 0)),     # Tucker only on both
    ("bf16", 2, 3, 256, 64, 2, (16, 16, 4), (16, 16, 5)),
    ("f32", 2, 4, 256, 64, 1, (16, 12, 4), (16, 12, 4)),        # the fp32 exact configuration's shape
]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_attention_over_oracle_payloads(case):
    """Payloads built from the oracle's own stored parameters and codes."""
    torch = torch_cuda()
    jb = jolt_binding()
    dtype, L, H, T, d, G, ka, va = case
    base = "tiny_exact_f32" if dtype == "f32" else "mistral7b_gqa_1k"
    cfg = synth.config(base, L=L, H=H, T=T, d=d, rank_t=min(16, T), rank_f=min(12, d), dtype=dtype)
    kit, vit = synth.make_items(cfg, 2)                           # K and V of group 0
    dev, Kd, Vd = [], None, None
    for it, (rt, rf, b) in ((kit, ka), (vit, va)):
        X = it.x
        U_t = tucker.token_factor_exact(X, max(rt, 8))[1]
        U_f = tucker.feature_factor(X)[1]
        sp = ocodec.stored_params(U_t, U_f, tucker.core_full(X, U_t, U_f), rt, rf, dtype)
        enc = ocodec.encode(X, sp, b, it.seed, it.item_id, dtype)
        jit = jb.make_item(L, H, T, d, dtype, it.item_id, it.seed)
        al = jb.jolt_alloc(rt, rf, b, 0, 0, 0.0)
        pay = payload_bytes(jb, jit, al, sp, dtype, enc.words, enc.scale_bits)
        dev.append((jit, al, to_dev_bytes(pay, torch)))
        dec = oatt.decoded(enc, (L, H, T, d), it.seed, it.item_id, dtype)
        if Kd is None:
            Kd = dec
        else:
            Vd = dec
    q = np.random.default_rng(T + d).standard_normal((L, G * H, d)).astype(np.float32)
    qd = torch.from_numpy(q).cuda()
    scale = 1.0 / np.sqrt(d)
    h = jb.jolt_create(0)
    try:
        print("attention", case, flush=True)
        (o,), (lse,) = _attend(torch, jb, h, [(dev[0][0], dev[0][1], dev[0][2], dev[1][0], dev[1][1], dev[1][2], qd)],
                               G * H, scale)
    finally:
        jb.jolt_destroy(h)
    _check(o, lse, Kd, Vd, q.astype(np.float64), float(np.float32(scale)))


@pytest.mark.parametrize("name,ratio,groups", [("mistral7b_gqa_1k", 2.0, 8), ("llama31_8b_gqa_64k", 4.0, 1)])
def test_attention_after_compress(name, ratio, groups):
    """The library's own payloads (jolt_plan + jolt_compress) at full item
    size: the whole 8-group Mistral-7B-shaped cache, and one group of the
    65536-token cache at 4x (a binding budget); every layer and query head of
    the first group and the last is checked (Mistral-7B: 32 query heads on 8
    KV heads per layer)."""
    torch = torch_cuda()
    jb = jolt_binding()
    import json
    import os
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    delta = json.load(open(os.path.join(root, "tests", "golden", "delta_b.json")))["delta"]
    cfg = synth.config(name)
    items = synth.make_items(cfg, 2 * groups)
    jitems = [jb.make_item(i.L, i.H, i.T, i.d, "bf16", i.item_id, i.seed) for i in items]
    budget = synth.budget_for_ratio(cfg, ratio, n_items=len(items))
    J = jb.Jolt(jb.make_config("randomized", rt_max=cfg.rt_max, budget=budget, delta=delta, bits=cfg.bits), jitems)
    xs = [to_device(i, torch) for i in items]
    print("plan", name, len(items), flush=True)
    allocs, lam = J.plan(xs)
    assert J.status == jb.JOLT_OK
    pays = J.alloc_payloads(allocs)
    J.compress(xs, pays, allocs)
    del xs
    torch.cuda.synchronize()
    Hq = 4 * cfg.H
    rng = np.random.default_rng(11)
    qs = [rng.standard_normal((cfg.L, Hq, cfg.d)).astype(np.float32) for _ in range(groups)]
    qd = [torch.from_numpy(q).cuda() for q in qs]
    pairs = [(jitems[2 * g], allocs[2 * g], pays[2 * g], jitems[2 * g + 1], allocs[2 * g + 1], pays[2 * g + 1], qd[g])
             for g in range(groups)]
    scale = float(np.float32(1.0 / np.sqrt(cfg.d)))
    h = jb.jolt_create(0)
    try:
        outs, lses = _attend(torch, jb, h, pairs, Hq, scale)
    finally:
        jb.jolt_destroy(h)
    for g in sorted({0, groups - 1}):
        encs = []
        for k in (2 * g, 2 * g + 1):
            host = pays[k].cpu().numpy().tobytes()
            encs.append(_payload_encoded(host, jb, jitems[k], allocs[k], "bf16"))
        print("group", g, "K", (allocs[2 * g].rt, allocs[2 * g].rf, allocs[2 * g].bits), "V",
              (allocs[2 * g + 1].rt, allocs[2 * g + 1].rf, allocs[2 * g + 1].bits), flush=True)
        shape = (cfg.L, cfg.H, cfg.T, cfg.d)
        Kd = oatt.decoded(encs[0], shape, items[2 * g].seed, items[2 * g].item_id, "bf16")
        Vd = oatt.decoded(encs[1], shape, items[2 * g + 1].seed, items[2 * g + 1].item_id, "bf16")
        _check(outs[g], lses[g], Kd, Vd, qs[g].astype(np.float64), scale)
    J.close()
