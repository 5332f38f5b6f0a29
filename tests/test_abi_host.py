"""C-ABI checks that need no GPU: the library loads, exports every entry point
the header declares, and its pure-host calls agree with the oracle bit for bit
(byte accounting, payload layout / header, and the single-dual allocation
given the same distortion and byte tables)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from oracle import alloc as oalloc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libjolt.h")

jb = pytest.importorskip("kv_cache_compression_jolt_amd.binding")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(jb.LIB_PATH):
        pytest.skip("libjolt.so not built")
    return jb.lib()


def _declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"\b(jolt_[a-z_]+)\s*\(", txt)) - {"jolt_handle"})


def test_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", jb.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (jolt_\w+)", out))
    missing = [s for s in _declared() if s not in exported]
    assert not missing, missing
    assert set(jb.EXPORTED) <= exported


def test_status_strings(lib):
    for s in range(8):
        assert lib.jolt_status_str(s)


@pytest.mark.parametrize("dtype,e", [("bf16", 2), ("f32", 4)])
def test_item_bytes_matches_oracle(lib, dtype, e):
    for (L, H, T, d) in [(4, 8, 1024, 128), (2, 4, 256, 64), (4, 40, 4096, 128)]:
        it = jb.make_item(L, H, T, d, dtype)
        for rt, rf, b in [(0, 0, 0), (0, 0, 4), (8, 8, 2), (128, 64, 3), (64, 0, 4), (256, 128, 8)]:
            assert jb.jolt_item_bytes(it, rt, rf, b) == oalloc.item_bytes(L, H, T, d, e, rt, rf, b)


def test_payload_layout_counts_accounted_bytes(lib):
    it = jb.make_item(4, 8, 1024, 128, "bf16", 3, 7)
    for rt, rf, b in [(0, 0, 0), (0, 0, 4), (64, 48, 2), (128, 128, 4), (8, 8, 3)]:
        a = jb.jolt_alloc(rt, rf, b, 0, 0, 0.0)
        off, total = jb.jolt_payload_layout(it, a)
        assert off[0] == 256 and all(o % 256 == 0 for o in off) and total % 256 == 0
        sizes = [off[1] - off[0], off[2] - off[1], off[3] - off[2], off[4] - off[3], total - off[4]]
        # sections hold exactly the accounted bytes, up to 256-byte alignment
        N = 4 * 8 * 1024 * 128
        want = [2 * 1024 * rt, 2 * 128 * rf, 2 * 32 * rt * rf, (2 * N // 64) if b else 0, (N * b // 8) if b else 0]
        for s, w in zip(sizes, want):
            assert w <= s < w + 256 or (w == 0 and s == 0)
        assert sum(want) == jb.jolt_item_bytes(it, rt, rf, b)


def test_header_validate_and_corruption(lib):
    it = jb.make_item(2, 4, 256, 64, "f32", 9, 123)
    a = jb.jolt_alloc(16, 16, 4, 0, 0, 0.0)
    hdr = jb.jolt_payload_header(it, a)
    assert hdr[:4] == b"JOLT"
    assert jb.jolt_payload_validate(hdr, it, a) == jb.JOLT_OK
    bad = bytearray(hdr)
    bad[20] ^= 1                      # shape byte
    assert jb.jolt_payload_validate(bytes(bad), it, a) == jb.JOLT_E_CORRUPT
    other = jb.jolt_alloc(16, 16, 3, 0, 0, 0.0)
    assert jb.jolt_payload_validate(hdr, it, other) == jb.JOLT_E_CORRUPT


def test_invalid_arguments_rejected_before_launch(lib):
    items = [jb.make_item(2, 4, 256, 96)]                       # d not 64 / 128
    cfg = jb.make_config(rt_max=16, fixed=(16, 16, 4))
    with pytest.raises(jb.JoltError) as e:
        jb.jolt_workspace_size(cfg, items)
    assert e.value.status == jb.JOLT_E_UNSUPPORTED
    items = [jb.make_item(2, 4, 256, 64)]
    bad = jb.make_config(rt_max=16, fixed=(16, 16, 4))
    bad.group_size = 32
    with pytest.raises(jb.JoltError):
        jb.jolt_workspace_size(bad, items)
    bad = jb.make_config(rt_max=16, fixed=(16, 16, 4), bits=(0, 1, 4))
    with pytest.raises(jb.JoltError):
        jb.jolt_workspace_size(bad, items)
    bad = jb.make_config(rt_max=16, budget=10 ** 6, delta=[0.5, 0, 0.5, 0.1, 0.01])  # delta_0 != 1
    with pytest.raises(jb.JoltError):
        jb.jolt_workspace_size(bad, items)
    ok = jb.make_config(rt_max=16, fixed=(16, 16, 4))
    p, c = jb.jolt_workspace_size(ok, items)
    assert p > 0 and c > 0


def _tables(n_items, grid, seed, structured=False):
    rg = np.random.default_rng(seed)
    out = []
    for _ in range(n_items):
        cand = grid.copy()
        if structured:
            # realistic shape: D = delta_b * truncation energy, bytes from the formula
            E = np.sort(rg.exponential(1.0, (16, 16)))[::-1]
            tot = float(E.sum()) * 1.5
            delta = [1.0, None, 0.515, 0.063, 0.0116]
            D = oalloc.distortion_table(E, tot, delta, cand)
            B = oalloc.bytes_table(2, 4, 64, 128, 2, cand)
        else:
            D = rg.uniform(0, 100, len(cand))
            B = rg.integers(10, 10 ** 6, len(cand)).astype(np.int64)
        out.append({"cand": cand, "D": D, "B": B})
    return out


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("structured", [False, True])
def test_plan_from_tables_bit_exact(lib, seed, structured):
    grid = oalloc.candidate_grid(16, 16, 8, (0, 2, 3, 4))
    tabs = _tables(5, grid, seed, structured)
    Bmin = sum(int(t["B"].min()) for t in tabs)
    Bmax = sum(int(t["B"].max()) for t in tabs)
    rg = np.random.default_rng(seed + 100)
    budgets = sorted(set([Bmin, Bmax, Bmin - 1] + [int(v) for v in rg.integers(Bmin, Bmax, 12)]))
    for budget in budgets:
        ch, lam, ok = oalloc.lagrangian_allocate(tabs, budget)
        st, al, lam_c = jb.jolt_plan_from_tables([t["cand"] for t in tabs], [t["D"] for t in tabs],
                                                 [t["B"] for t in tabs], budget)
        if not ok:
            assert st == jb.JOLT_E_INFEASIBLE
        else:
            assert st == jb.JOLT_OK
            assert abs(lam_c - float(lam)) <= 1e-12 * max(1.0, abs(float(lam)))
        for t, c, a in zip(tabs, ch, al):
            assert (a.rt, a.rf, a.bits) == tuple(int(v) for v in t["cand"][c])
            assert a.bytes == int(t["B"][c]) and a.distortion == float(t["D"][c])


@pytest.mark.parametrize("seed", range(3))
def test_plan_from_tables_tied_slopes(lib, seed):
    # Groups of items with identical integer tables share every hull slope
    # exactly: the selection of lambda* must take all edges of one slope, over
    # all items, together (the pages' single dual, landing page abstract).
    grid = oalloc.candidate_grid(16, 16, 8, (0, 2, 3, 4))
    rg = np.random.default_rng(seed + 7)
    base = []
    for _ in range(3):
        D = rg.integers(0, 40, len(grid)).astype(np.float64)
        B = (rg.integers(1, 64, len(grid)) * 16).astype(np.int64)
        base.append((D, B))
    tabs = [{"cand": grid, "D": base[i % 3][0], "B": base[i % 3][1]} for i in range(12)]
    Bmin = sum(int(t["B"].min()) for t in tabs)
    Bmax = sum(int(t["B"].max()) for t in tabs)
    budgets = sorted(set([Bmin, Bmax] + [int(v) for v in rg.integers(Bmin, Bmax, 40)]))
    for budget in budgets:
        ch, lam, ok = oalloc.lagrangian_allocate(tabs, budget)
        st, al, lam_c = jb.jolt_plan_from_tables([t["cand"] for t in tabs], [t["D"] for t in tabs],
                                                 [t["B"] for t in tabs], budget)
        assert ok and st == jb.JOLT_OK
        assert abs(lam_c - float(lam)) <= 1e-12 * max(1.0, abs(float(lam)))
        for t, c, a in zip(tabs, ch, al):
            assert (a.rt, a.rf, a.bits) == tuple(int(v) for v in t["cand"][c])


def test_plan_from_tables_full_grid(lib):
    # one c2-sized problem: 16 items x 1028 candidates
    grid = oalloc.candidate_grid(128, 128, 8, (0, 2, 3, 4))
    rg = np.random.default_rng(5)
    tabs = []
    for i in range(16):
        E = np.sort(rg.exponential(1.0, (128, 128)), axis=None)[::-1].reshape(128, 128) * rg.uniform(0.5, 2)
        tot = float(E.sum()) * rg.uniform(1.2, 3.0)
        D = oalloc.distortion_table(E, tot, [1.0, None, 0.515, 0.063, 0.0116], grid)
        B = oalloc.bytes_table(4, 8, 1024, 128, 2, grid)
        tabs.append({"cand": grid, "D": D, "B": B})
    budget = 16 * 4 * 8 * 1024 * 128 * 2 // 2
    ch, lam, ok = oalloc.lagrangian_allocate(tabs, budget)
    st, al, lam_c = jb.jolt_plan_from_tables([t["cand"] for t in tabs], [t["D"] for t in tabs],
                                             [t["B"] for t in tabs], budget)
    assert ok and st == 0
    assert [(a.rt, a.rf, a.bits) for a in al] == [tuple(int(v) for v in t["cand"][c]) for t, c in zip(tabs, ch)]
