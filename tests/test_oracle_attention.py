"""Pins for the oracle's decode attention (oracle/attention.py): closed forms
and invariants of softmax attention that a dropped term, a wrong sign, a wrong
axis or a wrong head mapping would break."""
import numpy as np

from oracle import attention as oatt


def test_single_token_returns_its_value():
    rng = np.random.default_rng(1)
    q, K, V = rng.standard_normal((3, 16)), rng.standard_normal((1, 16)), rng.standard_normal((1, 16))
    o, lse = oatt.softmax_attention(q, K, V, 0.25)
    assert np.allclose(o, np.repeat(V, 3, axis=0), rtol=0, atol=1e-15)
    assert np.allclose(lse, 0.25 * (q @ K[0]), rtol=0, atol=1e-14)


def test_equal_scores_average_the_values():
    rng = np.random.default_rng(2)
    T, d = 37, 8
    K = np.tile(rng.standard_normal((1, d)), (T, 1))             # every key the same
    V = rng.standard_normal((T, d))
    q = rng.standard_normal((2, d))
    o, lse = oatt.softmax_attention(q, K, V, 0.5)
    assert np.allclose(o, np.repeat(V.mean(axis=0, keepdims=True), 2, axis=0), atol=1e-14)
    assert np.allclose(lse, 0.5 * (q @ K[0]) + np.log(T), atol=1e-13)


def test_shift_invariance_and_lse_shift():
    """Adding u to every key adds scale q.u to every score: the output is
    unchanged and the log-sum-exp moves by exactly that amount."""
    rng = np.random.default_rng(3)
    T, d = 50, 16
    q, K, V, u = (rng.standard_normal((4, d)), rng.standard_normal((T, d)), rng.standard_normal((T, d)),
                  rng.standard_normal(d))
    o1, l1 = oatt.softmax_attention(q, K, V, 0.3)
    o2, l2 = oatt.softmax_attention(q, K + u, V, 0.3)
    assert np.allclose(o1, o2, atol=1e-13)
    assert np.allclose(l2 - l1, 0.3 * (q @ u), atol=1e-12)


def test_dominant_key_selects_its_value_and_order_is_irrelevant():
    rng = np.random.default_rng(4)
    T, d = 20, 8
    K, V = rng.standard_normal((T, d)), rng.standard_normal((T, d))
    q = K[7:8] * 60.0                                             # key 7 wins by a wide margin
    o, lse = oatt.softmax_attention(q, K, V, 1.0)
    s = (q @ K.T)[0]
    gap = s[7] - np.max(np.delete(s, 7))
    assert gap > 50 and np.allclose(o[0], V[7], atol=np.exp(-gap) * 10 * np.abs(V).max())
    perm = rng.permutation(T)
    o2, lse2 = oatt.softmax_attention(q, K[perm], V[perm], 1.0)
    assert np.allclose(o, o2, atol=1e-14) and np.allclose(lse, lse2, atol=1e-13)


def test_convexity_and_grouped_query_mapping():
    """Outputs are convex combinations of the values (inside their bounding
    box), and query head j attends to KV head j // G."""
    rng = np.random.default_rng(5)
    L, H, G, T, d = 2, 3, 2, 9, 4
    K, V = rng.standard_normal((L, H, T, d)), rng.standard_normal((L, H, T, d))
    q = rng.standard_normal((L, H * G, d))
    o, lse = oatt.decode_attention(q, K, V, 0.5)
    for l in range(L):
        for j in range(H * G):
            h = j // G
            assert np.all(o[l, j] <= V[l, h].max(axis=0) + 1e-14) and np.all(o[l, j] >= V[l, h].min(axis=0) - 1e-14)
            # replacing every other head's values leaves this head's output alone
            V2 = V.copy()
            V2[:, [x for x in range(H) if x != h]] += 100.0
            V2[[x for x in range(L) if x != l]] += 100.0
            o2, _ = oatt.decode_attention(q, K, V2, 0.5)
            assert np.allclose(o2[l, j], o[l, j], atol=1e-13)
