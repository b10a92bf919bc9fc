"""Pins of the oracle's projection + norm + rotary (the step before the insert; vLLM M3.1
post, "QKV GEMM + norm + RoPE + KV insert fusion").  Each check ties the oracle to
something other than itself: a library matrix product, closed forms of the norm, the
rotation written as a complex product, and the relative-position property of rotary
embeddings."""
import numpy as np

import workload as W


def _decode_bf16(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def _inputs(n=5, hidden=256, seed=3, rope=None):
    q = W.make_qkv_inputs(seed, n, hidden, max_pos=64)
    if rope is not None:
        q.rope = rope
        q.positions = np.minimum(q.positions, rope.shape[0] - 1).astype(np.int32)
    return q


def test_bf16_decode(oracle):
    assert oracle.bf16_value(0x3F80) == 1.0
    assert oracle.bf16_value(0xC000) == -2.0
    assert oracle.bf16_value(0x0001) == 2.0 ** -133      # smallest subnormal
    assert oracle.bf16_value(0x7F80) == float("inf")
    assert oracle.bf16_value(0x4049) == 3.140625          # 1.1001001b x 2


def test_value_heads_are_the_matrix_product(oracle):
    """Values are stored as projected: heads 36..39 = x W^T (numpy float64 matmul)."""
    q = _inputs()
    out = oracle.qkv_project(q.x, q.w, q.norm_weight, q.eps, q.rope, q.positions)
    ref = _decode_bf16(q.x) @ _decode_bf16(q.w).T  # [n][45*128]
    got = out[:, 36:40, :].reshape(q.x.shape[0], -1)
    np.testing.assert_allclose(got, ref[:, 36 * 128:40 * 128].astype(np.float32), rtol=1e-6, atol=1e-6)


def _identity_rope(rows=4):
    return np.concatenate([np.ones((rows, 64)), np.zeros((rows, 64))], axis=1).astype(np.float32)


def test_rms_norm_closed_form(oracle):
    """With no rotation: a normalised head is h / sqrt(mean(h^2) + eps) * weight, so with a
    unit weight its mean square is ms / (ms + eps), and the weight scales it per dim."""
    q = _inputs(rope=_identity_rope())
    q.norm_weight[:] = 1.0
    q.eps = 0.25
    out = oracle.qkv_project(q.x, q.w, q.norm_weight, q.eps, q.rope, q.positions).astype(np.float64)
    h = _decode_bf16(q.x) @ _decode_bf16(q.w).T
    for hd in list(range(0, 36)) + list(range(40, 45)):
        ms = np.mean(h[:, hd * 128:(hd + 1) * 128] ** 2, axis=1)
        np.testing.assert_allclose(np.mean(out[:, hd] ** 2, axis=1), ms / (ms + q.eps), rtol=1e-5)
    g = np.linspace(0.5, 2.0, 128).astype(np.float32)
    q.norm_weight[1] = g  # keys only
    out2 = oracle.qkv_project(q.x, q.w, q.norm_weight, q.eps, q.rope, q.positions).astype(np.float64)
    np.testing.assert_allclose(out2[:, 32:36], out[:, 32:36] * g, rtol=1e-6, atol=1e-7)
    np.testing.assert_array_equal(out2[:, 0:32], out[:, 0:32])


def test_rotation_is_a_complex_product(oracle):
    """Rotate-half: (o_i + j o_{i+64}) = (y_i + j y_{i+64}) e^{j angle_i}, where y is the same
    token's head at a position whose table row is the identity."""
    rows = 3
    ang = np.random.default_rng(5).uniform(-np.pi, np.pi, size=(rows, 64))
    tab = np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)
    tab[0] = _identity_rope(1)[0]
    ang[0] = 0.0
    q = _inputs(n=1, rope=tab)
    for p in (1, 2):
        y = oracle.qkv_project(q.x, q.w, q.norm_weight, q.eps, tab, np.array([0], np.int32))[0].astype(np.float64)
        o = oracle.qkv_project(q.x, q.w, q.norm_weight, q.eps, tab, np.array([p], np.int32))[0].astype(np.float64)
        c = tab[p, :64].astype(np.float64) + 1j * tab[p, 64:].astype(np.float64)
        for hd in (0, 33, 40, 44):
            want = (y[hd, :64] + 1j * y[hd, 64:]) * c
            np.testing.assert_allclose(o[hd, :64], want.real, rtol=1e-5, atol=1e-6)
            np.testing.assert_allclose(o[hd, 64:], want.imag, rtol=1e-5, atol=1e-6)
        np.testing.assert_array_equal(o[36:40], y[36:40])  # values are not rotated


def test_scores_depend_on_relative_position(oracle):
    """Query-key products of rotated heads depend only on the position difference."""
    q = W.make_qkv_inputs(4, 2, 256, max_pos=200)
    def heads(pq, pk):
        o = oracle.qkv_project(q.x, q.w, q.norm_weight, q.eps, q.rope, np.array([pq, pk], np.int32))
        return o.astype(np.float64)
    a = heads(10, 3)
    b = heads(110, 103)
    for hq, hk in ((0, 32), (9, 33), (40, 44)):
        np.testing.assert_allclose(a[0, hq] @ a[1, hk], b[0, hq] @ b[1, hk], rtol=1e-4, atol=1e-5)
    c = heads(110, 3)
    assert abs(a[0, 0] @ a[1, 32] - c[0, 0] @ c[1, 32]) > 1e-3  # and they do depend on it


def test_position_outside_the_table_gives_no_row(oracle):
    q = W.make_qkv_inputs(6, 3, 256, max_pos=16, bad_positions=1)
    out = oracle.qkv_project(q.x, q.w, q.norm_weight, q.eps, q.rope, q.positions)
    assert np.isnan(out[0]).all() and np.isfinite(out[1:]).all()
