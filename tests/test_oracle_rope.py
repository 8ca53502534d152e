"""Pins of the oracle's 3D rotary position embedding (rope_3d, reading R10), from its mathematics:
a rotation keeps every pair's norm; the scores of rotated q and k depend only on the difference of
their positions along each axis; position 0 is the identity; a single pair turns by the textbook
angle in the stated direction."""
import numpy as np

from block_sparse_causal_lcsa_amd import workloads as W
from oracle import lcsa_oracle as O

P = W.Workload("rope", 1, 2, 16, 4, 6, 4, 0, 4, dtype="f32")
DIMS = (6, 4, 6)
THETA = 100.0


def rand(n, seed=0):
    return np.random.default_rng(seed).standard_normal((1, 2, n, 16))


def test_pair_norms_preserved():
    x = rand(4 * 24)
    y = O.rope_3d(P, x, 3, DIMS, THETA)
    nx = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    ny = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    np.testing.assert_allclose(ny, nx, rtol=1e-13)


def test_scores_depend_on_relative_position_only():
    # one q and one k vector placed at every token; shifting both by the same frame count (frame0)
    # or reading them one row / one column further leaves q.k unchanged
    rng = np.random.default_rng(1)
    qv, kv = rng.standard_normal(16), rng.standard_normal(16)
    n = 4 * 24
    q = np.broadcast_to(qv, (1, 1, n, 16)).copy()
    k = np.broadcast_to(kv, (1, 1, n, 16)).copy()
    p1 = P.replace(heads=1)
    rq0, rk0 = O.rope_3d(p1, q, 0, DIMS, THETA)[0, 0], O.rope_3d(p1, k, 0, DIMS, THETA)[0, 0]
    rq5, rk5 = O.rope_3d(p1, q, 5, DIMS, THETA)[0, 0], O.rope_3d(p1, k, 5, DIMS, THETA)[0, 0]
    tok = lambda t, h, w: (t * 4 + h) * 6 + w
    a, b = tok(0, 1, 2), tok(2, 0, 4)
    s = rq0[a] @ rk0[b]
    np.testing.assert_allclose(rq5[a] @ rk5[b], s, rtol=1e-12)                            # frames + 5
    np.testing.assert_allclose(rq0[tok(1, 2, 2)] @ rk0[tok(3, 1, 4)], s, rtol=1e-12)      # frame + 1, row + 1
    np.testing.assert_allclose(rq0[tok(0, 1, 3)] @ rk0[tok(2, 0, 5)], s, rtol=1e-12)      # column + 1
    assert not np.isclose(rq0[tok(0, 1, 3)] @ rk0[b], s)                                 # q moved alone


def test_position_zero_is_identity():
    x = rand(24, 2)
    y = O.rope_3d(P, x, 0, DIMS, THETA)
    np.testing.assert_array_equal(y[:, :, 0], x[:, :, 0])   # token 0: frame 0, row 0, column 0


def test_single_pair_closed_form():
    p = P.replace(heads=1, head_dim=6, grid_h=1, grid_w=3)
    x = np.zeros((1, 1, 3, 6))
    x[..., 4] = 1.0                                 # first pair of the w group, at columns 0, 1, 2
    y = O.rope_3d(p, x, 0, (2, 2, 2), 10.0)         # frequency theta^0 = 1: turn by w radians
    for w in range(3):
        np.testing.assert_allclose(y[0, 0, w, 4:6], [np.cos(w), np.sin(w)], atol=1e-15)
        np.testing.assert_array_equal(y[0, 0, w, :4], 0.0)
    x2 = np.zeros((1, 1, 3, 6))
    x2[..., 0:2] = [0.0, 1.0]                       # the t pair at frame 3: (0, 1) -> (-sin 3, cos 3)
    y2 = O.rope_3d(p, x2, 3, (2, 2, 2), 10.0)
    np.testing.assert_allclose(y2[0, 0, 1, 0:2], [-np.sin(3), np.cos(3)], atol=1e-15)


def test_frequency_schedule_exact_angles():
    """Every pair of every axis group, not only the first: with theta = 256 and 8 dims per axis the
    four pairs of a group rotate at 1, 1/4, 1/16 and 1/64 radians per position step (theta raised to
    minus twice the pair index over the group width), so pair j at position 4^j has turned by exactly
    one radian and at position 2 * 4^j by two; every other pair of the token is turned by another
    angle. A schedule with another exponent (pair index over the width, or counting pairs from one)
    moves these angles and fails here."""
    theta, dims = 256.0, (8, 8, 8)
    unit = np.zeros((1, 1, 1, 24))
    for axis, g0 in (("t", 0), ("h", 8), ("w", 16)):
        for j in range(4):
            for turns in (1, 2):
                pos = turns * 4 ** j
                x = np.zeros(24)
                x[g0 + 2 * j] = 1.0                       # (1, 0) in pair j of this axis group
                if axis == "t":                           # a 1x1 grid at absolute frame pos
                    p = P.replace(heads=1, head_dim=24, grid_h=1, grid_w=1)
                    y = O.rope_3d(p, unit + x, pos, dims, theta)[0, 0, 0]
                elif axis == "h":                         # a column of pos + 1 rows, token at row pos
                    p = P.replace(heads=1, head_dim=24, grid_h=pos + 1, grid_w=1)
                    y = O.rope_3d(p, np.broadcast_to(x, (1, 1, pos + 1, 24)).copy(), 0, dims, theta)[0, 0, pos]
                else:                                     # a row of pos + 1 columns, token at column pos
                    p = P.replace(heads=1, head_dim=24, grid_h=1, grid_w=pos + 1)
                    y = O.rope_3d(p, np.broadcast_to(x, (1, 1, pos + 1, 24)).copy(), 0, dims, theta)[0, 0, pos]
                want = np.zeros(24)
                want[g0 + 2 * j: g0 + 2 * j + 2] = [np.cos(turns), np.sin(turns)]
                np.testing.assert_allclose(y, want, atol=1e-12, err_msg=f"axis {axis} pair {j} position {pos}")
