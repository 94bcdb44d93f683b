"""CPU pins of the float64 oracle.

Each test fixes the oracle against something other than itself: an
independent scalar-loop spelling, a closed form worked by hand, a library
routine in a special case that reduces to it, or an invariant of the
mathematics (permutation equivariance, the transpose relation between the two
directions, mask semantics, additivity of tile partial sums).  The pages print
no numeric example for this layer, so nothing here comes from the pages'
numbers.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import bruteforce
from oracle.trimul_ref import array_getters
import workloads as wl

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def rand_weights(c_z, c, seed, random_ln=True):
    """float64 weights for oracle-only tests (not tied to a storage dtype)."""
    r = np.random.default_rng(seed)
    w = {
        "w_a_proj": r.standard_normal((c, c_z)) / math.sqrt(c_z),
        "w_a_gate": r.standard_normal((c, c_z)) / math.sqrt(c_z),
        "w_b_proj": r.standard_normal((c, c_z)) / math.sqrt(c_z),
        "w_b_gate": r.standard_normal((c, c_z)) / math.sqrt(c_z),
        "w_out_gate": r.standard_normal((c_z, c_z)) / math.sqrt(c_z),
        "w_out_proj": r.standard_normal((c_z, c)) / math.sqrt(c),
        "ln_in_w": 1 + 0.1 * r.standard_normal(c_z) if random_ln else np.ones(c_z),
        "ln_in_b": 0.1 * r.standard_normal(c_z) if random_ln else np.zeros(c_z),
        "ln_out_w": 1 + 0.1 * r.standard_normal(c) if random_ln else np.ones(c),
        "ln_out_b": 0.1 * r.standard_normal(c) if random_ln else np.zeros(c),
    }
    return w


def rand_inputs(n, c_z, seed, keep=0.8):
    r = np.random.default_rng(seed + 1000)
    z = r.standard_normal((n, n, c_z))
    m = (r.random((n, n)) < keep).astype(np.uint8)
    return z, m


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.max(np.abs(a - b)) / max(np.sqrt(np.mean(b * b)), 1e-300)


# ---------------------------------------------------------------------------
# elementary pieces
# ---------------------------------------------------------------------------

def test_bf16_round_properties():
    r = np.random.default_rng(0)
    x = r.standard_normal(20000) * np.exp2(r.integers(-30, 30, 20000))
    q = oracle.bf16_round(x)
    # representable: a float32 whose low 16 bits are zero
    q32 = q.astype(np.float32)
    assert np.all(q32.astype(np.float64) == q)
    assert np.all((q32.view(np.uint32) & 0xFFFF) == 0)
    # nearest: no bf16 neighbour is closer
    bits = q32.view(np.uint32)
    up = ((bits + 0x10000) & 0xFFFFFFFF).astype(np.uint32).view(np.float32).astype(np.float64)
    dn = ((bits - 0x10000) & 0xFFFFFFFF).astype(np.uint32).view(np.float32).astype(np.float64)
    err = np.abs(x - q)
    assert np.all(err <= np.abs(x - up))
    assert np.all(err <= np.abs(x - dn))


def test_bf16_round_ties_and_specials():
    one = 1.0
    ulp = 2.0 ** -7                      # bf16 spacing in [1, 2)
    assert oracle.bf16_round(one + ulp / 2) == one                  # tie -> even (1.0)
    assert oracle.bf16_round(one + 1.5 * ulp) == one + 2 * ulp      # tie -> even mantissa
    assert oracle.bf16_round(one + ulp / 2 + 2.0 ** -40) == one + ulp
    assert oracle.bf16_round(-(one + ulp / 2)) == -one
    assert oracle.bf16_round(0.0) == 0.0
    assert oracle.bf16_round(2.0 ** -133) == 2.0 ** -133            # smallest subnormal
    assert oracle.bf16_round(3.4e38) == np.inf                      # beyond max finite
    assert np.isnan(oracle.bf16_round(np.nan))


def test_bf16_round_matches_torch_on_float32_inputs():
    # torch rounds float32 -> bfloat16 to nearest-even; on float32-exact inputs the
    # one-step float64 rounding must agree with it.
    x = np.random.default_rng(1).standard_normal(50000).astype(np.float32)
    t = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.bf16_round(x.astype(np.float64)), t)


def test_sigmoid():
    t = np.linspace(-30, 30, 601)
    ref = np.array([1.0 / (1.0 + math.exp(-v)) for v in t])
    assert np.max(np.abs(oracle.sigmoid(t) - ref)) < 1e-15
    assert oracle.sigmoid(0.0) == 0.5
    assert oracle.sigmoid(-1000.0) == 0.0 and oracle.sigmoid(1000.0) == 1.0
    assert np.allclose(oracle.sigmoid(t) + oracle.sigmoid(-t), 1.0, atol=1e-15)


def test_layer_norm_closed_form():
    v = np.array([1.0, 2.0, 3.0, 4.0])
    # mean 2.5, biased variance 1.25
    want = (v - 2.5) / math.sqrt(1.25 + 1e-5)
    got = oracle.layer_norm(v, np.ones(4), np.zeros(4))
    assert np.max(np.abs(got - want)) < 1e-15
    g = np.array([2.0, -1.0, 0.5, 3.0])
    b = np.array([0.1, 0.2, 0.3, 0.4])
    assert np.max(np.abs(oracle.layer_norm(v, g, b) - (want * g + b))) < 1e-15
    # constant vector: zero deviation, the eps branch returns beta exactly
    assert np.array_equal(oracle.layer_norm(np.full(4, 7.0), g, b), b)
    # shift invariance
    r = np.random.default_rng(2).standard_normal((5, 16))
    assert np.max(np.abs(oracle.layer_norm(r + 3.25, np.ones(16), np.zeros(16))
                         - oracle.layer_norm(r, np.ones(16), np.zeros(16)))) < 1e-13


def test_gate_half_and_identity_projection():
    c = 8
    z, m = rand_inputs(3, c, 5, keep=1.0)
    w = rand_weights(c, c, 5)
    w["w_a_gate"][:] = 0
    w["w_b_gate"][:] = 0
    w["w_a_proj"] = np.eye(c)
    w["w_b_proj"] = 2 * np.eye(c)
    a, b = oracle.project(z, m, w)
    zh = oracle.layer_norm(z, w["ln_in_w"], w["ln_in_b"])
    assert np.max(np.abs(a - 0.5 * zh)) < 1e-15
    assert np.max(np.abs(b - zh)) < 1e-15


# ---------------------------------------------------------------------------
# whole definition vs the scalar-loop spelling
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
@pytest.mark.parametrize("n,c_z,c", [(1, 4, 4), (2, 4, 8), (3, 8, 4), (5, 6, 4), (6, 8, 8)])
def test_vectorised_matches_bruteforce_small(direction, n, c_z, c):
    w = rand_weights(c_z, c, 10 + n)
    z, m = rand_inputs(n, c_z, 20 + n, keep=0.75)
    got = oracle.trimul(z, m, w, direction)
    want = np.array(bruteforce.trimul_loops(z.tolist(), m.tolist(), w, direction))
    assert rel(got, want) < 1e-12


@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
def test_vectorised_matches_bruteforce_full_width(direction):
    n, c_z, c = 4, 128, 128
    w = rand_weights(c_z, c, 33)
    z, m = rand_inputs(n, c_z, 34, keep=0.8)
    got = oracle.trimul(z, m, w, direction)
    want = np.array(bruteforce.trimul_loops(z.tolist(), m.tolist(), w, direction))
    assert rel(got, want) < 1e-12


def test_hand_worked_example_c2():
    """c_z = c = 2 worked by hand.

    With two channels, LN(p, q) = sign(p - q) * s * (1, -1) for
    s = h / sqrt(h^2 + eps), h = |p - q| / 2 (gamma = 1, beta = 0).  With
    W_ag = W_bg = 0 (gates 1/2), W_ap = diag(1, 2), W_bp = I, the operands are
    a = zh * (1/2, 1), b = zh / 2, so outgoing x_ij = (T_ij / 4) * (1, 2) with
    T_ij = sum_k u_ik u_jk, u = sign * s.  LN of (t, 2t) is
    sign(t) * r * (-1, 1), r = (|t|/2) / sqrt(t^2/4 + eps).  With W_o = I,
    W_g = 0 (gate 1/2) and mask 1: out_ij = (1/2) * sign(T) * r(T/4) * (-1, 1).
    """
    eps = 1e-5
    p = np.array([[0.3, -1.2], [2.0, 0.7]])
    q = np.array([[1.1, 0.4], [-0.5, 0.7 + 1e-3]])
    z = np.stack([p, q], axis=-1)
    m = np.ones((2, 2), np.uint8)
    w = {
        "w_a_proj": np.diag([1.0, 2.0]), "w_a_gate": np.zeros((2, 2)),
        "w_b_proj": np.eye(2), "w_b_gate": np.zeros((2, 2)),
        "w_out_gate": np.zeros((2, 2)), "w_out_proj": np.eye(2),
        "ln_in_w": np.ones(2), "ln_in_b": np.zeros(2),
        "ln_out_w": np.ones(2), "ln_out_b": np.zeros(2),
    }
    u = np.zeros((2, 2))
    for i in range(2):
        for j in range(2):
            h = abs(p[i, j] - q[i, j]) / 2
            u[i, j] = math.copysign(h / math.sqrt(h * h + eps), p[i, j] - q[i, j])
    want = np.zeros((2, 2, 2))
    for i in range(2):
        for j in range(2):
            T = u[i, 0] * u[j, 0] + u[i, 1] * u[j, 1]
            t = T / 4
            r = (abs(t) / 2) / math.sqrt(t * t / 4 + eps)
            want[i, j] = 0.5 * math.copysign(r, t) * np.array([-1.0, 1.0])
    got = oracle.trimul(z, m, w, "outgoing")
    assert np.max(np.abs(got - want)) < 1e-13


# ---------------------------------------------------------------------------
# special cases that reduce to a library routine
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
def test_contraction_reduces_to_gram_matmul(direction):
    """Gates 0 (sigma = 1/2), identity projections, mask 1: a = b = zh / 2, so
    outgoing X_d = Zh_d Zh_d^T / 4 and incoming X_d = Zh_d^T Zh_d / 4 (torch.bmm)."""
    n, c = 7, 16
    w = rand_weights(c, c, 41)
    for k in ("w_a_gate", "w_b_gate"):
        w[k][:] = 0
    w["w_a_proj"] = np.eye(c)
    w["w_b_proj"] = np.eye(c)
    z, _ = rand_inputs(n, c, 42)
    m = np.ones((n, n), np.uint8)
    _, x = oracle.trimul(z, m, w, direction, return_x=True)
    zh = torch.from_numpy(oracle.layer_norm(z, w["ln_in_w"], w["ln_in_b"])).permute(2, 0, 1)
    if direction == "outgoing":
        X = torch.bmm(zh, zh.transpose(1, 2).contiguous()) / 4
    else:
        X = torch.bmm(zh.transpose(1, 2).contiguous(), zh) / 4
    assert rel(x, X.permute(1, 2, 0).numpy()) < 1e-13


def test_single_k_mask_gives_outer_product():
    """Pair mask m_ik = [k == k0] leaves one term: x_ij = a_ik0 * b_jk0."""
    n, c_z, c, k0 = 6, 8, 8, 2
    w = rand_weights(c_z, c, 51)
    z, _ = rand_inputs(n, c_z, 52)
    m = np.zeros((n, n), np.uint8)
    m[:, k0] = 1
    _, x = oracle.trimul(z, m, w, "outgoing", return_x=True)
    a, b = oracle.project(z, np.ones((n, n)), w)
    want = a[:, k0, None, :] * b[None, :, k0, :]
    assert rel(x, want) < 1e-13


def test_tied_weights_gram_is_psd():
    n, c = 9, 8
    w = rand_weights(c, c, 61)
    w["w_b_proj"] = w["w_a_proj"].copy()
    w["w_b_gate"] = w["w_a_gate"].copy()
    z, m = rand_inputs(n, c, 62, keep=0.9)
    _, x = oracle.trimul(z, m, w, "outgoing", return_x=True)
    for d in range(c):
        X = x[:, :, d]
        assert np.max(np.abs(X - X.T)) < 1e-13
        assert np.min(np.linalg.eigvalsh((X + X.T) / 2)) > -1e-12


def test_n1():
    c_z, c = 8, 8
    w = rand_weights(c_z, c, 71)
    z, _ = rand_inputs(1, c_z, 72)
    m = np.ones((1, 1), np.uint8)
    o_out, x_out = oracle.trimul(z, m, w, "outgoing", return_x=True)
    o_in, x_in = oracle.trimul(z, m, w, "incoming", return_x=True)
    a, b = oracle.project(z, m, w)
    assert np.max(np.abs(x_out[0, 0] - a[0, 0] * b[0, 0])) < 1e-15
    assert np.array_equal(o_out, o_in)


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
def test_permutation_equivariance(direction):
    n, c_z, c = 11, 8, 8
    w = rand_weights(c_z, c, 81)
    z, m = rand_inputs(n, c_z, 82, keep=0.8)
    perm = np.random.default_rng(83).permutation(n)
    out = oracle.trimul(z, m, w, direction)
    out_p = oracle.trimul(z[np.ix_(perm, perm)], m[np.ix_(perm, perm)], w, direction)
    assert rel(out_p, out[np.ix_(perm, perm)]) < 1e-12


def test_transpose_relation_between_directions():
    """incoming(z, m; W) = outgoing(z^T, m^T; W with a <-> b swapped)^T.  The
    literal 'same weights' form holds only when the a and b weights are tied."""
    n, c_z, c = 10, 8, 8
    w = rand_weights(c_z, c, 91)
    z, m = rand_inputs(n, c_z, 92, keep=0.85)
    zt = np.swapaxes(z, 0, 1)
    mt = m.T
    inc = oracle.trimul(z, m, w, "incoming")
    ws = dict(w)
    ws["w_a_proj"], ws["w_b_proj"] = w["w_b_proj"], w["w_a_proj"]
    ws["w_a_gate"], ws["w_b_gate"] = w["w_b_gate"], w["w_a_gate"]
    assert rel(inc, np.swapaxes(oracle.trimul(zt, mt, ws, "outgoing"), 0, 1)) < 1e-12
    # untied, unswapped: genuinely different
    assert rel(inc, np.swapaxes(oracle.trimul(zt, mt, w, "outgoing"), 0, 1)) > 1e-3
    wt = dict(w)
    wt["w_b_proj"], wt["w_b_gate"] = w["w_a_proj"], w["w_a_gate"]
    assert rel(oracle.trimul(z, m, wt, "incoming"),
               np.swapaxes(oracle.trimul(zt, mt, wt, "outgoing"), 0, 1)) < 1e-12


@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
def test_masked_pairs_contribute_nothing(direction):
    n, c_z, c = 9, 8, 8
    w = rand_weights(c_z, c, 101)
    z, m = rand_inputs(n, c_z, 102, keep=0.7)
    out = oracle.trimul(z, m, w, direction)
    assert np.all(out[m == 0] == 0)
    z2 = z.copy()
    z2[m == 0] = np.random.default_rng(103).standard_normal(z2[m == 0].shape) * 50
    assert np.array_equal(oracle.trimul(z2, m, w, direction), out)
    assert np.all(oracle.trimul(z, np.zeros_like(m), w, direction) == 0)


@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
def test_tile_partials_sum_to_full(direction):
    n, c_z, c = 12, 8, 8
    w = rand_weights(c_z, c, 111)
    z, m = rand_inputs(n, c_z, 112, keep=0.85)
    gz, gm = array_getters(z, m)
    _, x = oracle.trimul(z, m, w, direction, return_x=True)
    out = oracle.trimul(z, m, w, direction)
    h = n // 2
    chunks = [np.arange(t * 3, t * 3 + 3) for t in range(4)]
    for r0 in (0, h):
        for c0 in (0, h):
            rows, cols = np.arange(r0, r0 + h), np.arange(c0, c0 + h)
            parts = [oracle.tile_partial(gz, gm, n, w, direction, rows, cols, k) for k in chunks]
            ring = sum(parts)
            rotated = sum(parts[2:] + parts[:2])
            assert np.max(np.abs(ring - x[r0:r0 + h, c0:c0 + h])) < 1e-13
            assert np.max(np.abs(rotated - ring)) < 1e-13
            fin = oracle.finish(ring, z[r0:r0 + h, c0:c0 + h], m[r0:r0 + h, c0:c0 + h], w)
            assert np.max(np.abs(fin - out[r0:r0 + h, c0:c0 + h])) < 1e-13


@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
def test_sampled_and_blockwise_match_full(direction):
    n, c_z, c = 20, 8, 8
    w = rand_weights(c_z, c, 121)
    z, m = rand_inputs(n, c_z, 122, keep=0.9)
    out = oracle.trimul(z, m, w, direction)
    rows = np.array([0, 3, 19, 7])
    cols = np.array([19, 0, 5])
    gz, gm = array_getters(z, m)
    s = oracle.trimul_sampled(gz, gm, n, w, direction, rows, cols)
    assert np.max(np.abs(s - out[np.ix_(rows, cols)])) < 1e-13
    assert np.max(np.abs(oracle.trimul_blockwise(z, m, w, direction, block=6) - out)) < 1e-13


# ---------------------------------------------------------------------------
# Q-mode (bf16 contraction operands)
# ---------------------------------------------------------------------------

def test_qmode_operands_are_bf16_and_contract_exactly():
    n, c_z, c = 6, 16, 8
    w = rand_weights(c_z, c, 131)
    z, m = rand_inputs(n, c_z, 132, keep=0.8)
    a, b = oracle.project(z, m, w, quant=True)
    for t in (a, b):
        assert np.array_equal(t.astype(np.float32).astype(np.float64), t)
        assert np.all((t.astype(np.float32).view(np.uint32) & 0xFFFF) == 0)
    _, xq = oracle.trimul(z, m, w, "outgoing", quant=True, return_x=True)
    # contraction of the rounded operands, by explicit loops
    want = np.zeros((n, n, c))
    for i in range(n):
        for j in range(n):
            for k in range(n):
                want[i, j] += a[i, k] * b[j, k]
    assert np.max(np.abs(xq - want)) < 1e-13


def test_qmode_is_close_to_but_not_exact():
    wts = wl.make_weights(128, 128, seed=3, dtype="bf16")
    w = wl.weights_f64(wts)
    z = wl.make_pair_tensor(48, 128, 3, "bf16", "cpu").double().numpy()
    m = np.ones((48, 48), np.uint8)
    ex = oracle.trimul(z, m, w, "outgoing")
    q = oracle.trimul(z, m, w, "outgoing", quant=True)
    e = rel(q, ex)
    assert 1e-4 < e < 6e-2


def test_bf16_nearest_agrees_with_oracle_rounding():
    """The scalar-loop rounding (math.frexp + round) and the oracle's
    vectorised one (frexp + rint) agree on normal values, exact ties, values
    one float64 step either side of a tie, subnormals and overflow."""
    r = np.random.default_rng(140)
    vals = list(r.standard_normal(2000) * np.exp2(r.integers(-40, 40, 2000)))
    for k in range(1, 300):                      # ties between neighbours 1 + (k-1)/128 and 1 + k/128
        t = 1.0 + (2 * k - 1) / 256.0
        vals += [t, -t, np.nextafter(t, 0.0), np.nextafter(t, 9.0), t * 2.0 ** -130]
    vals += [0.0, -0.0, 2.0 ** -140, 3 * 2.0 ** -134, 1e-45, (2 - 2 ** -8) * 2.0 ** 127, 3.4e38, 1e39]
    got = np.array([bruteforce.bf16_nearest(float(v)) for v in vals])
    assert np.array_equal(got, oracle.bf16_round(np.array(vals)))


@pytest.mark.parametrize("n,c_z,c", [(3, 8, 4), (2, 128, 128)])
def test_qmode_project_matches_loops(n, c_z, c):
    """Q-mode operands equal the scalar-loop spelling's exactly: zh rounded
    after its affine map, a and b rounded when finished."""
    w = rand_weights(c_z, c, 141 + n)
    z, m = rand_inputs(n, c_z, 142 + n, keep=0.8)
    a, b = oracle.project(z, m, w, quant=True)
    la, lb = bruteforce.project_loops(z.tolist(), m.tolist(), w, quant=True)
    assert np.array_equal(a, np.array(la)) and np.array_equal(b, np.array(lb))
    # and the rounding matters at these sizes: the exact operands differ
    ea, _ = oracle.project(z, m, w)
    assert np.max(np.abs(ea - a)) > 0


@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
def test_qmode_trimul_matches_loops(direction):
    n, c_z, c = 4, 8, 8
    w = rand_weights(c_z, c, 150)
    z, m = rand_inputs(n, c_z, 151, keep=0.8)
    got = oracle.trimul(z, m, w, direction, quant=True)
    want = np.array(bruteforce.trimul_loops(z.tolist(), m.tolist(), w, direction, quant=True))
    assert rel(got, want) < 1e-12


def test_qmode_rounding_point_worked_by_hand():
    """One pair, c_z = 4, c = 2, worked by hand.  z = (-3, -1, 1, 3) has mean 0
    and biased variance 5, so LN gives zhh = z / sqrt(5 + 1e-5), i.e.
    zhh_0 = -1.3416394..., zhh_3 = 1.3416394...  The gates are zero
    (sigmoid = 1/2) and W_ap picks 3 * channel 0 (row 0) and 3 * channel 3
    (row 1), so a_d = 1.5 * zh.

    Channel 0, gamma 1.3, beta 0.5: zh_0 = 1.3 * zhh_0 + 0.5 = -1.2441313.
    bf16 spacing on [1, 2) is 2^-7: -1.2441313 * 128 = -159.25 -> -159, so
    bf16(zh_0) = -1.2421875 and a_0 = 1.5 * -1.2421875 = -1.86328125 =
    -238.5 * 2^-7, an exact tie -> even -238 -> a_0 = -1.859375.
    Dropping the zh rounding gives 1.5 * -1.2441313 = -1.8661969 -> -238.87 ->
    a_0 = -1.8671875; rounding before the affine map gives
    1.5 * (1.3 * bf16(-1.3416394) + 0.5) = 1.5 * (1.3 * -1.34375 + 0.5) =
    -1.8703125 -> -239.4 -> -1.8671875.

    Channel 3, gamma 1.25, beta 0.5: zh_3 = 2.1770493; spacing on [2, 4) is
    2^-6: 139.33 -> 139 -> 2.171875; a_1 = 1.5 * 2.171875 = 3.2578125 =
    208.5 * 2^-6, a tie -> even 208 -> 3.25.  Without the zh rounding:
    3.2655740 -> 208.997 -> 3.265625; rounding before the affine map:
    1.5 * (1.25 * 1.34375 + 0.5) = 3.26953125 -> 209.25 -> 3.265625.
    """
    c_z, c = 4, 2
    w = {
        "w_a_proj": np.array([[3.0, 0, 0, 0], [0, 0, 0, 3.0]]), "w_a_gate": np.zeros((c, c_z)),
        "w_b_proj": np.zeros((c, c_z)), "w_b_gate": np.zeros((c, c_z)),
        "w_out_gate": np.zeros((c_z, c_z)), "w_out_proj": np.zeros((c_z, c)),
        "ln_in_w": np.array([1.3, 1.0, 1.0, 1.25]), "ln_in_b": np.array([0.5, 0.0, 0.0, 0.5]),
        "ln_out_w": np.ones(c), "ln_out_b": np.zeros(c),
    }
    z = np.array([[[-3.0, -1.0, 1.0, 3.0]]])
    m = np.ones((1, 1), np.uint8)
    a, _ = oracle.project(z, m, w, quant=True)
    assert a[0, 0, 0] == -1.859375 and a[0, 0, 1] == 3.25
    la, _ = bruteforce.project_loops(z.tolist(), m.tolist(), w, quant=True)
    assert la[0][0] == [-1.859375, 3.25]
    # the unrounded operands, for contrast
    a_exact, _ = oracle.project(z, m, w)
    assert oracle.bf16_round(a_exact)[0, 0].tolist() == [-1.8671875, 3.265625]


@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
def test_qmode_sampled_and_blockwise_match_full(direction):
    n, c_z, c = 20, 8, 4
    w = rand_weights(c_z, c, 160)
    z, m = rand_inputs(n, c_z, 161, keep=0.9)
    out = oracle.trimul(z, m, w, direction, quant=True)
    rows, cols = np.array([0, 4, 19, 11]), np.array([19, 0, 7])
    gz, gm = array_getters(z, m)
    s = oracle.trimul_sampled(gz, gm, n, w, direction, rows, cols, quant=True)
    assert np.max(np.abs(s - out[np.ix_(rows, cols)])) < 1e-13
    assert np.max(np.abs(oracle.trimul_blockwise(z, m, w, direction, quant=True, block=6) - out)) < 1e-13


# ---------------------------------------------------------------------------
# stored regression fixture (written by tests/golden/make_golden.py from the
# brute-force loops only)
# ---------------------------------------------------------------------------

def test_golden_fixture():
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "trimul_n4_c6.json")
    g = json.load(open(path))
    w = {k: np.array(v) for k, v in g["weights"].items()}
    z = np.array(g["z"])
    m = np.array(g["mask"], np.uint8)
    for d in ("outgoing", "incoming"):
        assert rel(oracle.trimul(z, m, w, d), np.array(g["out_" + d])) < 1e-12


# ---------------------------------------------------------------------------
# gradients of the contraction step (backward pass): pinned by the
# bilinearity identity, finite differences, scalar loops and one-hot inputs
# ---------------------------------------------------------------------------

def _vjp_case(seed, mi=5, mj=4, k=6, c=3):
    r = np.random.default_rng(seed)
    return (r.standard_normal((mi, k, c)), r.standard_normal((mj, k, c)), r.standard_normal((mi, mj, c)))


def test_contract_vjp_bilinearity():
    # x is linear in each operand, so <dx, x(a, b)> = <da, a> = <db, b>
    a, b, dx = _vjp_case(1)
    da, db = oracle.contract_rows_vjp(a, b, dx)
    L = float(np.sum(dx * oracle.contract_rows(a, b)))
    assert abs(float(np.sum(da * a)) - L) <= 1e-12 * abs(L) + 1e-12
    assert abs(float(np.sum(db * b)) - L) <= 1e-12 * abs(L) + 1e-12
    assert da.shape == a.shape and db.shape == b.shape


def test_contract_vjp_finite_differences():
    # L(a + h v) - L(a - h v) = 2 h <da, v> exactly for a linear L (up to rounding)
    a, b, dx = _vjp_case(2)
    da, db = oracle.contract_rows_vjp(a, b, dx)
    r = np.random.default_rng(3)
    L = lambda a_, b_: float(np.sum(dx * oracle.contract_rows(a_, b_)))
    for _ in range(3):
        v = r.standard_normal(a.shape)
        h = 1e-3
        fd = (L(a + h * v, b) - L(a - h * v, b)) / (2 * h)
        assert abs(fd - float(np.sum(da * v))) < 1e-9 * (1 + abs(fd))
        u = r.standard_normal(b.shape)
        fd = (L(a, b + h * u) - L(a, b - h * u)) / (2 * h)
        assert abs(fd - float(np.sum(db * u))) < 1e-9 * (1 + abs(fd))


def test_contract_vjp_matches_loops():
    a, b, dx = _vjp_case(4, mi=3, mj=4, k=5, c=2)
    da, db = oracle.contract_rows_vjp(a, b, dx)
    la, lb = bruteforce.contract_vjp_loops(a.tolist(), b.tolist(), dx.tolist())
    assert np.max(np.abs(da - np.array(la))) < 1e-12
    assert np.max(np.abs(db - np.array(lb))) < 1e-12


def test_contract_vjp_one_hot():
    # dx = e_(i0, j0, d0): da is row j0 of b in channel d0, placed at row i0;
    # db is row i0 of a, placed at row j0
    a, b, _ = _vjp_case(5)
    dx = np.zeros((a.shape[0], b.shape[0], a.shape[2]))
    i0, j0, d0 = 3, 1, 2
    dx[i0, j0, d0] = 1.0
    da, db = oracle.contract_rows_vjp(a, b, dx)
    ea = np.zeros_like(a); ea[i0, :, d0] = b[j0, :, d0]
    eb = np.zeros_like(b); eb[j0, :, d0] = a[i0, :, d0]
    assert np.array_equal(da, ea) and np.array_equal(db, eb)


# ---------------------------------------------------------------------------
# gradients of the epilogue: pinned by central finite differences of
# oracle.finish, closed-form special cases and the LayerNorm shift invariance
# ---------------------------------------------------------------------------

def _epi_case(seed, p=6, c=5, cz=7, keep=0.7):
    r = np.random.default_rng(seed)
    w = {"ln_out_w": 1 + 0.3 * r.standard_normal(c), "ln_out_b": 0.2 * r.standard_normal(c),
         "ln_in_w": 1 + 0.3 * r.standard_normal(cz), "ln_in_b": 0.2 * r.standard_normal(cz),
         "w_out_proj": r.standard_normal((cz, c)) / np.sqrt(c), "w_out_gate": r.standard_normal((cz, cz)) / np.sqrt(cz)}
    x = r.standard_normal((p, c)) * 2 + 0.5
    z = r.standard_normal((p, cz))
    m = (r.random(p) < keep).astype(np.uint8)
    m[0] = 1
    dout = r.standard_normal((p, cz))
    return x, z, m, w, dout


def test_finish_vjp_finite_differences():
    x, z, m, w, dout = _epi_case(21)
    g = oracle.finish_vjp(x, z, m, w, dout)
    L = lambda x_, z_, w_: float(np.sum(dout * oracle.finish(x_, z_, m, w_)))
    r = np.random.default_rng(22)
    h = 1e-5
    for name in ("x", "z"):
        v = r.standard_normal(x.shape if name == "x" else z.shape)
        if name == "x":
            fd = (L(x + h * v, z, w) - L(x - h * v, z, w)) / (2 * h)
        else:
            fd = (L(x, z + h * v, w) - L(x, z - h * v, w)) / (2 * h)
        assert abs(fd - float(np.sum(g[name] * v))) < 1e-7 * (1 + abs(fd)), name
    for key in ("w_out_proj", "w_out_gate", "ln_out_w", "ln_out_b", "ln_in_w", "ln_in_b"):
        v = r.standard_normal(np.shape(w[key]))
        wp = dict(w); wp[key] = w[key] + h * v
        wm = dict(w); wm[key] = w[key] - h * v
        fd = (L(x, z, wp) - L(x, z, wm)) / (2 * h)
        assert abs(fd - float(np.sum(g[key] * v))) < 1e-7 * (1 + abs(fd)), key


def test_finish_vjp_special_cases():
    x, z, m, w, dout = _epi_case(23)
    # LayerNorm removes a common shift, so each pair's input gradients sum to 0
    g = oracle.finish_vjp(x, z, m, w, dout)
    assert np.max(np.abs(g["x"].sum(axis=-1))) < 1e-12
    assert np.max(np.abs(g["z"].sum(axis=-1))) < 1e-12
    # all pairs masked: the output is identically 0, so is every gradient
    g0 = oracle.finish_vjp(x, z, np.zeros_like(m), w, dout)
    assert all(np.max(np.abs(v)) == 0 for v in g0.values())
    # gamma_out = 0: the output does not depend on x
    w1 = dict(w); w1["ln_out_w"] = np.zeros_like(w["ln_out_w"])
    assert np.max(np.abs(oracle.finish_vjp(x, z, m, w1, dout)["x"])) == 0
    # W_g = 0: sigmoid = 1/2, so d/dW_o = sum 0.5 m dout (x) n and dz = 0
    w2 = dict(w); w2["w_out_gate"] = np.zeros_like(w["w_out_gate"])
    g2 = oracle.finish_vjp(x, z, m, w2, dout)
    n = oracle.layer_norm(x, w["ln_out_w"], w["ln_out_b"])
    want = (0.5 * m[:, None] * dout).T @ n
    assert np.max(np.abs(g2["w_out_proj"] - want)) < 1e-12
    assert np.max(np.abs(g2["z"])) == 0


def _proj_case(seed, p=6, c=5, cz=7, keep=0.7):
    r = np.random.default_rng(seed)
    w = {"ln_in_w": 1 + 0.3 * r.standard_normal(cz), "ln_in_b": 0.2 * r.standard_normal(cz)}
    for k in ("w_a_proj", "w_a_gate", "w_b_proj", "w_b_gate"):
        w[k] = r.standard_normal((c, cz)) / np.sqrt(cz)
    z = r.standard_normal((p, cz)) * 1.5 + 0.3
    m = (r.random(p) < keep).astype(np.uint8)
    m[0] = 1
    da = r.standard_normal((p, c))
    db = r.standard_normal((p, c))
    return z, m, w, da, db


def test_project_vjp_finite_differences():
    z, m, w, da, db = _proj_case(31)
    g = oracle.project_vjp(z, m, w, da, db)

    def L(z_, w_):
        a, b = oracle.project(z_, m, w_)
        return float(np.sum(da * a) + np.sum(db * b))

    r = np.random.default_rng(32)
    h = 1e-5
    v = r.standard_normal(z.shape)
    fd = (L(z + h * v, w) - L(z - h * v, w)) / (2 * h)
    assert abs(fd - float(np.sum(g["z"] * v))) < 1e-7 * (1 + abs(fd))
    for key in ("w_a_proj", "w_a_gate", "w_b_proj", "w_b_gate", "ln_in_w", "ln_in_b"):
        v = r.standard_normal(np.shape(w[key]))
        wp = dict(w); wp[key] = w[key] + h * v
        wm = dict(w); wm[key] = w[key] - h * v
        fd = (L(z, wp) - L(z, wm)) / (2 * h)
        assert abs(fd - float(np.sum(g[key] * v))) < 1e-7 * (1 + abs(fd)), key


def test_project_vjp_special_cases():
    z, m, w, da, db = _proj_case(33)
    g = oracle.project_vjp(z, m, w, da, db)
    # the input LayerNorm removes a common shift: each pair's dz sums to 0
    assert np.max(np.abs(g["z"].sum(axis=-1))) < 1e-12
    # every pair masked: a = b = 0 identically, so is every gradient
    g0 = oracle.project_vjp(z, np.zeros_like(m), w, da, db)
    assert all(np.max(np.abs(v)) == 0 for v in g0.values())
    # db = 0: nothing flows through the b side
    gb = oracle.project_vjp(z, m, w, da, np.zeros_like(db))
    assert np.max(np.abs(gb["w_b_proj"])) == 0 and np.max(np.abs(gb["w_b_gate"])) == 0
    # gates at zero: sigmoid = 1/2 and its slope 1/4, so with zh = LN(z)
    #   dW_ap = sum (m/2) da (x) zh,  dW_ag = sum (m/4) (W_ap zh) da (x) zh
    w0 = dict(w); w0["w_a_gate"] = np.zeros_like(w["w_a_gate"]); w0["w_b_gate"] = np.zeros_like(w["w_b_gate"])
    g0 = oracle.project_vjp(z, m, w0, da, db)
    zh = oracle.layer_norm(z, w["ln_in_w"], w["ln_in_b"])
    mm = m[:, None].astype(np.float64)
    assert np.max(np.abs(g0["w_a_proj"] - (0.5 * mm * da).T @ zh)) < 1e-12
    assert np.max(np.abs(g0["w_a_gate"] - (0.25 * mm * (zh @ w["w_a_proj"].T) * da).T @ zh)) < 1e-12


def _layer_case(seed, n=4, c=5, cz=6, keep=0.8):
    r = np.random.default_rng(seed)
    w = {"ln_in_w": 1 + 0.3 * r.standard_normal(cz), "ln_in_b": 0.2 * r.standard_normal(cz),
         "ln_out_w": 1 + 0.3 * r.standard_normal(c), "ln_out_b": 0.2 * r.standard_normal(c),
         "w_out_proj": r.standard_normal((cz, c)) / np.sqrt(c), "w_out_gate": r.standard_normal((cz, cz)) / np.sqrt(cz)}
    for k in ("w_a_proj", "w_a_gate", "w_b_proj", "w_b_gate"):
        w[k] = r.standard_normal((c, cz)) / np.sqrt(cz)
    z = r.standard_normal((n, n, cz)) + 0.2
    m = (r.random((n, n)) < keep).astype(np.uint8)
    m[0, 0] = 1
    dout = r.standard_normal((n, n, cz))
    return z, m, w, dout


@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
def test_trimul_vjp_finite_differences(direction):
    """The whole layer's gradient against central differences of the
    forward definition, for z and every parameter."""
    z, m, w, dout = _layer_case(41)
    g = oracle.trimul_vjp(z, m, w, direction, dout)
    L = lambda z_, w_: float(np.sum(dout * oracle.trimul(z_, m, w_, direction)))
    r = np.random.default_rng(42)
    h = 1e-5
    v = r.standard_normal(z.shape)
    fd = (L(z + h * v, w) - L(z - h * v, w)) / (2 * h)
    assert abs(fd - float(np.sum(g["z"] * v))) < 1e-6 * (1 + abs(fd))
    for key in oracle.WEIGHT_KEYS:
        v = r.standard_normal(np.shape(w[key]))
        wp = dict(w); wp[key] = w[key] + h * v
        wm = dict(w); wm[key] = w[key] - h * v
        fd = (L(z, wp) - L(z, wm)) / (2 * h)
        assert abs(fd - float(np.sum(g[key] * v))) < 1e-6 * (1 + abs(fd)), key


def test_trimul_vjp_transpose_relation():
    """incoming(z, m; W) = outgoing(z^T, m^T; W with a <-> b swapped)^T, so the
    incoming gradients are the outgoing ones of that problem: dz transposed,
    the a and b weights' gradients swapped, the rest equal."""
    z, m, w, dout = _layer_case(43)
    ws = dict(w)
    ws["w_a_proj"], ws["w_b_proj"] = w["w_b_proj"], w["w_a_proj"]
    ws["w_a_gate"], ws["w_b_gate"] = w["w_b_gate"], w["w_a_gate"]
    gi = oracle.trimul_vjp(z, m, w, "incoming", dout)
    go = oracle.trimul_vjp(np.swapaxes(z, 0, 1), m.T, ws, "outgoing", np.swapaxes(dout, 0, 1))
    assert np.max(np.abs(gi["z"] - np.swapaxes(go["z"], 0, 1))) < 1e-12
    swap = {"w_a_proj": "w_b_proj", "w_b_proj": "w_a_proj", "w_a_gate": "w_b_gate", "w_b_gate": "w_a_gate"}
    for key in oracle.WEIGHT_KEYS:
        assert np.max(np.abs(gi[key] - go[swap.get(key, key)])) < 1e-10, key
