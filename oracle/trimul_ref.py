"""Vectorised float64 definition of the triangle multiplicative update.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

Source of the operation
-----------------------
Page 1 ("NVIDIA BioNeMo escala modelagem biomolecular com context
parallelism ...", section "Exemplo de codigo: triangle multiplication
CP-aware") builds ``TriangleMultiplicationOutgoing(size_input_embed)`` and
calls it as ``layer(x, mask)`` on the pair representation; its
"2D tiling da pair representation" section splits the N x N pair grid into
sub-blocks, one per device.  Page 4 (hyper.ai, French summary) names the
"module de multiplication triangulaire" among the parts adapted for that
tiling.  The pages do not print the layer's equations; this module writes out
the AlphaFold3-style definition, with the readings listed below.

Definition (per pair (i, j); vectors run over the channel axis)::

    zh_ij  = LN(z_ij; g_in, b_in)                          input LayerNorm
    a_ij   = m_ij * sigmoid(W_ag zh_ij) * (W_ap zh_ij)     gated projection a
    b_ij   = m_ij * sigmoid(W_bg zh_ij) * (W_bp zh_ij)     gated projection b
    x_ij   = sum_k a_ik * b_jk        (outgoing)
    x_ij   = sum_k a_ki * b_kj        (incoming)
    n_ij   = LN(x_ij; g_out, b_out)                        output LayerNorm
    y_ij   = W_o n_ij                                      output projection
    g_ij   = sigmoid(W_g zh_ij)                            output gate
    out_ij = m_ij * g_ij * y_ij                            masked update

Readings where the pages are silent: LayerNorm over the channel axis with
biased variance and eps = 1e-5; linear maps carry no bias; the gates read the
normalised zh; the pair mask multiplies a, b and the output; no residual add
and no dropout.  W_* are stored as (out_features, in_features), so
``W v`` is ``v @ W.T``.

Q-mode (``quant=True``) is the same definition with exactly two rounding
points added, both round-to-nearest-even to bfloat16: zh where it enters the
four a/b projections, and the finished a and b.  These are the operand
roundings that a bf16 matrix-core contraction with fp32 accumulation makes;
every other quantity stays float64.
"""

from __future__ import annotations

import numpy as np

LN_EPS = 1e-5

WEIGHT_KEYS = (
    "ln_in_w", "ln_in_b",
    "w_a_proj", "w_a_gate", "w_b_proj", "w_b_gate",
    "w_out_gate", "ln_out_w", "ln_out_b", "w_out_proj",
)


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def bf16_round(x):
    """Round float64 values to the nearest bfloat16 value, ties to even.

    bfloat16 keeps 8 significant bits (7 stored + the implicit one) and the
    float32 exponent range, so subnormals have spacing 2**-133 and the
    largest finite value is (2 - 2**-7) * 2**127.  The rounding is done in one
    step from float64 (never via float32, which would round twice).
    """
    x = _f64(x)
    out = np.empty_like(x)
    finite = np.isfinite(x)
    xf = np.where(finite, x, 0.0)
    mant, expo = np.frexp(xf)                    # xf = mant * 2**expo, 0.5 <= |mant| < 1
    normal = np.abs(xf) >= 2.0 ** -126
    # normal range: 8 significant bits -> mant * 2**8 in [128, 256)
    r_norm = np.ldexp(np.rint(mant * 256.0), expo - 8)
    # subnormal range: fixed quantum 2**-133
    r_sub = np.ldexp(np.rint(np.ldexp(xf, 133)), -133)
    r = np.where(normal, r_norm, r_sub)
    r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, r), r)
    out[...] = np.where(finite, r, x)
    return out


def sigmoid(t):
    """Logistic function 1 / (1 + e^-t), evaluated without overflow."""
    t = _f64(t)
    e = np.exp(-np.abs(t))                       # in (0, 1], never overflows
    return np.where(t >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def layer_norm(v, gamma, beta, eps=LN_EPS):
    """LayerNorm over the last axis: (v - mean) / sqrt(var + eps) * gamma + beta,
    with the biased (population) variance."""
    v = _f64(v)
    mu = v.mean(axis=-1, keepdims=True)
    d = v - mu
    var = (d * d).mean(axis=-1, keepdims=True)
    return d / np.sqrt(var + eps) * _f64(gamma) + _f64(beta)


def _lin(v, w):
    """Bias-free linear map W v for W stored as (out_features, in_features)."""
    return _f64(v) @ _f64(w).T


def project(z, mask, w, quant=False, eps=LN_EPS):
    """Gated a/b projections of every pair in ``z`` (shape [..., c_z]).

    Returns (a, b), each [..., c].  ``mask`` has the shape of ``z`` without
    the channel axis; nonzero keeps the pair.
    """
    zh = layer_norm(z, w["ln_in_w"], w["ln_in_b"], eps)
    if quant:
        zh = bf16_round(zh)
    m = (_f64(mask) != 0).astype(np.float64)[..., None]
    a = m * sigmoid(_lin(zh, w["w_a_gate"])) * _lin(zh, w["w_a_proj"])
    b = m * sigmoid(_lin(zh, w["w_b_gate"])) * _lin(zh, w["w_b_proj"])
    if quant:
        a = bf16_round(a)
        b = bf16_round(b)
    return a, b


def contract_rows(a_rows, b_rows):
    """x[i, j, d] = sum_k a_rows[i, k, d] * b_rows[j, k, d].

    ``a_rows`` is [Mi, K, c] and ``b_rows`` is [Mj, K, c]; the result is
    [Mi, Mj, c].  Per channel d this is one matrix product A_d B_d^T, done by
    ``numpy.matmul`` on channel-major copies.
    """
    A = np.ascontiguousarray(np.moveaxis(_f64(a_rows), 2, 0))       # [c, Mi, K]
    B = np.ascontiguousarray(np.moveaxis(_f64(b_rows), 2, 0))       # [c, Mj, K]
    X = np.matmul(A, np.swapaxes(B, 1, 2))                          # [c, Mi, Mj]
    return np.moveaxis(X, 0, 2)


def contract_rows_vjp(a_rows, b_rows, dx):
    """Gradients of the scalar L = sum_{i,j,d} dx[i, j, d] * x[i, j, d] with
    x = contract_rows(a_rows, b_rows), with respect to both operands:

        da[i, k, d] = sum_j dx[i, j, d] * b_rows[j, k, d]
        db[j, k, d] = sum_i dx[i, j, d] * a_rows[i, k, d]

    (per channel d: dA_d = dX_d B_d and dB_d = dX_d^T A_d), done by
    ``numpy.matmul`` on channel-major copies.  ``dx`` is [Mi, Mj, c]; the
    results have the shapes of ``a_rows`` and ``b_rows``.  This is the backward
    of the contraction step of the layer, which page 1 (section "Pra quem e")
    expects to be wrapped in custom autograd functions for training.
    """
    A = np.ascontiguousarray(np.moveaxis(_f64(a_rows), 2, 0))       # [c, Mi, K]
    B = np.ascontiguousarray(np.moveaxis(_f64(b_rows), 2, 0))       # [c, Mj, K]
    DX = np.ascontiguousarray(np.moveaxis(_f64(dx), 2, 0))          # [c, Mi, Mj]
    dA = np.matmul(DX, B)                                           # [c, Mi, K]
    dB = np.matmul(np.swapaxes(DX, 1, 2), A)                        # [c, Mj, K]
    return np.moveaxis(dA, 0, 2), np.moveaxis(dB, 0, 2)


def contract(a, b, direction):
    """The k-contraction over the full pair grid ([N, N, c] each).

    outgoing: x_ij = sum_k a_ik * b_jk ;  incoming: x_ij = sum_k a_ki * b_kj.
    """
    if direction == "outgoing":
        return contract_rows(a, b)
    if direction == "incoming":
        return contract_rows(np.swapaxes(a, 0, 1), np.swapaxes(b, 0, 1))
    raise ValueError(f"unknown direction {direction!r}")


def finish(x, z, mask, w, eps=LN_EPS):
    """Epilogue: out = m * sigmoid(W_g LN_in(z)) * (W_o LN_out(x)).

    ``x`` is [..., c], ``z`` the matching [..., c_z] input pairs, ``mask`` the
    matching pair mask.  Computed in float64 with no rounding.
    """
    n = layer_norm(x, w["ln_out_w"], w["ln_out_b"], eps)
    y = _lin(n, w["w_out_proj"])
    zh = layer_norm(z, w["ln_in_w"], w["ln_in_b"], eps)
    g = sigmoid(_lin(zh, w["w_out_gate"]))
    m = (_f64(mask) != 0).astype(np.float64)[..., None]
    return m * g * y


def _ln_parts(v, eps):
    """Normalised v (before the affine map) and 1 / sqrt(var + eps), biased var."""
    v = _f64(v)
    mu = v.mean(axis=-1, keepdims=True)
    d = v - mu
    r = 1.0 / np.sqrt((d * d).mean(axis=-1, keepdims=True) + eps)
    return d * r, r


def _ln_vjp(g_hat, v_hat, r):
    """Gradient with respect to the LayerNorm input v, given the gradient g_hat
    with respect to the normalised v_hat = (v - mean) * r (biased variance):
    r * (g_hat - mean(g_hat) - v_hat * mean(g_hat * v_hat))."""
    return r * (g_hat - g_hat.mean(axis=-1, keepdims=True)
                - v_hat * (g_hat * v_hat).mean(axis=-1, keepdims=True))


def finish_vjp(x, z, mask, w, dout, eps=LN_EPS):
    """Gradients of L = sum(dout * finish(x, z, mask, w)), the backward of the
    epilogue (the layer's output LayerNorm, output projection, output gate and
    mask), with respect to x, to z through the gate's input LayerNorm (the
    gate path's share of dL/dz; the a/b projections add the rest), and to the
    parameters the epilogue uses.  Returns a dict with keys x, z, w_out_proj,
    w_out_gate, ln_out_w, ln_out_b, ln_in_w, ln_in_b (the last two: the gate
    path's share).  float64, following the forward's steps backwards:

        n = LN(x) = nh*g_o + b_o,  y = W_o n,  zh = LN(z) = zhh*g_i + b_i,
        t = W_g zh,  s = sigmoid(t),  out = m * s * y
        dy = m*s*dout,  dt = m*y*dout * s*(1 - s)
        dW_o = sum dy (x) n,  dn = W_o^T dy,  dg_o = sum dn*nh,  db_o = sum dn
        dx = LN backward of dn*g_o
        dW_g = sum dt (x) zh,  dzh = W_g^T dt,  dg_i = sum dzh*zhh,  db_i = sum dzh
        dz = LN backward of dzh*g_i
    (sums over all pairs).  Page 1 (section "Pra quem e") expects the layer to
    be trained through custom autograd functions; this is the epilogue's part.
    """
    x, z, g = _f64(x), _f64(z), _f64(dout)
    m = (_f64(mask) != 0).astype(np.float64)[..., None]
    nh, rx = _ln_parts(x, eps)
    n = nh * _f64(w["ln_out_w"]) + _f64(w["ln_out_b"])
    y = _lin(n, w["w_out_proj"])
    zhh, rz = _ln_parts(z, eps)
    zh = zhh * _f64(w["ln_in_w"]) + _f64(w["ln_in_b"])
    s = sigmoid(_lin(zh, w["w_out_gate"]))
    dy = m * s * g
    dt = m * y * g * s * (1.0 - s)
    c, cz = n.shape[-1], zh.shape[-1]
    dy2, n2, dt2, zh2 = dy.reshape(-1, cz), n.reshape(-1, c), dt.reshape(-1, cz), zh.reshape(-1, cz)
    dn = dy @ _f64(w["w_out_proj"])
    dzh = dt @ _f64(w["w_out_gate"])
    return {
        "x": _ln_vjp(dn * _f64(w["ln_out_w"]), nh, rx),
        "z": _ln_vjp(dzh * _f64(w["ln_in_w"]), zhh, rz),
        "w_out_proj": dy2.T @ n2,
        "w_out_gate": dt2.T @ zh2,
        "ln_out_w": (dn * nh).reshape(-1, c).sum(axis=0),
        "ln_out_b": dn.reshape(-1, c).sum(axis=0),
        "ln_in_w": (dzh * zhh).reshape(-1, cz).sum(axis=0),
        "ln_in_b": dzh.reshape(-1, cz).sum(axis=0),
    }


def trimul(z, mask, w, direction, quant=False, eps=LN_EPS, return_x=False):
    """Whole update on a full [N, N, c_z] pair tensor; returns [N, N, c_z]."""
    a, b = project(z, mask, w, quant, eps)
    x = contract(a, b, direction)
    out = finish(x, z, mask, w, eps)
    return (out, x) if return_x else out


def project_vjp(z, mask, w, da, db, eps=LN_EPS):
    """Gradients of L = sum(da * a) + sum(db * b) with (a, b) = project(z,
    mask, w) (exact, no rounding): the backward of the gated a/b projections.
    Returns a dict with keys z (the projections' share of dL/dz), w_a_proj,
    w_a_gate, w_b_proj, w_b_gate, ln_in_w, ln_in_b (the projections' share).
    float64, the forward's steps backwards, per side s in (a, b):

        zh = LN(z) = zhh*g_i + b_i,  u = W_sp zh,  v = W_sg zh,
        g = sigmoid(v),  s = m * g * u
        du = m*g*ds,  dv = m*u*ds * g*(1 - g)
        dW_sp = sum du (x) zh,  dW_sg = sum dv (x) zh
        dzh = sum over sides of (W_sp^T du + W_sg^T dv)
        dg_i = sum dzh*zhh,  db_i = sum dzh,  dz = LN backward of dzh*g_i
    (sums over all pairs).  Page 1 (section "Pra quem e") expects the layer to
    be trained through custom autograd functions; this is the projections'
    part.
    """
    z = _f64(z)
    m = (_f64(mask) != 0).astype(np.float64)[..., None]
    zhh, rz = _ln_parts(z, eps)
    zh = zhh * _f64(w["ln_in_w"]) + _f64(w["ln_in_b"])
    cz = zh.shape[-1]
    zh2 = zh.reshape(-1, cz)
    out = {}
    dzh = np.zeros_like(zh)
    for side, ds in (("a", _f64(da)), ("b", _f64(db))):
        wp, wg = _f64(w[f"w_{side}_proj"]), _f64(w[f"w_{side}_gate"])
        u = _lin(zh, wp)
        g = sigmoid(_lin(zh, wg))
        du = m * g * ds
        dv = m * u * ds * g * (1.0 - g)
        c = u.shape[-1]
        out[f"w_{side}_proj"] = du.reshape(-1, c).T @ zh2
        out[f"w_{side}_gate"] = dv.reshape(-1, c).T @ zh2
        dzh = dzh + du @ wp + dv @ wg
    out["z"] = _ln_vjp(dzh * _f64(w["ln_in_w"]), zhh, rz)
    out["ln_in_w"] = (dzh * zhh).reshape(-1, cz).sum(axis=0)
    out["ln_in_b"] = dzh.reshape(-1, cz).sum(axis=0)
    return out


def trimul_vjp(z, mask, w, direction, dout, eps=LN_EPS):
    """Gradients of L = sum(dout * trimul(z, mask, w, direction)) (exact) with
    respect to z and every parameter (keys z and WEIGHT_KEYS): the whole
    layer's backward, composed of the three steps' gradients in reverse order
    -- finish_vjp (epilogue), contract_rows_vjp (the k-contraction; incoming
    contracts the transposed operands) and project_vjp (projections) -- with
    dL/dz and the input LayerNorm's parameters summed over the gate path and
    the projections.  Page 1 (section "Pra quem e") expects the layer to be
    trained through custom autograd functions; this is its full gradient.
    """
    a, b = project(z, mask, w, False, eps)
    x = contract(a, b, direction)
    ge = finish_vjp(x, z, mask, w, dout, eps)
    if direction == "outgoing":
        da, db = contract_rows_vjp(a, b, ge["x"])
    elif direction == "incoming":
        dat, dbt = contract_rows_vjp(np.swapaxes(a, 0, 1), np.swapaxes(b, 0, 1), ge["x"])
        da, db = np.swapaxes(dat, 0, 1), np.swapaxes(dbt, 0, 1)
    else:
        raise ValueError(f"unknown direction {direction!r}")
    gp = project_vjp(z, mask, w, da, db, eps)
    return {
        "z": ge["z"] + gp["z"],
        "ln_in_w": ge["ln_in_w"] + gp["ln_in_w"],
        "ln_in_b": ge["ln_in_b"] + gp["ln_in_b"],
        "w_a_proj": gp["w_a_proj"], "w_a_gate": gp["w_a_gate"],
        "w_b_proj": gp["w_b_proj"], "w_b_gate": gp["w_b_gate"],
        "w_out_gate": ge["w_out_gate"], "ln_out_w": ge["ln_out_w"], "ln_out_b": ge["ln_out_b"],
        "w_out_proj": ge["w_out_proj"],
    }


# ---------------------------------------------------------------------------
# Evaluation on parts of the grid.  Every output pair (i, j) needs only the
# operand rows i and j (outgoing) or the operand columns i and j (incoming),
# so these are exact, not approximations.
# ---------------------------------------------------------------------------

def _operand_rows(get_z, get_mask, idx, n, direction, w, quant, eps, k_idx=None):
    """Operand strip for residues ``idx``: [len(idx), K, c] with entry [r, k]
    the operand of pair (idx[r], k) (outgoing) or (k, idx[r]) (incoming)."""
    ks = np.arange(n) if k_idx is None else np.asarray(k_idx)
    if direction == "outgoing":
        zs, ms = get_z(idx, ks), get_mask(idx, ks)
    elif direction == "incoming":
        zs = np.swapaxes(get_z(ks, idx), 0, 1)
        ms = np.swapaxes(get_mask(ks, idx), 0, 1)
    else:
        raise ValueError(f"unknown direction {direction!r}")
    return project(zs, ms, w, quant, eps)


def tile_partial(get_z, get_mask, n, w, direction, rows, cols, k_idx, quant=False, eps=LN_EPS):
    """Partial contraction of one tile over the residues ``k_idx`` only:
    x[r, s, d] = sum_{k in k_idx} (operand of row rows[r]) * (operand of col cols[s]).

    ``get_z(ri, ci)`` returns z[ri][:, ci] as an array [len(ri), len(ci), c_z];
    ``get_mask`` likewise for the pair mask.  Summing the partials over a set of
    disjoint k ranges that covers [0, n) gives the full x of the tile.
    """
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    a_rows, _ = _operand_rows(get_z, get_mask, rows, n, direction, w, quant, eps, k_idx)
    _, b_rows = _operand_rows(get_z, get_mask, cols, n, direction, w, quant, eps, k_idx)
    return contract_rows(a_rows, b_rows)


def trimul_sampled(get_z, get_mask, n, w, direction, rows, cols, quant=False, eps=LN_EPS,
                   return_x=False):
    """Output of the update at the pairs rows x cols only: [len(rows), len(cols), c_z]."""
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    x = tile_partial(get_z, get_mask, n, w, direction, rows, cols, None, quant, eps)
    out = finish(x, get_z(rows, cols), get_mask(rows, cols), w, eps)
    return (out, x) if return_x else out


def trimul_blockwise(z, mask, w, direction, quant=False, eps=LN_EPS, block=128):
    """Whole update, evaluated in blocks of output rows to bound host memory.

    The a/b operands are computed once (they are [N, N, c]); the contraction
    and epilogue are done ``block`` output rows at a time.
    """
    n = z.shape[0]
    a, b = project(z, mask, w, quant, eps)
    if direction == "incoming":
        a = np.swapaxes(a, 0, 1)
        b = np.swapaxes(b, 0, 1)
    out = np.empty(z.shape[:2] + (np.asarray(w["w_out_proj"]).shape[0],), dtype=np.float64)
    for r0 in range(0, n, block):
        r1 = min(n, r0 + block)
        x = contract_rows(a[r0:r1], b)
        out[r0:r1] = finish(x, z[r0:r1], mask[r0:r1], w, eps)
    return out


def array_getters(z, mask):
    """``get_z``/``get_mask`` callables over in-memory arrays."""
    def get_z(ri, ci):
        return _f64(z[np.ix_(np.asarray(ri), np.asarray(ci))])

    def get_mask(ri, ci):
        return np.asarray(mask[np.ix_(np.asarray(ri), np.asarray(ci))])

    return get_z, get_mask
