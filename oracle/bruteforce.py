"""Per-element scalar loops of the triangle multiplicative update.

TEST INFRASTRUCTURE ONLY.  A second, independent spelling of the definition
in ``trimul_ref`` (same readings, see that module's docstring): every sum is
an explicit Python loop over plain floats, nothing is vectorised and no
library routine is used, so that an index, transpose or sign mistake in the
vectorised oracle cannot also be present here by construction.  Only for tiny
inputs (N <= 8).
"""

from __future__ import annotations

import math


def _ln(v, gamma, beta, eps):
    n = len(v)
    mu = 0.0
    for t in v:
        mu += t
    mu /= n
    var = 0.0
    for t in v:
        var += (t - mu) * (t - mu)
    var /= n
    inv = 1.0 / math.sqrt(var + eps)
    return [(v[e] - mu) * inv * gamma[e] + beta[e] for e in range(n)]


def _sig(t):
    if t >= 0:
        return 1.0 / (1.0 + math.exp(-t))
    e = math.exp(t)
    return e / (1.0 + e)


def _matvec(W, v):
    out = []
    for row in W:
        s = 0.0
        for e in range(len(v)):
            s += row[e] * v[e]
        out.append(s)
    return out


def bf16_nearest(t):
    """The bfloat16 value nearest to the float t, ties to the even neighbour.

    bfloat16 has 8 significant bits and float32's exponent range.  For a
    normal t = m * 2**e (0.5 <= |m| < 1) the spacing of bfloat16 values around
    t is 2**(e - 8); below 2**-126 it is the fixed 2**-133.  t divided by the
    spacing is a float with at most 9 integer bits, so Python's round() (which
    rounds halves to the even integer) picks the neighbour exactly.  Values
    that round to 2**128 or beyond become infinite."""
    if t == 0.0 or math.isinf(t) or math.isnan(t):
        return t
    if abs(t) >= 2.0 ** -126:
        _, e = math.frexp(t)
        q = e - 8
    else:
        q = -133
    r = round(math.ldexp(t, -q))
    if abs(r) >= 2 ** (128 - q):
        return math.copysign(math.inf, t)
    return math.ldexp(float(r), q)


def project_loops(z, mask, w, quant=False, eps=1e-5):
    """The gated a/b operands of every pair, as nested lists [N][N][c].

    quant=True adds the two roundings to bfloat16 of a bf16 matrix-core
    contraction: the normalised input after its affine map (gamma, beta),
    where it enters the four projections, and the finished a and b values.
    """
    n = len(z)
    W = {k: (v.tolist() if hasattr(v, "tolist") else v) for k, v in w.items()}
    c = len(W["w_a_proj"])
    a = [[None] * n for _ in range(n)]
    b = [[None] * n for _ in range(n)]
    for i in range(n):
        for j in range(n):
            zh = _ln(list(map(float, z[i][j])), W["ln_in_w"], W["ln_in_b"], eps)
            if quant:
                zh = [bf16_nearest(t) for t in zh]
            m = 1.0 if mask[i][j] else 0.0
            ap = _matvec(W["w_a_proj"], zh)
            ag = _matvec(W["w_a_gate"], zh)
            bp = _matvec(W["w_b_proj"], zh)
            bg = _matvec(W["w_b_gate"], zh)
            a[i][j] = [m * _sig(ag[d]) * ap[d] for d in range(c)]
            b[i][j] = [m * _sig(bg[d]) * bp[d] for d in range(c)]
            if quant:
                a[i][j] = [bf16_nearest(t) for t in a[i][j]]
                b[i][j] = [bf16_nearest(t) for t in b[i][j]]
    return a, b


def trimul_loops(z, mask, w, direction, eps=1e-5, quant=False):
    """z: nested lists [N][N][c_z]; mask: [N][N]; w: dict of nested lists.
    Returns out as nested lists [N][N][c_z].  quant=True rounds the
    contraction operands as ``project_loops`` does; nothing else is rounded."""
    n = len(z)
    W = {k: (v.tolist() if hasattr(v, "tolist") else v) for k, v in w.items()}
    c = len(W["w_a_proj"])
    zh = [[_ln(list(map(float, z[i][j])), W["ln_in_w"], W["ln_in_b"], eps) for j in range(n)]
          for i in range(n)]
    a, b = project_loops(z, mask, w, quant, eps)
    out = [[None] * n for _ in range(n)]
    for i in range(n):
        for j in range(n):
            x = []
            for d in range(c):
                s = 0.0
                for k in range(n):
                    if direction == "outgoing":
                        s += a[i][k][d] * b[j][k][d]
                    else:
                        s += a[k][i][d] * b[k][j][d]
                x.append(s)
            nn = _ln(x, W["ln_out_w"], W["ln_out_b"], eps)
            y = _matvec(W["w_out_proj"], nn)
            g = _matvec(W["w_out_gate"], zh[i][j])
            m = 1.0 if mask[i][j] else 0.0
            out[i][j] = [m * _sig(g[e]) * y[e] for e in range(len(y))]
    return out


def contract_vjp_loops(a_rows, b_rows, dx):
    """Scalar loops for the gradients of L = sum dx[i][j][d] * x[i][j][d],
    x[i][j][d] = sum_k a_rows[i][k][d] * b_rows[j][k][d]: every term of L
    that contains a_rows[i][k][d] is dx[i][j][d] * a_rows[i][k][d] *
    b_rows[j][k][d] for some j, so its derivative collects those b values
    (and symmetrically for b_rows).  Nested lists in, nested lists out."""
    Mi, K, c = len(a_rows), len(a_rows[0]), len(a_rows[0][0])
    Mj = len(b_rows)
    da = [[[0.0] * c for _ in range(K)] for _ in range(Mi)]
    db = [[[0.0] * c for _ in range(K)] for _ in range(Mj)]
    for i in range(Mi):
        for j in range(Mj):
            for k in range(K):
                for d in range(c):
                    g = dx[i][j][d]
                    da[i][k][d] += g * b_rows[j][k][d]
                    db[j][k][d] += g * a_rows[i][k][d]
    return da, db


def window_attention_loops(q, k, v, bias=None, mask=None, scale=None):
    """Scalar-loop spelling of ``atom_attention.window_attention`` (same
    readings: query block i // 32, keys 32*(i // 32) - 48 .. + 127 that lie in
    the sequence and are unmasked, softmax of scale * q.k + bias, 0 when no key
    is left).  q, k, v are nested lists or arrays [batch][n][heads][d]."""
    bsz, n, heads, d = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = [[[[0.0] * d for _ in range(heads)] for _ in range(n)] for _ in range(bsz)]
    for b in range(bsz):
        for i in range(n):
            w = i // 32
            first = 32 * w - 48
            for h in range(heads):
                logits = []
                for t in range(128):
                    j = first + t
                    if j < 0 or j >= n or (mask is not None and mask[b][j] == 0):
                        continue
                    s = 0.0
                    for e in range(d):
                        s += float(q[b][i][h][e]) * float(k[b][j][h][e])
                    s *= scale
                    if bias is not None:
                        s += float(bias[b][w][h][i - 32 * w][t])
                    logits.append((j, s))
                if not logits:
                    continue
                top = max(s for _, s in logits)
                den = 0.0
                for _, s in logits:
                    den += math.exp(s - top)
                for j, s in logits:
                    p = math.exp(s - top) / den
                    for e in range(d):
                        out[b][i][h][e] += p * float(v[b][j][h][e])
    return out
