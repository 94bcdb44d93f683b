"""CPU tests of the C ABI: the library loads, exports every function that
include/trimul.h declares, sizes workspaces by the documented closed form, and
rejects every invalid argument with its status code before any HIP call.

Pointers here are fake (aligned or deliberately misaligned integers): each case
fails validation, which runs before the first HIP call, so nothing is ever
dereferenced or launched.
"""

import ctypes
import os
import re

import pytest
import torch

import pair_representation_amd as pra

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "trimul.h")

FAKE = 0x7F0000000000  # 256-byte aligned fake device address


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(trimul_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_function():
    L = pra.lib()
    names = header_functions()
    assert "trimul_outgoing" in names and "trimul_tile" in names
    for name in names:
        assert hasattr(L, name), f"{name} declared in trimul.h but not exported"


def weights(dtype=pra.BF16, c_z=128, c=128, eps=1e-5, null=None, misalign=None):
    s = pra._Weights()
    s.c_z, s.c, s.dtype, s.ln_eps = c_z, c, dtype, eps
    names = [f[0] for f in pra._Weights._fields_[4:]]
    for i, k in enumerate(names):
        setattr(s, k, FAKE + 0x10000 * (i + 1))
    if null:
        setattr(s, null, None)
    if misalign:
        setattr(s, misalign, FAKE + 0x10000 * 20 + 8)
    return s


def call_full(w, n=16, z=FAKE, mask=FAKE + 1, out=FAKE + 0x100000, ws=FAKE + 0x200000, ws_bytes=None,
              incoming=False):
    L = pra.lib()
    if ws_bytes is None:
        ws_bytes = L.trimul_workspace_bytes(ctypes.byref(w), n)
    fn = L.trimul_incoming if incoming else L.trimul_outgoing
    return fn(ctypes.byref(w), z, mask, out, n, ws, ws_bytes, None)


def round_up(v, m):
    return (v + m - 1) // m * m


@pytest.mark.parametrize("dtype,elt", [(pra.BF16, 2), (pra.F32, 4)])
@pytest.mark.parametrize("n", [1, 2, 63, 64, 65, 768, 3605, 10000])
def test_workspace_closed_form(dtype, elt, n):
    w = weights(dtype)
    kp = round_up(n, 64)
    a256 = lambda v: round_up(v, 256)
    xacc = 128 * round_up(n, 4) * round_up(n, 16) * 4
    want = 2 * a256(128 * round_up(n, 256) * kp * elt) + a256(xacc)
    assert pra.lib().trimul_workspace_bytes(ctypes.byref(w), n) == want
    assert pra.lib().trimul_tile_xacc_bytes(ctypes.byref(w), n, n) == xacc


def test_workspace_invalid():
    L = pra.lib()
    assert L.trimul_workspace_bytes(None, 10) == 0
    assert L.trimul_workspace_bytes(ctypes.byref(weights()), -1) == 0
    assert L.trimul_workspace_bytes(ctypes.byref(weights()), 70000) == 0
    assert L.trimul_workspace_bytes(ctypes.byref(weights(dtype=7)), 10) == 0
    # operand rows are padded to a multiple of 256
    assert L.trimul_tile_operand_bytes(ctypes.byref(weights()), 5000, 1280) == 128 * 5120 * 1280 * 2


def test_n_zero_is_noop():
    assert call_full(weights(), n=0, z=None, mask=None, out=None, ws=None, ws_bytes=0) == pra.OK


@pytest.mark.parametrize("incoming", [False, True])
def test_full_validation(incoming):
    L = pra.lib()
    E = dict(incoming=incoming)
    assert L.trimul_outgoing(None, FAKE, FAKE, FAKE, 4, FAKE, 1 << 30, None) == pra.ERR_INVALID_ARG
    assert call_full(weights(c_z=64), **E) == pra.ERR_UNSUPPORTED
    assert call_full(weights(c=256), **E) == pra.ERR_UNSUPPORTED
    assert call_full(weights(dtype=3), **E) == pra.ERR_UNSUPPORTED
    assert call_full(weights(eps=0.0), **E) == pra.ERR_INVALID_ARG
    assert call_full(weights(eps=float("nan")), **E) == pra.ERR_INVALID_ARG
    for k in ("ln_in_w", "w_a_proj", "w_b_gate", "w_out_gate", "ln_out_b", "w_out_proj"):
        assert call_full(weights(null=k), **E) == pra.ERR_INVALID_ARG
        assert call_full(weights(misalign=k), **E) == pra.ERR_ALIGNMENT
    w = weights()
    assert call_full(w, n=-1, **E) == pra.ERR_INVALID_ARG
    assert call_full(w, n=65536, **E) == pra.ERR_INVALID_ARG
    assert call_full(w, z=None, **E) == pra.ERR_INVALID_ARG
    assert call_full(w, mask=None, **E) == pra.ERR_INVALID_ARG
    assert call_full(w, out=None, **E) == pra.ERR_INVALID_ARG
    assert call_full(w, ws=None, **E) == pra.ERR_INVALID_ARG
    assert call_full(w, z=FAKE + 4, **E) == pra.ERR_ALIGNMENT
    assert call_full(w, out=FAKE + 0x100008, **E) == pra.ERR_ALIGNMENT
    assert call_full(w, ws=FAKE + 0x200010, **E) == pra.ERR_ALIGNMENT
    need = L.trimul_workspace_bytes(ctypes.byref(w), 16)
    assert call_full(w, ws_bytes=need - 1, **E) == pra.ERR_WORKSPACE_TOO_SMALL
    msg = L.trimul_last_error().decode()
    assert "workspace" in msg and str(need) in msg


def call_chunked(w=None, direction=pra.OUTGOING, n=300, blocks=(64, 0, 100), z=FAKE, mask=FAKE + 1,
                 out=FAKE + 0x100000, ws=FAKE + 0x200000, ws_bytes=None):
    w = weights() if w is None else w
    L = pra.lib()
    if ws_bytes is None:
        ws_bytes = L.trimul_chunked_workspace_bytes(ctypes.byref(w), n, *blocks)
    return L.trimul_forward_chunked(ctypes.byref(w), direction, z, mask, out, n, *blocks, ws, ws_bytes, None)


@pytest.mark.parametrize("dtype,elt", [(pra.BF16, 2), (pra.F32, 4)])
def test_chunked_workspace_closed_form(dtype, elt):
    L = pra.lib()
    w = weights(dtype)
    a256 = lambda v: round_up(v, 256)
    for n, R, C, K in ((300, 64, 0, 100), (14000, 3500, 0, 7000), (14000, 512, 512, 512), (77, 0, 0, 0),
                       (77, 500, 1, 3)):
        R2, C2, K2 = (v if 0 < v <= n else n for v in (R, C, K))
        want = (a256(128 * round_up(R2, 256) * round_up(K2, 64) * elt)
                + a256(128 * round_up(C2, 256) * round_up(K2, 64) * elt)
                + a256(128 * round_up(R2, 4) * round_up(C2, 16) * 4))
        assert L.trimul_chunked_workspace_bytes(ctypes.byref(w), n, R, C, K) == want
    # the whole-grid workspace is the special case of one block per axis
    assert L.trimul_chunked_workspace_bytes(ctypes.byref(w), 3605, 0, 0, 0) == \
        L.trimul_workspace_bytes(ctypes.byref(w), 3605)
    assert L.trimul_chunked_workspace_bytes(ctypes.byref(w), 0, 1, 1, 1) == 0
    assert L.trimul_chunked_workspace_bytes(ctypes.byref(w), 10, -1, 1, 1) == 0
    assert L.trimul_chunked_workspace_bytes(None, 10, 1, 1, 1) == 0


def test_chunked_validation():
    L = pra.lib()
    assert call_chunked(n=0, z=None, mask=None, out=None, ws=None, ws_bytes=0) == pra.OK
    assert call_chunked(w=weights(c_z=64)) == pra.ERR_UNSUPPORTED
    assert call_chunked(direction=2) == pra.ERR_INVALID_ARG
    assert call_chunked(blocks=(-1, 0, 0)) == pra.ERR_INVALID_ARG
    assert call_chunked(blocks=(0, 0, -5)) == pra.ERR_INVALID_ARG
    assert call_chunked(n=65536) == pra.ERR_INVALID_ARG
    assert call_chunked(z=None) == pra.ERR_INVALID_ARG
    assert call_chunked(ws=None) == pra.ERR_INVALID_ARG
    assert call_chunked(out=FAKE + 0x100004) == pra.ERR_ALIGNMENT
    assert call_chunked(ws=FAKE + 0x200040) == pra.ERR_ALIGNMENT
    need = L.trimul_chunked_workspace_bytes(ctypes.byref(weights()), 300, 64, 0, 100)
    assert call_chunked(ws_bytes=need - 1) == pra.ERR_WORKSPACE_TOO_SMALL
    assert str(need) in L.trimul_last_error().decode()


def test_noalloc_validation():
    """The allocation-free variant validates like trimul_forward_chunked and
    rejects blocks whose workspace exceeds its scratch array, before any HIP
    call (the array's address is looked up only after validation)."""
    L = pra.lib()
    text = open(HEADER).read()
    m = re.search(r"#define TRIMUL_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == pra.NOALLOC_SCRATCH_BYTES

    def call(w=None, direction=pra.OUTGOING, n=300, blocks=(0, 0, 0), z=FAKE, mask=FAKE + 1, out=FAKE + 0x100000):
        w = weights() if w is None else w
        return L.trimul_forward_chunked_noalloc(ctypes.byref(w), direction, z, mask, out, n, *blocks, None)

    assert call(n=0, z=None, mask=None, out=None) == pra.OK
    assert call(w=weights(c=64)) == pra.ERR_UNSUPPORTED
    assert call(direction=5) == pra.ERR_INVALID_ARG
    assert call(blocks=(0, -1, 0)) == pra.ERR_INVALID_ARG
    assert call(z=None) == pra.ERR_INVALID_ARG
    assert call(out=FAKE + 0x100004) == pra.ERR_ALIGNMENT
    assert call(n=70000) == pra.ERR_INVALID_ARG
    # n = 600 in one block needs more than the array; bf16 n = 512 and fp32
    # n = 356 are the largest whole-grid sizes that fit
    w16, w32 = weights(pra.BF16), weights(pra.F32)
    assert L.trimul_chunked_workspace_bytes(ctypes.byref(w16), 512, 0, 0, 0) <= pra.NOALLOC_SCRATCH_BYTES
    assert L.trimul_chunked_workspace_bytes(ctypes.byref(w16), 513, 0, 0, 0) > pra.NOALLOC_SCRATCH_BYTES
    assert L.trimul_chunked_workspace_bytes(ctypes.byref(w32), 356, 0, 0, 0) <= pra.NOALLOC_SCRATCH_BYTES
    assert L.trimul_chunked_workspace_bytes(ctypes.byref(w32), 357, 0, 0, 0) > pra.NOALLOC_SCRATCH_BYTES
    assert L.trimul_chunked_workspace_bytes(ctypes.byref(w16), 65535, 512, 512, 512) <= pra.NOALLOC_SCRATCH_BYTES
    assert L.trimul_chunked_workspace_bytes(ctypes.byref(w32), 65535, 512, 512, 256) <= pra.NOALLOC_SCRATCH_BYTES
    assert call(n=600) == pra.ERR_WORKSPACE_TOO_SMALL
    msg = L.trimul_last_error().decode()
    assert str(pra.NOALLOC_SCRATCH_BYTES) in msg and "600 x 600 x 600" in msg
    assert call(w=w32, n=2000, blocks=(512, 512, 512)) == pra.ERR_WORKSPACE_TOO_SMALL


def call_ops(w=None, direction=pra.OUTGOING, z=FAKE, mask=FAKE, n=100, row_off=0, n_rows=10, col_off=0,
             n_cols=10, k_off=0, k_len=100, ld=128, a=FAKE + 0x10000000, b=FAKE + 0x20000000):
    w = weights() if w is None else w
    return pra.lib().trimul_tile_operands(ctypes.byref(w), direction, z, mask, n, row_off, n_rows, col_off,
                                          n_cols, k_off, k_len, ld, a, b, None)


def test_tile_operands_validation():
    assert call_ops(w=weights(c=64)) == pra.ERR_UNSUPPORTED
    assert call_ops(direction=2) == pra.ERR_INVALID_ARG
    assert call_ops(n=0) == pra.ERR_INVALID_ARG
    assert call_ops(z=None) == pra.ERR_INVALID_ARG
    assert call_ops(mask=None) == pra.ERR_INVALID_ARG
    assert call_ops(a=None, b=None) == pra.ERR_INVALID_ARG
    assert call_ops(row_off=95, n_rows=10) == pra.ERR_INVALID_ARG
    assert call_ops(row_off=-1) == pra.ERR_INVALID_ARG
    assert call_ops(n_rows=0) == pra.ERR_INVALID_ARG
    assert call_ops(col_off=91, n_cols=10) == pra.ERR_INVALID_ARG
    assert call_ops(k_off=1, k_len=100) == pra.ERR_INVALID_ARG
    assert call_ops(k_len=0) == pra.ERR_INVALID_ARG
    assert call_ops(ld=96) == pra.ERR_INVALID_ARG            # not a multiple of 64
    assert call_ops(k_len=100, ld=64) == pra.ERR_INVALID_ARG   # ld < k_len
    assert call_ops(a=FAKE + 8) == pra.ERR_ALIGNMENT
    assert call_ops(z=FAKE + 2) == pra.ERR_ALIGNMENT
    # a range that only matters for the operand that is requested
    assert call_ops(a=None, row_off=95, n_rows=10, col_off=0, n_cols=200) == pra.ERR_INVALID_ARG


def call_tile(chunks=None, n=100, row_off=0, n_rows=50, col_off=50, n_cols=50, flags=pra.TILE_FIRST,
              x=FAKE, z=FAKE, mask=FAKE, out=FAKE, w=None, n_chunks=None):
    w = weights() if w is None else w
    if chunks is None:
        chunks = [(0, 100, 128)]
    arr = (pra.KChunk * max(1, len(chunks)))()
    for i, (ko, kl, ld) in enumerate(chunks):
        arr[i] = pra.KChunk(ko, kl, ld, FAKE + 0x1000000 * (i + 1), FAKE + 0x1000000 * (i + 40))
    nc = len(chunks) if n_chunks is None else n_chunks
    return pra.lib().trimul_tile(ctypes.byref(w), n, row_off, n_rows, col_off, n_cols, arr, nc, flags, x, z,
                                 mask, out, None)


def test_tile_validation():
    assert call_tile(w=weights(c_z=32)) == pra.ERR_UNSUPPORTED
    assert call_tile(n=0) == pra.ERR_INVALID_ARG
    assert call_tile(row_off=60, n_rows=50) == pra.ERR_INVALID_ARG
    assert call_tile(col_off=-2) == pra.ERR_INVALID_ARG
    assert call_tile(n_cols=0) == pra.ERR_INVALID_ARG
    assert call_tile(flags=4) == pra.ERR_INVALID_ARG
    assert call_tile(n_chunks=33, chunks=[(0, 100, 128)] * 33) == pra.ERR_INVALID_ARG
    assert call_tile(n_chunks=-1) == pra.ERR_INVALID_ARG
    assert call_tile(chunks=[], flags=pra.TILE_FIRST) == pra.ERR_INVALID_ARG
    assert call_tile(chunks=[], flags=pra.TILE_FIRST | pra.TILE_LAST) == pra.ERR_INVALID_ARG
    assert call_tile(x=None) == pra.ERR_INVALID_ARG
    assert call_tile(x=FAKE + 4) == pra.ERR_ALIGNMENT
    assert call_tile(chunks=[(0, 101, 128)]) == pra.ERR_INVALID_ARG          # past n
    assert call_tile(chunks=[(-1, 10, 64)]) == pra.ERR_INVALID_ARG
    assert call_tile(chunks=[(0, 0, 64)]) == pra.ERR_INVALID_ARG
    assert call_tile(chunks=[(0, 100, 96)]) == pra.ERR_INVALID_ARG           # ld % 64
    assert call_tile(chunks=[(0, 100, 64)]) == pra.ERR_INVALID_ARG           # ld < k_len
    assert call_tile(chunks=[(0, 60, 64), (50, 50, 64)]) == pra.ERR_INVALID_ARG  # overlap
    # FIRST|LAST must cover [0, n) exactly
    both = pra.TILE_FIRST | pra.TILE_LAST
    assert call_tile(chunks=[(0, 50, 64), (60, 40, 64)], flags=both) == pra.ERR_INVALID_ARG
    assert call_tile(chunks=[(0, 50, 64)], flags=both) == pra.ERR_INVALID_ARG
    assert "cover" in pra.lib().trimul_last_error().decode()
    assert call_tile(chunks=[(10, 90, 128)], flags=both) == pra.ERR_INVALID_ARG
    # LAST needs z, mask, out
    assert call_tile(flags=pra.TILE_LAST, z=None) == pra.ERR_INVALID_ARG
    assert call_tile(flags=pra.TILE_LAST, mask=None) == pra.ERR_INVALID_ARG
    assert call_tile(flags=pra.TILE_LAST, out=None) == pra.ERR_INVALID_ARG
    assert call_tile(flags=pra.TILE_LAST, out=FAKE + 4) == pra.ERR_ALIGNMENT
    assert "aligned" in pra.lib().trimul_last_error().decode()


def call_bwd(chunks=None, n_rows=50, n_cols=40, dx=FAKE, da=FAKE + 0x3000000, db=FAKE + 0x4000000,
             ws=FAKE + 0x8000000, ws_bytes=None, w=None, n_chunks=None, null_out=None):
    L = pra.lib()
    w = weights() if w is None else w
    if chunks is None:
        chunks = [(0, 100, 128)]
    arr = (pra.KChunk * max(1, len(chunks)))()
    for i, (ko, kl, ld) in enumerate(chunks):
        arr[i] = pra.KChunk(ko, kl, ld, FAKE + 0x1000000 * (i + 1), FAKE + 0x1000000 * (i + 40))
    nc = len(chunks) if n_chunks is None else n_chunks
    das = (ctypes.c_void_p * max(1, len(chunks)))(*([da] * max(1, len(chunks))))
    dbs = (ctypes.c_void_p * max(1, len(chunks)))(*([db] * max(1, len(chunks))))
    if null_out == "da":
        das[0] = None
    if ws_bytes is None:
        ws_bytes = L.trimul_tile_backward_workspace_bytes(ctypes.byref(w), n_rows, n_cols, arr, nc)
    return L.trimul_tile_backward(ctypes.byref(w), n_rows, n_cols, arr, nc, dx, das, dbs, ws, ws_bytes, None)


@pytest.mark.parametrize("dtype,elt", [(pra.BF16, 2), (pra.F32, 4)])
def test_backward_workspace_closed_form(dtype, elt):
    L = pra.lib()
    w = weights(dtype)
    a256 = lambda v: round_up(v, 256)
    arr = (pra.KChunk * 2)(pra.KChunk(0, 1250, 1280, FAKE, FAKE), pra.KChunk(1250, 700, 704, FAKE, FAKE))
    n_rows, n_cols, kmax = 5000, 300, 1250
    li, lj = round_up(n_rows, 64), round_up(n_cols, 64)
    want = (a256(128 * round_up(n_rows, 256) * lj * elt) + a256(128 * round_up(n_cols, 256) * li * elt)
            + a256(128 * round_up(kmax, 256) * li * elt) + a256(128 * round_up(kmax, 256) * lj * elt))
    assert L.trimul_tile_backward_workspace_bytes(ctypes.byref(w), n_rows, n_cols, arr, 2) == want
    assert L.trimul_tile_backward_workspace_bytes(ctypes.byref(w), 0, n_cols, arr, 2) == 0
    assert L.trimul_tile_backward_workspace_bytes(ctypes.byref(w), n_rows, n_cols, arr, 0) == 0


def test_backward_validation():
    assert call_bwd(w=weights(c=64)) == pra.ERR_UNSUPPORTED
    assert call_bwd(n_rows=0) == pra.ERR_INVALID_ARG
    assert call_bwd(n_cols=70000) == pra.ERR_INVALID_ARG
    assert call_bwd(chunks=[]) == pra.ERR_INVALID_ARG
    assert call_bwd(n_chunks=33, chunks=[(0, 100, 128)] * 33) == pra.ERR_INVALID_ARG
    assert call_bwd(chunks=[(0, 0, 64)]) == pra.ERR_INVALID_ARG
    assert call_bwd(chunks=[(0, 100, 96)]) == pra.ERR_INVALID_ARG        # ld % 64
    assert call_bwd(chunks=[(0, 100, 64)]) == pra.ERR_INVALID_ARG        # ld < k_len
    assert call_bwd(dx=None) == pra.ERR_INVALID_ARG
    assert call_bwd(dx=FAKE + 4) == pra.ERR_ALIGNMENT
    assert call_bwd(null_out="da") == pra.ERR_INVALID_ARG
    assert call_bwd(db=FAKE + 8) == pra.ERR_ALIGNMENT
    assert call_bwd(ws=None) == pra.ERR_INVALID_ARG
    assert call_bwd(ws=FAKE + 0x10) == pra.ERR_ALIGNMENT
    L = pra.lib()
    arr = (pra.KChunk * 1)(pra.KChunk(0, 100, 128, FAKE, FAKE))
    need = L.trimul_tile_backward_workspace_bytes(ctypes.byref(weights()), 50, 40, arr, 1)
    assert call_bwd(ws_bytes=need - 1) == pra.ERR_WORKSPACE_TOO_SMALL
    assert str(need) in L.trimul_last_error().decode()


def call_ebwd(w=None, n=100, row_off=10, n_rows=50, col_off=20, n_cols=40, x=FAKE, z=FAKE + 0x1000000,
              mask=FAKE + 0x2000000, dout=FAKE + 0x3000000, dx=FAKE + 0x4000000, dz=FAKE + 0x5000000,
              grads="ok", null_grad=None, misalign_grad=None, ws=FAKE + 0x8000000, ws_bytes=None, flags=0):
    L = pra.lib()
    w = weights() if w is None else w
    g = pra._EpilogueGrads(*[FAKE + 0x6000000 + 0x10000 * i for i in range(6)])
    if null_grad:
        setattr(g, null_grad, None)
    if misalign_grad:
        setattr(g, misalign_grad, FAKE + 0x6800000 + 4)
    gp = ctypes.byref(g) if grads == "ok" else None
    if ws_bytes is None:
        ws_bytes = L.trimul_epilogue_backward_workspace_bytes(ctypes.byref(w))
    return L.trimul_epilogue_backward(ctypes.byref(w), n, row_off, n_rows, col_off, n_cols, x, z, mask, dout, dx,
                                      dz, flags, gp, ws, ws_bytes, None)


@pytest.mark.parametrize("dtype,elt", [(pra.BF16, 2), (pra.F32, 4)])
def test_epilogue_backward_workspace_closed_form(dtype, elt):
    # transposed W_out_proj and W_out_gate, then one slot of sums plus 256
    # per-work-group slots: G and H (128 x 128 fp32 each), S and T (128 each)
    slot = round_up((2 * 128 * 128 + 2 * 128) * 4, 256)
    want = round_up(2 * 128 * 128 * elt, 256) + slot + 256 * slot
    assert pra.lib().trimul_epilogue_backward_workspace_bytes(ctypes.byref(weights(dtype))) == want
    assert pra.lib().trimul_epilogue_backward_workspace_bytes(ctypes.byref(weights(dtype, c=64))) == 0


def test_epilogue_backward_validation():
    assert call_ebwd(w=weights(c_z=64)) == pra.ERR_UNSUPPORTED
    assert call_ebwd(w=weights(null="w_out_gate")) == pra.ERR_INVALID_ARG
    assert call_ebwd(n=0) == pra.ERR_INVALID_ARG
    assert call_ebwd(n=70000) == pra.ERR_INVALID_ARG
    assert call_ebwd(row_off=60) == pra.ERR_INVALID_ARG          # rows past n
    assert call_ebwd(n_cols=0) == pra.ERR_INVALID_ARG
    assert call_ebwd(col_off=-1) == pra.ERR_INVALID_ARG
    for name in ("x", "z", "mask", "dout", "dx", "dz"):
        assert call_ebwd(**{name: None}) == pra.ERR_INVALID_ARG, name
    for name in ("x", "z", "dout", "dx", "dz"):
        assert call_ebwd(**{name: FAKE + 0x9000000 + 8}) == pra.ERR_ALIGNMENT, name
    assert call_ebwd(grads=None) == pra.ERR_INVALID_ARG
    assert call_ebwd(flags=2) == pra.ERR_INVALID_ARG
    for name in ("w_out_proj", "w_out_gate", "ln_out_w", "ln_out_b", "ln_in_w", "ln_in_b"):
        assert call_ebwd(null_grad=name) == pra.ERR_INVALID_ARG, name
        assert call_ebwd(misalign_grad=name) == pra.ERR_ALIGNMENT, name
    assert call_ebwd(ws=None) == pra.ERR_INVALID_ARG
    assert call_ebwd(ws=FAKE + 0x40) == pra.ERR_ALIGNMENT
    L = pra.lib()
    need = L.trimul_epilogue_backward_workspace_bytes(ctypes.byref(weights()))
    assert call_ebwd(ws_bytes=need - 1) == pra.ERR_WORKSPACE_TOO_SMALL
    assert str(need) in L.trimul_last_error().decode()


def call_pbwd(w=None, direction=pra.OUTGOING, n=100, row_off=10, n_rows=50, col_off=20, n_cols=40, k_off=5,
              k_len=60, z=FAKE, mask=FAKE + 0x1000000, da=FAKE + 0x2000000, db=FAKE + 0x3000000,
              dz=FAKE + 0x4000000, flags=0, grads="ok", null_grad=None, misalign_grad=None, ws=FAKE + 0x8000000,
              ws_bytes=None):
    L = pra.lib()
    w = weights() if w is None else w
    g = pra._ProjectionGrads(*[FAKE + 0x6000000 + 0x10000 * i for i in range(6)])
    if null_grad:
        setattr(g, null_grad, None)
    if misalign_grad:
        setattr(g, misalign_grad, FAKE + 0x6800000 + 4)
    gp = ctypes.byref(g) if grads == "ok" else None
    if ws_bytes is None:
        ws_bytes = L.trimul_tile_operands_backward_workspace_bytes(ctypes.byref(w))
    return L.trimul_tile_operands_backward(ctypes.byref(w), direction, z, mask, n, row_off, n_rows, col_off, n_cols,
                                           k_off, k_len, da, db, dz, flags, gp, ws, ws_bytes, None)


def test_tile_operands_backward_workspace_and_validation():
    L = pra.lib()
    for dt in (pra.BF16, pra.F32):
        assert (L.trimul_tile_operands_backward_workspace_bytes(ctypes.byref(weights(dt)))
                == L.trimul_epilogue_backward_workspace_bytes(ctypes.byref(weights(dt))))
    assert call_pbwd(w=weights(c=64)) == pra.ERR_UNSUPPORTED
    assert call_pbwd(direction=2) == pra.ERR_INVALID_ARG
    assert call_pbwd(n=0) == pra.ERR_INVALID_ARG
    assert call_pbwd(da=None, db=None) == pra.ERR_INVALID_ARG
    assert call_pbwd(row_off=60) == pra.ERR_INVALID_ARG                 # a rows past n
    assert call_pbwd(col_off=70) == pra.ERR_INVALID_ARG                 # b rows past n
    assert call_pbwd(k_off=50, k_len=60) == pra.ERR_INVALID_ARG         # k past n
    assert call_pbwd(k_len=0) == pra.ERR_INVALID_ARG
    assert call_pbwd(flags=4) == pra.ERR_INVALID_ARG
    for name in ("z", "mask", "dz"):
        assert call_pbwd(**{name: None}) == pra.ERR_INVALID_ARG, name
    for name in ("z", "dz", "da", "db"):
        assert call_pbwd(**{name: FAKE + 0x9000000 + 8}) == pra.ERR_ALIGNMENT, name
    assert call_pbwd(grads=None) == pra.ERR_INVALID_ARG
    for name in ("w_a_proj", "w_a_gate", "w_b_proj", "w_b_gate", "ln_in_w", "ln_in_b"):
        assert call_pbwd(null_grad=name) == pra.ERR_INVALID_ARG, name
        assert call_pbwd(misalign_grad=name) == pra.ERR_ALIGNMENT, name
    # a side that is not computed needs neither its rows nor its gradients
    assert call_pbwd(da=None, row_off=90, null_grad="w_a_proj", ws=None) == pra.ERR_INVALID_ARG   # fails on ws only
    assert "workspace" in L.trimul_last_error().decode()
    assert call_pbwd(ws=FAKE + 0x40) == pra.ERR_ALIGNMENT
    need = L.trimul_tile_operands_backward_workspace_bytes(ctypes.byref(weights()))
    assert call_pbwd(ws_bytes=need - 1) == pra.ERR_WORKSPACE_TOO_SMALL


def call_attn(batch=2, n=100, heads=4, d=32, q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, bias=None, mask=None,
              scale=0.17, out=FAKE + 0x300000):
    return pra.lib().trimul_atom_window_attention(batch, n, heads, d, q, k, v, bias, mask, scale, out, None)


def test_atom_window_attention_validation():
    assert call_attn(batch=0) == pra.ERR_INVALID_ARG
    assert call_attn(n=0) == pra.ERR_INVALID_ARG
    assert call_attn(d=64) == pra.ERR_UNSUPPORTED
    assert call_attn(heads=0) == pra.ERR_INVALID_ARG
    assert call_attn(heads=2000) == pra.ERR_INVALID_ARG
    assert call_attn(batch=1 << 30, n=1 << 20) == pra.ERR_INVALID_ARG
    for name in ("q", "k", "v", "out"):
        assert call_attn(**{name: None}) == pra.ERR_INVALID_ARG, name
        assert call_attn(**{name: FAKE + 0x400000 + 8}) == pra.ERR_ALIGNMENT, name
    assert call_attn(bias=FAKE + 0x500000 + 4) == pra.ERR_ALIGNMENT
    assert call_attn(scale=float("nan")) == pra.ERR_INVALID_ARG
    assert call_attn(scale=float("inf")) == pra.ERR_INVALID_ARG


def test_status_strings():
    L = pra.lib()
    for s in range(6):
        assert L.trimul_status_string(s).decode()
    assert L.trimul_status_string(99).decode() == "unknown status"


def test_binding_checks_tensors_before_calling():
    import torch
    w = type("W", (), {})()
    w.torch_dtype = torch.bfloat16
    with pytest.raises((ValueError, TypeError)):
        pra._need(torch.zeros(3), "z", torch.bfloat16)  # CPU tensor is rejected


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(pra, "_lib", None)
    monkeypatch.setattr(pra, "LIB_PATH", "/nonexistent/libtrimul.so")
    with pytest.raises(RuntimeError, match="missing"):
        pra.lib()


def test_plan_chunked_picks_fitting_blocks():
    """plan_chunked: the tallest full-width row tile with k in one chunk that
    fits the budget, else chunks of k, else square tiles; never a workspace
    beyond the budget."""
    mats = {k: torch.zeros(128, 128) for k in pra.Weights.MATRICES}
    vecs = {k: torch.zeros(128) for k in pra.Weights.VECTORS}
    w = pra.Weights({**mats, **vecs}, pra.BF16, device="cpu")
    n = 14000
    # a 288 GiB device holding z, mask and out, with 4 GiB to spare
    budget = (288 << 30) - n * n * (128 * 2 + 1 + 128 * 4) - (4 << 30)
    R, C, K = pra.plan_chunked(w, n, budget)
    assert (C, K) == (0, 0) and R % 256 == 0 and 0 < R < n
    assert pra.chunked_workspace_bytes(w, n, R, C, K) <= budget
    assert pra.chunked_workspace_bytes(w, n, R + 256, 0, 0) > budget
    small = pra.chunked_workspace_bytes(w, n, 512, 512, 512)
    R, C, K = pra.plan_chunked(w, n, small)
    assert pra.chunked_workspace_bytes(w, n, R, C, K) <= small
    assert pra.plan_chunked(w, 300, 1 << 40) == (0, 0, 0)
    with pytest.raises(ValueError):
        pra.plan_chunked(w, n, 1000)
