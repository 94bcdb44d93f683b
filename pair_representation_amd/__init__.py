"""Python binding of libtrimul.so, the gfx950 triangle multiplicative update.

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, their data pointers and torch's current HIP stream are handed to
the C entry points declared in include/trimul.h, and a non-OK status becomes a
``TrimulError``.  Every step of the computation runs in the HIP kernels; there
is no fallback.  If the library has not been built, the first call raises.

Entry points (same names as the C ABI, without the ``trimul_`` prefix):
    workspace_bytes(w, n)
    outgoing(z, mask, w, ...), incoming(z, mask, w, ...)
    chunked_workspace_bytes(w, n, row_block, col_block, k_block)
    forward_chunked(z, mask, w, direction, row_block, col_block, k_block, ...)
    forward_chunked_noalloc(z, mask, w, direction, row_block, col_block, k_block, out=None)
    plan_chunked(w, n, budget_bytes)   (host helper: blocks whose workspace fits a budget)
    tile_operand_bytes(w, rows, ld)
    tile_operands(w, direction, z, mask, row_off, n_rows, col_off, n_cols, k_off, k_len, ld, ...)
    tile(w, n, row_off, n_rows, col_off, n_cols, chunks, flags, x_acc, z, mask, out_tile)
    tile_backward_workspace_bytes(w, n_rows, n_cols, chunks)
    tile_backward(w, n_rows, n_cols, chunks, dx, ...)
    epilogue_backward_workspace_bytes(w)
    epilogue_backward(w, n, row_off, n_rows, col_off, n_cols, x_acc, z, mask, dout, ...)
    tile_operands_backward_workspace_bytes(w)
    tile_operands_backward(w, direction, z, mask, row_off, n_rows, col_off, n_cols, k_off, k_len, da, db, dz, ...)
    atom_window_attention(q, k, v, bias=None, atom_mask=None, scale=None, out=None)
"""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtrimul.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_ALIGNMENT, ERR_WORKSPACE_TOO_SMALL, ERR_HIP = range(6)
F32, BF16 = 0, 1
OUTGOING, INCOMING = 0, 1
TILE_FIRST, TILE_LAST = 1, 2
MAX_CHUNKS = 32
C = 128
C_Z = 128


class TrimulError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"trimul status {status}: {message}")
        self.status = status
        self.message = message


class _Weights(ctypes.Structure):
    _fields_ = [
        ("c_z", ctypes.c_int32), ("c", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("ln_eps", ctypes.c_float),
        ("ln_in_w", ctypes.c_void_p), ("ln_in_b", ctypes.c_void_p),
        ("w_a_proj", ctypes.c_void_p), ("w_a_gate", ctypes.c_void_p),
        ("w_b_proj", ctypes.c_void_p), ("w_b_gate", ctypes.c_void_p),
        ("w_out_gate", ctypes.c_void_p),
        ("ln_out_w", ctypes.c_void_p), ("ln_out_b", ctypes.c_void_p),
        ("w_out_proj", ctypes.c_void_p),
    ]


class KChunk(ctypes.Structure):
    _fields_ = [("k_off", ctypes.c_int64), ("k_len", ctypes.c_int64), ("ld", ctypes.c_int64),
                ("a", ctypes.c_void_p), ("b", ctypes.c_void_p)]


class _EpilogueGrads(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in
                ("w_out_proj", "w_out_gate", "ln_out_w", "ln_out_b", "ln_in_w", "ln_in_b")]


class _ProjectionGrads(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in
                ("w_a_proj", "w_a_gate", "w_b_proj", "w_b_gate", "ln_in_w", "ln_in_b")]


PROJECTION_GRAD_SHAPES = {"w_a_proj": (C, C_Z), "w_a_gate": (C, C_Z), "w_b_proj": (C, C_Z), "w_b_gate": (C, C_Z),
                          "ln_in_w": (C_Z,), "ln_in_b": (C_Z,)}
GRAD_ACCUMULATE = 1

EPILOGUE_GRAD_SHAPES = {"w_out_proj": (C_Z, C), "w_out_gate": (C_Z, C_Z), "ln_out_w": (C,), "ln_out_b": (C,),
                        "ln_in_w": (C_Z,), "ln_in_b": (C_Z,)}

_lib = None


def lib():
    """The loaded C library (loaded on first use; raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m pair_representation_amd.build` (needs hipcc)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, u32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32, ctypes.c_size_t
        W = ctypes.POINTER(_Weights)
        L.trimul_workspace_bytes.argtypes = [W, i64]
        L.trimul_workspace_bytes.restype = sz
        for name in ("trimul_outgoing", "trimul_incoming"):
            f = getattr(L, name)
            f.argtypes = [W, vp, vp, vp, i64, vp, sz, vp]
            f.restype = ctypes.c_int
        L.trimul_chunked_workspace_bytes.argtypes = [W, i64, i64, i64, i64]
        L.trimul_chunked_workspace_bytes.restype = sz
        L.trimul_forward_chunked.argtypes = [W, ctypes.c_int, vp, vp, vp, i64, i64, i64, i64, vp, sz, vp]
        L.trimul_forward_chunked.restype = ctypes.c_int
        L.trimul_forward_chunked_noalloc.argtypes = [W, ctypes.c_int, vp, vp, vp, i64, i64, i64, i64, vp]
        L.trimul_forward_chunked_noalloc.restype = ctypes.c_int
        L.trimul_tile_operand_bytes.argtypes = [W, i64, i64]
        L.trimul_tile_operand_bytes.restype = sz
        L.trimul_tile_xacc_bytes.argtypes = [W, i64, i64]
        L.trimul_tile_xacc_bytes.restype = sz
        L.trimul_tile_operands.argtypes = [W, ctypes.c_int, vp, vp, i64, i64, i64, i64, i64, i64, i64,
                                           i64, vp, vp, vp]
        L.trimul_tile_operands.restype = ctypes.c_int
        L.trimul_tile.argtypes = [W, i64, i64, i64, i64, i64, ctypes.POINTER(KChunk), i32, u32, vp, vp,
                                  vp, vp, vp]
        L.trimul_tile.restype = ctypes.c_int
        L.trimul_tile_backward_workspace_bytes.argtypes = [W, i64, i64, ctypes.POINTER(KChunk), i32]
        L.trimul_tile_backward_workspace_bytes.restype = sz
        L.trimul_tile_backward.argtypes = [W, i64, i64, ctypes.POINTER(KChunk), i32, vp,
                                           ctypes.POINTER(vp), ctypes.POINTER(vp), vp, sz, vp]
        L.trimul_tile_backward.restype = ctypes.c_int
        L.trimul_epilogue_backward_workspace_bytes.argtypes = [W]
        L.trimul_epilogue_backward_workspace_bytes.restype = sz
        L.trimul_epilogue_backward.argtypes = [W, i64, i64, i64, i64, i64, vp, vp, vp, vp, vp, vp, u32,
                                               ctypes.POINTER(_EpilogueGrads), vp, sz, vp]
        L.trimul_epilogue_backward.restype = ctypes.c_int
        L.trimul_tile_operands_backward_workspace_bytes.argtypes = [W]
        L.trimul_tile_operands_backward_workspace_bytes.restype = sz
        L.trimul_tile_operands_backward.argtypes = [W, ctypes.c_int, vp, vp, i64, i64, i64, i64, i64, i64, i64,
                                                    vp, vp, vp, u32, ctypes.POINTER(_ProjectionGrads), vp, sz, vp]
        L.trimul_tile_operands_backward.restype = ctypes.c_int
        L.trimul_atom_window_attention.argtypes = [i64, i64, i32, i32, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp]
        L.trimul_atom_window_attention.restype = ctypes.c_int
        L.trimul_status_string.argtypes = [ctypes.c_int]
        L.trimul_status_string.restype = ctypes.c_char_p
        L.trimul_last_error.argtypes = []
        L.trimul_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(status):
    if status != OK:
        raise TrimulError(status, lib().trimul_last_error().decode())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


_TORCH_DTYPE = {F32: torch.float32, BF16: torch.bfloat16}


class Weights:
    """Device-resident layer parameters plus the C struct pointing at them.

    ``tensors`` maps the names of trimul_weights_t (ln_in_w, ln_in_b, w_a_proj,
    w_a_gate, w_b_proj, w_b_gate, w_out_gate, ln_out_w, ln_out_b, w_out_proj)
    to tensors; matrices are (out_features, in_features).  They are copied to
    ``device`` in the storage dtype (matrices) and fp32 (LayerNorm vectors).
    """

    MATRICES = ("w_a_proj", "w_a_gate", "w_b_proj", "w_b_gate", "w_out_gate", "w_out_proj")
    VECTORS = ("ln_in_w", "ln_in_b", "ln_out_w", "ln_out_b")

    def __init__(self, tensors, dtype=BF16, eps=1e-5, device="cuda"):
        self.dtype = dtype
        td = _TORCH_DTYPE[dtype]
        self.t = {}
        for k in self.MATRICES:
            self.t[k] = tensors[k].to(device=device, dtype=td).contiguous()
        for k in self.VECTORS:
            self.t[k] = tensors[k].to(device=device, dtype=torch.float32).contiguous()
        s = _Weights()
        s.c_z, s.c, s.dtype, s.ln_eps = C_Z, C, dtype, eps
        for k, v in self.t.items():
            setattr(s, k, v.data_ptr())
        self.struct = s

    @property
    def ref(self):
        return ctypes.byref(self.struct)

    @property
    def torch_dtype(self):
        return _TORCH_DTYPE[self.dtype]


def workspace_bytes(w: Weights, n: int) -> int:
    return int(lib().trimul_workspace_bytes(w.ref, n))


def tile_operand_bytes(w: Weights, rows: int, ld: int) -> int:
    return int(lib().trimul_tile_operand_bytes(w.ref, rows, ld))


def new_workspace(w: Weights, n: int, device="cuda"):
    nb = workspace_bytes(w, n)
    return torch.empty(max(nb, 256), dtype=torch.uint8, device=device)


def _full(fn, z, mask, w, workspace, out):
    n = z.shape[0]
    _need(z, "z", w.torch_dtype, (n, n, C_Z))
    _need(mask, "mask", torch.uint8, (n, n))
    if out is None:
        out = torch.empty((n, n, C_Z), dtype=torch.float32, device=z.device)
    _need(out, "out", torch.float32, (n, n, C_Z))
    if workspace is None:
        workspace = new_workspace(w, n, z.device)
    _need(workspace, "workspace", torch.uint8)
    _check(fn(w.ref, _ptr(z), _ptr(mask), _ptr(out), n, _ptr(workspace), workspace.numel(), _stream()))
    return out


def outgoing(z, mask, w: Weights, workspace=None, out=None):
    """out_ij = update with x_ij = sum_k a_ik * b_jk; returns fp32 [n, n, 128]."""
    return _full(lib().trimul_outgoing, z, mask, w, workspace, out)


def incoming(z, mask, w: Weights, workspace=None, out=None):
    """out_ij = update with x_ij = sum_k a_ki * b_kj; returns fp32 [n, n, 128]."""
    return _full(lib().trimul_incoming, z, mask, w, workspace, out)


def chunked_workspace_bytes(w: Weights, n: int, row_block: int = 0, col_block: int = 0, k_block: int = 0) -> int:
    return int(lib().trimul_chunked_workspace_bytes(w.ref, n, row_block, col_block, k_block))


def forward_chunked(z, mask, w: Weights, direction: int, row_block: int = 0, col_block: int = 0, k_block: int = 0,
                    workspace=None, out=None):
    """The update (direction OUTGOING or INCOMING) in bounded device memory:
    R x C output tiles, each contracting k in chunks of K (0 = n); the
    workspace holds one tile's operands and accumulator
    (chunked_workspace_bytes).  Returns fp32 [n, n, 128]."""
    n = z.shape[0]
    _need(z, "z", w.torch_dtype, (n, n, C_Z))
    _need(mask, "mask", torch.uint8, (n, n))
    if out is None:
        out = torch.empty((n, n, C_Z), dtype=torch.float32, device=z.device)
    _need(out, "out", torch.float32, (n, n, C_Z))
    if workspace is None:
        nb = chunked_workspace_bytes(w, n, row_block, col_block, k_block)
        workspace = torch.empty(max(nb, 256), dtype=torch.uint8, device=z.device)
    _need(workspace, "workspace", torch.uint8)
    _check(lib().trimul_forward_chunked(w.ref, direction, _ptr(z), _ptr(mask), _ptr(out), n, row_block, col_block,
                                        k_block, _ptr(workspace), workspace.numel(), _stream()))
    return out


def plan_chunked(w: Weights, n: int, budget_bytes: int):
    """Blocks (row_block, col_block, k_block) for forward_chunked whose
    workspace fits in ``budget_bytes``, in order of preference: k in one
    chunk at full width (each operand built once; the tallest row tile that
    fits, in multiples of 256 rows), then k in chunks at full width, then
    square tiles.  Sizes come from chunked_workspace_bytes; raises
    ValueError when not even 256 x 256 x 256 blocks fit."""
    if n < 1:
        raise ValueError("n must be positive")

    def fits(r, c, k):
        return chunked_workspace_bytes(w, n, r, c, k) <= budget_bytes

    rows = sorted({n} | set(range(256, n, 256)), reverse=True)
    for r in rows:
        if fits(r, 0, 0):
            return (0 if r >= n else r, 0, 0)
    ks = [k for k in (n // 2, n // 4, n // 8, 1024, 512, 256) if 64 <= k < n]
    for k in sorted({(k + 63) // 64 * 64 for k in ks}, reverse=True):
        for r in rows:
            if fits(r, 0, k):
                return (0 if r >= n else r, 0, k)
    for b in (4096, 2048, 1024, 512, 256):
        b = min(b, n)
        if fits(b, b, b):
            return (b, b, b)
    raise ValueError(f"no blocks fit a workspace of {budget_bytes} bytes at n={n}")


NOALLOC_SCRATCH_BYTES = 256 << 20   # TRIMUL_NOALLOC_SCRATCH_BYTES


def forward_chunked_noalloc(z, mask, w: Weights, direction: int, row_block: int = 0, col_block: int = 0,
                            k_block: int = 0, out=None):
    """forward_chunked with the workspace in the library's device scratch
    array (no allocation by the library; ``out`` is allocated here only when
    not given).  The blocks' workspace must fit in NOALLOC_SCRATCH_BYTES.
    Calls that overlap on one device race on the shared array."""
    n = z.shape[0]
    _need(z, "z", w.torch_dtype, (n, n, C_Z))
    _need(mask, "mask", torch.uint8, (n, n))
    if out is None:
        out = torch.empty((n, n, C_Z), dtype=torch.float32, device=z.device)
    _need(out, "out", torch.float32, (n, n, C_Z))
    _check(lib().trimul_forward_chunked_noalloc(w.ref, direction, _ptr(z), _ptr(mask), _ptr(out), n, row_block,
                                                col_block, k_block, _stream()))
    return out


def operand_shape(rows, ld):
    """Shape of one operand buffer in the library's operand layout: blocks of
    256 rows x 64 columns, the 128 channel blocks of a block adjacent:
    [ceil(rows/256), ld/64, 128, 256, 64]."""
    return ((rows + 255) // 256, ld // 64, C, 256, 64)


def new_operand(rows, ld, dtype, device="cuda"):
    return torch.empty(operand_shape(rows, ld), dtype=dtype, device=device)


def operand_to_planar(op, rows):
    """[128, rows, ld] copy of an operand buffer (layout conversion only)."""
    rb, kb = op.shape[0], op.shape[1]
    return op.permute(2, 0, 3, 1, 4).reshape(C, rb * 256, kb * 64)[:, :rows]


def planar_to_operand(planar):
    """Operand buffer holding planar [128, rows, ld] (rows zero-padded to 256)."""
    _, rows, ld = planar.shape
    rb = (rows + 255) // 256
    full = torch.zeros((C, rb * 256, ld), dtype=planar.dtype, device=planar.device)
    full[:, :rows] = planar
    return full.reshape(C, rb, 256, ld // 64, 64).permute(1, 3, 0, 2, 4).contiguous()


def tile_operands(w: Weights, direction, z, mask, row_off, n_rows, col_off, n_cols, k_off, k_len, ld,
                  a_out=None, b_out=None, want_a=True, want_b=True):
    """Operand chunk (operand layout, see operand_shape) for one tile and
    k-range; returns (a, b)."""
    n = z.shape[0]
    _need(z, "z", w.torch_dtype, (n, n, C_Z))
    _need(mask, "mask", torch.uint8, (n, n))
    if want_a and a_out is None:
        a_out = new_operand(n_rows, ld, w.torch_dtype, z.device)
    if want_b and b_out is None:
        b_out = new_operand(n_cols, ld, w.torch_dtype, z.device)
    if a_out is not None:
        _need(a_out, "a_out", w.torch_dtype, operand_shape(n_rows, ld))
    if b_out is not None:
        _need(b_out, "b_out", w.torch_dtype, operand_shape(n_cols, ld))
    _check(lib().trimul_tile_operands(w.ref, direction, _ptr(z), _ptr(mask), n, row_off, n_rows, col_off,
                                      n_cols, k_off, k_len, ld, _ptr(a_out), _ptr(b_out), _stream()))
    return a_out, b_out


def tile_xacc_bytes(w: Weights, n_rows: int, n_cols: int) -> int:
    return int(lib().trimul_tile_xacc_bytes(w.ref, n_rows, n_cols))


def xacc_shape(n_rows, n_cols):
    """Shape of a tile accumulator: blocks of 4 rows x 16 columns, the 128
    channels of a block adjacent: [ceil(n_rows/4), ceil(n_cols/16), 128, 16, 4]."""
    return ((n_rows + 3) // 4, (n_cols + 15) // 16, C, 16, 4)


def new_xacc(n_rows, n_cols, device="cuda"):
    """Tile accumulator (uninitialised fp32, see xacc_shape)."""
    return torch.empty(xacc_shape(n_rows, n_cols), dtype=torch.float32, device=device)


def xacc_to_planar(x_acc, n_rows, n_cols):
    """[128, n_rows, n_cols] copy of an accumulator (layout conversion only)."""
    rb, cb = x_acc.shape[0], x_acc.shape[1]
    return x_acc.permute(2, 0, 4, 1, 3).reshape(C, rb * 4, cb * 16)[:, :n_rows, :n_cols]


def tile(w: Weights, n, row_off, n_rows, col_off, n_cols, chunks, flags, x_acc, z=None, mask=None,
         out_tile=None):
    """Contract ``chunks`` (list of (k_off, k_len, a, b) in arrival order) into
    x_acc (see new_xacc for its layout); with TILE_LAST also write out_tile
    [n_rows, n_cols, 128] fp32 (allocated if None).  Returns out_tile."""
    _need(x_acc, "x_acc", torch.float32, xacc_shape(n_rows, n_cols))
    arr = (KChunk * max(1, len(chunks)))()
    for i, (k_off, k_len, a, b) in enumerate(chunks):
        _need(a, f"chunk {i} a", w.torch_dtype)
        _need(b, f"chunk {i} b", w.torch_dtype)
        ld = a.shape[1] * 64 if a.dim() == 5 else -1
        if tuple(a.shape) != operand_shape(n_rows, ld):
            raise ValueError(f"chunk {i} a must have shape operand_shape({n_rows}, ld)")
        if tuple(b.shape) != operand_shape(n_cols, ld):
            raise ValueError(f"chunk {i} b must have shape operand_shape({n_cols}, ld) with a's ld")
        arr[i] = KChunk(k_off, k_len, ld, a.data_ptr(), b.data_ptr())
    if flags & TILE_LAST:
        _need(z, "z", w.torch_dtype, (n, n, C_Z))
        _need(mask, "mask", torch.uint8, (n, n))
        if out_tile is None:
            out_tile = torch.empty((n_rows, n_cols, C_Z), dtype=torch.float32, device=x_acc.device)
        _need(out_tile, "out_tile", torch.float32, (n_rows, n_cols, C_Z))
    _check(lib().trimul_tile(w.ref, n, row_off, n_rows, col_off, n_cols, arr, len(chunks), flags,
                             _ptr(x_acc), _ptr(z), _ptr(mask), _ptr(out_tile), _stream()))
    return out_tile


def _chunk_array(w: Weights, n_rows, n_cols, chunks):
    arr = (KChunk * max(1, len(chunks)))()
    for i, (k_off, k_len, a, b) in enumerate(chunks):
        _need(a, f"chunk {i} a", w.torch_dtype)
        _need(b, f"chunk {i} b", w.torch_dtype)
        ld = a.shape[1] * 64 if a.dim() == 5 else -1
        if tuple(a.shape) != operand_shape(n_rows, ld):
            raise ValueError(f"chunk {i} a must have shape operand_shape({n_rows}, ld)")
        if tuple(b.shape) != operand_shape(n_cols, ld):
            raise ValueError(f"chunk {i} b must have shape operand_shape({n_cols}, ld) with a's ld")
        arr[i] = KChunk(k_off, k_len, ld, a.data_ptr(), b.data_ptr())
    return arr


def tile_backward_workspace_bytes(w: Weights, n_rows, n_cols, chunks) -> int:
    return int(lib().trimul_tile_backward_workspace_bytes(w.ref, n_rows, n_cols,
                                                          _chunk_array(w, n_rows, n_cols, chunks), len(chunks)))


def tile_backward(w: Weights, n_rows, n_cols, chunks, dx, da=None, db=None, workspace=None):
    """Gradients of a tile's contraction with respect to the chunk operands.

    ``chunks`` is a list of (k_off, k_len, a, b) as for tile(); ``dx`` is the
    gradient of the tile's contraction result in the accumulator layout
    (xacc_shape(n_rows, n_cols), fp32).  Returns (da, db): per chunk, fp32
    accumulator-layout tensors of shapes xacc_shape(n_rows, k_len) and
    xacc_shape(n_cols, k_len) (allocated if not given)."""
    _need(dx, "dx", torch.float32, xacc_shape(n_rows, n_cols))
    arr = _chunk_array(w, n_rows, n_cols, chunks)
    if da is None:
        da = [new_xacc(n_rows, k_len, dx.device) for (_, k_len, _, _) in chunks]
    if db is None:
        db = [new_xacc(n_cols, k_len, dx.device) for (_, k_len, _, _) in chunks]
    for i, (_, k_len, _, _) in enumerate(chunks):
        _need(da[i], f"da[{i}]", torch.float32, xacc_shape(n_rows, k_len))
        _need(db[i], f"db[{i}]", torch.float32, xacc_shape(n_cols, k_len))
    need = int(lib().trimul_tile_backward_workspace_bytes(w.ref, n_rows, n_cols, arr, len(chunks)))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dx.device)
    _need(workspace, "workspace", torch.uint8)
    da_ptrs = (ctypes.c_void_p * len(chunks))(*[t.data_ptr() for t in da])
    db_ptrs = (ctypes.c_void_p * len(chunks))(*[t.data_ptr() for t in db])
    _check(lib().trimul_tile_backward(w.ref, n_rows, n_cols, arr, len(chunks), _ptr(dx), da_ptrs, db_ptrs,
                                      _ptr(workspace), workspace.numel(), _stream()))
    return da, db


def epilogue_backward_workspace_bytes(w: Weights) -> int:
    return int(lib().trimul_epilogue_backward_workspace_bytes(w.ref))


def epilogue_backward(w: Weights, n, row_off, n_rows, col_off, n_cols, x_acc, z, mask, dout, dx=None, dz=None,
                      grads=None, workspace=None, accumulate=False):
    """Backward of a tile's epilogue.

    ``x_acc`` is the tile's contraction result (accumulator layout, as
    tile() leaves it), ``z``/``mask`` the global [n, n] tensors and ``dout``
    the gradient of the tile's output [n_rows, n_cols, 128] fp32.  Returns
    (dx, dz, grads): dx in the accumulator layout (may be passed as x_acc
    itself), dz [n_rows, n_cols, 128] (the output gate's share of dL/dz) and a
    dict of fp32 parameter gradients keyed as EPILOGUE_GRAD_SHAPES (allocated
    when not given; with ``accumulate`` the gradients are added to them)."""
    _need(x_acc, "x_acc", torch.float32, xacc_shape(n_rows, n_cols))
    _need(z, "z", w.torch_dtype, (n, n, C_Z))
    _need(mask, "mask", torch.uint8, (n, n))
    _need(dout, "dout", torch.float32, (n_rows, n_cols, C_Z))
    dev = x_acc.device
    if dx is None:
        dx = new_xacc(n_rows, n_cols, dev)
    if dz is None:
        dz = torch.empty((n_rows, n_cols, C_Z), dtype=torch.float32, device=dev)
    _need(dx, "dx", torch.float32, xacc_shape(n_rows, n_cols))
    _need(dz, "dz", torch.float32, (n_rows, n_cols, C_Z))
    if grads is None:
        grads = {k: torch.empty(shp, dtype=torch.float32, device=dev) for k, shp in EPILOGUE_GRAD_SHAPES.items()}
    for k, shp in EPILOGUE_GRAD_SHAPES.items():
        _need(grads[k], f"grads[{k!r}]", torch.float32, shp)
    g = _EpilogueGrads(*[grads[k].data_ptr() for k in EPILOGUE_GRAD_SHAPES])
    need = epilogue_backward_workspace_bytes(w)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8)
    _check(lib().trimul_epilogue_backward(w.ref, n, row_off, n_rows, col_off, n_cols, _ptr(x_acc), _ptr(z),
                                          _ptr(mask), _ptr(dout), _ptr(dx), _ptr(dz),
                                          GRAD_ACCUMULATE if accumulate else 0, ctypes.byref(g),
                                          _ptr(workspace), workspace.numel(), _stream()))
    return dx, dz, grads


def tile_operands_backward_workspace_bytes(w: Weights) -> int:
    return int(lib().trimul_tile_operands_backward_workspace_bytes(w.ref))


def tile_operands_backward(w: Weights, direction, z, mask, row_off, n_rows, col_off, n_cols, k_off, k_len,
                           da=None, db=None, dz=None, grads=None, accumulate=False, workspace=None):
    """Backward of tile_operands: adds the projections' share of dL/dz to
    ``dz`` ([n, n, 128] fp32, zeros allocated if None) and writes (or with
    ``accumulate`` adds) the projection parameters' gradients into ``grads``
    (dict keyed as PROJECTION_GRAD_SHAPES; allocated if None).  ``da`` / ``db``
    are the gradients of the chunk's operands in the accumulator layout
    (xacc_shape(n_rows, k_len) / xacc_shape(n_cols, k_len)), as tile_backward
    returns them; either may be None.  Returns (dz, grads)."""
    n = z.shape[0]
    _need(z, "z", w.torch_dtype, (n, n, C_Z))
    _need(mask, "mask", torch.uint8, (n, n))
    if da is None and db is None:
        raise ValueError("da and db are both None")
    if da is not None:
        _need(da, "da", torch.float32, xacc_shape(n_rows, k_len))
    if db is not None:
        _need(db, "db", torch.float32, xacc_shape(n_cols, k_len))
    dev = z.device
    if dz is None:
        dz = torch.zeros((n, n, C_Z), dtype=torch.float32, device=dev)
    _need(dz, "dz", torch.float32, (n, n, C_Z))
    if grads is None:
        grads = {k: torch.empty(shp, dtype=torch.float32, device=dev) for k, shp in PROJECTION_GRAD_SHAPES.items()}
    ptrs = []
    for k, shp in PROJECTION_GRAD_SHAPES.items():
        used = (k.startswith("w_a") and da is not None) or (k.startswith("w_b") and db is not None) \
            or k.startswith("ln_in")
        if used:
            _need(grads[k], f"grads[{k!r}]", torch.float32, shp)
            ptrs.append(grads[k].data_ptr())
        else:
            ptrs.append(grads[k].data_ptr() if grads.get(k) is not None else None)
    g = _ProjectionGrads(*ptrs)
    need = tile_operands_backward_workspace_bytes(w)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8)
    _check(lib().trimul_tile_operands_backward(w.ref, direction, _ptr(z), _ptr(mask), n, row_off, n_rows, col_off,
                                               n_cols, k_off, k_len, _ptr(da), _ptr(db), _ptr(dz),
                                               GRAD_ACCUMULATE if accumulate else 0, ctypes.byref(g),
                                               _ptr(workspace), workspace.numel(), _stream()))
    return dz, grads


def atom_window_attention(q, k, v, bias=None, atom_mask=None, scale=None, out=None):
    """Window-batched sequence-local atom attention (32-atom query blocks, each
    attending to the 128 atoms centred on it).  q, k, v: bf16 [batch, n_atoms,
    heads, 32]; bias: bf16 [batch, ceil(n_atoms / 32), heads, 32, 128] or None;
    atom_mask: uint8 [batch, n_atoms] or None (keys only); scale defaults to
    1/sqrt(32).  Returns out, fp32 [batch, n_atoms, heads, 32]."""
    _need(q, "q", torch.bfloat16)
    if q.dim() != 4:
        raise ValueError("q must be [batch, n_atoms, heads, head_dim]")
    bsz, n, heads, d = q.shape
    _need(k, "k", torch.bfloat16, q.shape)
    _need(v, "v", torch.bfloat16, q.shape)
    nw = (n + 31) // 32
    if bias is not None:
        _need(bias, "bias", torch.bfloat16, (bsz, nw, heads, 32, 128))
    if atom_mask is not None:
        _need(atom_mask, "atom_mask", torch.uint8, (bsz, n))
    if out is None:
        out = torch.empty((bsz, n, heads, d), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, (bsz, n, heads, d))
    if scale is None:
        scale = d ** -0.5
    _check(lib().trimul_atom_window_attention(bsz, n, heads, d, _ptr(q), _ptr(k), _ptr(v), _ptr(bias),
                                              _ptr(atom_mask), float(scale), _ptr(out), _stream()))
    return out
