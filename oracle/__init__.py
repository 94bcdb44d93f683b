"""Float64 CPU oracle for the triangle multiplicative update.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
its Python binding) imports, links or calls anything in this package; only the
test-suite, the smoke check and the benchmark's CPU-baseline leg do.  It shares
no code with the HIP path: the only thing both sides consume is the seeded
input data produced by the ``workloads`` package, which holds none of the
method's arithmetic.

What it computes follows the layer that page 1 ("NVIDIA BioNeMo escala
modelagem biomolecular com context parallelism ...", section "Exemplo de
codigo: triangle multiplication CP-aware") instantiates as
``TriangleMultiplicationOutgoing(size_input_embed)`` and calls as
``layer(x, mask)``.  The pages name the layer but do not write its equations;
the oracle takes the AlphaFold3-style definition (input LayerNorm, gated a/b
projections, the k-contraction outgoing  x_ij = sum_k a_ik * b_jk  or incoming
x_ij = sum_k a_ki * b_kj, output LayerNorm, output projection, output gate,
pair mask).  Page 1's "2D tiling da pair representation" section is the
source of the tiled (sub-block) evaluation in ``tile_partial``.

Modules
-------
trimul_ref   vectorised float64 definition, Q-mode (bf16 contraction operands),
             blockwise and sampled evaluation, tile partial sums, and the
             gradients of the projections, the contraction step, the
             epilogue and the whole layer.
bruteforce   per-element scalar loops of the same definitions, for tiny inputs.
atom_attention  window-batched sequence-local atom attention (32-query blocks,
             128-key windows; page 1, "Atom sequence local attention eficiente").

Parity status: every function here is pinned by the CPU tests in
``tests/test_oracle.py`` and ``tests/test_oracle_atom.py`` (brute force, closed forms, invariants, library
special cases).  No function is "parity unpinned".
"""

from .trimul_ref import (  # noqa: F401
    LN_EPS,
    WEIGHT_KEYS,
    array_getters,
    contract_rows,
    contract_rows_vjp,
    bf16_round,
    contract,
    finish,
    finish_vjp,
    layer_norm,
    project,
    project_vjp,
    sigmoid,
    tile_partial,
    trimul,
    trimul_blockwise,
    trimul_vjp,
    trimul_sampled,
)
