"""CPU oracle for the equivariant message-passing convolution (TEST INFRASTRUCTURE).

This package is a plain, slow, obviously-correct fp64 implementation of the
convolution

    m_b = (1/N) * sum_{a -> b} (x_a (x) y_ab) (.) s_ab

as defined on the e3j ``Convolution`` API page (class description, the
formula, and the unfused JAX implementation the page describes: each edge
takes its sender's row of x, forms the product with its harmonics y,
weights it by its scalars s, and is summed into its receiver's row, with
the sum scaled by 1/avg_num_neighbors).

It exists only to check the HIP implementation.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  It shares no code with the HIP path: the irreps parser, the path
enumeration, the Racah Clebsch-Gordan builder, the real basis, the Wigner D
matrices and the convolution itself are all written here independently.

Modules
-------
irreps  -- irreps string parser (``"8x0e+8x1o"``, ``"64x(0e+1o+2e)"``).
so3     -- Racah complex CG, complex->real basis change, real CG tensors,
           real Wigner D matrices from the exponential map of generators.
conv    -- path enumeration, brute-force and vectorised forward, backward.
variants -- SENDER graph ordering, pair storage (one row of y and s per
           undirected pair), node_mask padding, forward-mode and second
           derivatives, built from ``conv``.
linear  -- the output linear (channel mixing per irrep block) and its gradients.
radial  -- edge scalars from edge lengths (radial basis, cutoff, two-layer
           network) and the convolution they feed.

Pins (what ties this oracle to something other than itself) live in
``tests/test_oracle_*.py``; every function here is pinned there.
"""

from . import irreps, so3, conv, variants, linear, radial  # noqa: F401
