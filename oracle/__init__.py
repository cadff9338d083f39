"""CPU oracle for one MatRIS-MoE interaction block (TEST INFRASTRUCTURE ONLY).

This package is the plain, slow reference the GPU library is checked
against.  Only the test-suite, the smoke check and the CPU-baseline leg of
the benchmark may import it; the product path never does.  It shares no code
with the HIP library: the two meet only in the seeded input generator, which
holds no arithmetic of the method.

Everything is computed in float64 from the float32 inputs, with NumPy.  Each
function follows the plain definition of its step; where the pages leave a
step open the reading taken is stated in the function's docstring.

Sources cited below:
  [news]   ScienceAI news article on MatRIS-MoE and Janus
           ("11.5B参数、1.2EFLOPS、训练从数周压到数小时 ..."), section on the
           model architecture and on conservative training.
  [review] xllm-io paper review of "Breaking the Training Barrier of
           Billion-Parameter Universal Machine Learning Interatomic
           Potentials"; section numbers refer to that review
           (3.1 architecture / Fig. 1 / Table II, 3.2 algorithmic design,
           3.3 forces and stresses, 3.4 Fig. 3 timeline, 3.5 kernels).

Parity status per function is listed in ``PINS`` (what fixes each function
independently of itself).
"""

PINS = {
    "graph.radius_graph": "brute force (pure-Python loops) on tiny cells; lattice "
                          "closed forms (sc, fcc, self images); symmetry; degree statistics",
    "graph.radius_graph_rows": "equal to the full graph's rows on small cells",
    "block.rbf / envelope": "closed forms at r=0, mu_k, r_c; analytic derivatives vs FD",
    "block.edge_embedding": "single-basis special case; smooth vanishing at r_c",
    "block.aggregate": "e=1, s=1 gives the degree; adjoint identity; atom permutation",
    "block.route": "numpy stable argsort; gates sum to 1; k=1 gives gate 1",
    "block.dispatch_tables": "numpy stable lexsort + bincount/cumsum",
    "block.moe_forward": "shared experts reduce to one dense MLP; X=k=1; expert relabelling; "
                         "scalar closed form",
    "block.readout": "dimer closed form",
    "block.block_vjp": "float64 central finite differences (positions, node features, "
                       "homogeneous strain of positions and cell); translation/rotation/"
                       "permutation invariance; sum of forces = 0; symmetric strain gradient; "
                       "dimer closed form",
    "attention.neighbour_softmax": "scipy.special.softmax of (score + log f_c) per receiver/head; "
                                   "empty rows give 0",
    "attention.attention_forward": "one neighbour -> weights 1 and the pinned aggregation; zero "
                                   "query -> envelope-weighted mean; head relabelling / in-head "
                                   "channel permutation invariance, cross-head move changes it",
    "attention.full_block_forward": "translation/rotation/permutation invariance; energy "
                                    "continuous (quadratic) across r_c",
    "attention.full_block_vjp": "float64 central finite differences (positions, node features, "
                                "strain per structure); sum of forces = 0; virial shares add up",
    "tri.legendre": "numpy.polynomial.legendre values",
    "tri.tri_row / tri_forward": "P_0 and P_1 closed forms (squared sums minus squares); a "
                                 "three-atom angle against numpy Legendre values",
    "tri.tri_vjp": "float64 central finite differences (positions, strain, node features), "
                   "alone and inside the complete block",
    "stack.stack_forward / stack_vjp": "float64 central finite differences through 2 and 6 "
                                       "blocks (positions, strain); sum of forces = 0; rotation",
    "train.loss_grads": "energies/forces equal block.block_forward/block_vjp; every parameter "
                        "gradient vs float64 central finite differences of L built from "
                        "oracle.block; the energy part equals block_vjp's input gradient",
}
