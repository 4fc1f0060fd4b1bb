"""CPU oracle for MLA with decoupled RoPE, weight-absorbed form.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
its Python binding) may import, call or link anything here.  Only the test
suite, the smoke check and the CPU-baseline leg of the benchmark use it.

Everything here is plain, slow, float64 numpy written from the pages'
equations:

* ``rope``        -- the rotary position operator R_p (RoFormer Theta, pairs
                     (2j, 2j+1)).
* ``attention``   -- the materialised definition (K = [W_UK c ; R_t k^R],
                     V = W_UV c, plain softmax attention), which is the
                     spec; the absorbed twin (q~ = W_UK^T q^C, score against
                     the latent), used only as a self-check; and a brute-force
                     pure-Python version for tiny cases.
* ``paging``      -- where a (sequence, position) lands in a paged cache.
* ``accounting``  -- per-token cache sizes of the layouts the pages compare.
* ``front``       -- the projections in front of the cache: the latent
                     c = W_DKV h, the position key W_KR h, the query latent
                     c^Q = W_DQ h and its content / position projections, and
                     the folded query weight W_UK^T W_UQ.
* ``obstruction`` -- why the rotated key cannot be absorbed: the position-
                     operator family W_QR^T R_delta W_UKR, its span over the
                     shifts, and the best single matrix with its residual.

No function here shares code with the GPU path, and none reads any value the
GPU produced.
"""

from . import accounting, attention, front, obstruction, paging, rope  # noqa: F401
