"""CPU oracle for the token-choice MoE forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
load anything under ``oracle/``; only ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` do.  The oracle shares no code with
the HIP library (no kernels, headers, helpers or constant tables); the only
module both sides use is ``synth`` (seeded input tensors, no layer arithmetic).

* ``moe``    -- the plain definition in float64 (numpy), one function per step.
* ``fp32spec`` -- the float32 sigmoid selection key, step by step.
* ``brute``  -- a pure-Python per-token loop for tiny inputs, written
  independently of ``moe`` so that each checks the other.
* ``backward`` -- the chain rule of ``moe``'s layer (gradients of the input,
  router and expert weights, with the balance and z-loss terms), pinned by
  finite differences of the forward definition.
"""

