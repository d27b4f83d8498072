"""fp64 CPU oracle for the fused attention forward.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product (the HIP library and its
Python binding) never imports, links or calls anything here, and this package
imports nothing from the product: the two share no code.

Modules
-------
``definition`` the plain definition: materialise the scaled scores (row chunk
               by row chunk), subtract the row max, exponentiate, sum,
               normalise, multiply by V; also the log-sum-exp.  This is the
               oracle every parity test compares against.
``online``     the online-softmax recurrence the pages derive (running max m,
               running exp-sum l, rescaled accumulator), in fp64, used only to
               pin "one pass equals two passes" on the oracle itself.
``backward``   the gradients dQ, dK, dV of the plain definition by the chain
               rule (the backward that page 3 section 6's autograd wrapper
               calls), in fp64.

Every function here is pinned by ``tests/test_oracle.py`` against hand-derived
values (``tests/golden/``), closed forms, brute force and invariants; no
function here is "parity unpinned".
"""
from .definition import attention, attention_rows, softmax_probs, scores
from .online import attention_online
from .backward import attention_backward

__all__ = ["attention", "attention_rows", "softmax_probs", "scores", "attention_online",
           "attention_backward"]
