"""CPU oracle for the sparse ternary BitLinear forward.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(``sparsity_amd``) never imports, links or executes anything here, and this
package shares no code with it: the only module both sides use is ``synth``,
which draws seeded random inputs and holds none of the method's arithmetic.

Every function is a plain, slow, obviously correct restatement of what the
pages define, in numpy, with int64 accumulation and exact (rational) arithmetic
where the definition calls for an exact value.  See ``bitlinear_ref`` for the
per-function citations and for the list of functions whose parity is pinned.
"""
from .bitlinear_ref import *  # noqa: F401,F403
