"""fp64 CPU oracle for draft-head decode attention over a paged KV cache.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or run anything in this
package. The product path (``draft_attention_amd``) never does, and this
package imports nothing from it: the two share no code.

Modules
  ``oracle.reference``  NumPy fp64 oracle (every logit materialised).
  ``oracle.brute``      pure-Python loops over scalars, for 8-64 token inputs;
                        written separately from ``reference`` so that each one
                        pins the other on tiny cases.

Pins (``tests/test_oracle_pins.py``): hand-derived closed forms, brute force on
tiny inputs, and the reductions the pages fix (window >= context is full
attention; FOLD with alpha=1, beta=0 is one softmax over the union; kappa=0 is
the unmodified drafter; weights sum to 1). The pages print no worked numeric
example of the attention, so ``tests/golden/closed_forms.json`` holds cases
worked out by hand from their definitions, each with its derivation.

Parity unpinned: the functional forms of FOLD's alpha/beta combination and of
SharpDraft's s(n). The pages print no formula for either; this library fixes
one reading of each (``oracle.reference`` docstring). The code that implements
those readings is pinned by closed forms; the readings themselves are not
pinned against anything printed on the pages.
"""

from . import reference, brute  # noqa: F401
from .reference import (  # noqa: F401
    MODES,
    append,
    bf16_round,
    decode,
    decode_with_draft,
    index_sets,
    visible_count,
    query_scale,
    rope_rotate,
    gather_keys,
    gather_values,
)
