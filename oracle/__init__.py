"""CPU fp64 oracle for frame-aligned block-sparse video attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the
HIP path (``block_sparse_video_frame_amd``); the two meet only in the seeded
input generators of ``synth``, which hold none of the method's arithmetic.

Sources (the pages): vatt-ghern.pages.dev "deep-heygen-avatar-iv-trillium-tpu"
(sections 把 block 縮到 16, the 16-token frame-aligned blocks, and
拿掉 softmax 的序列相依, the Cauchy-Schwarz bound softmax); bytechap.com
"Optimizing HeyGen's Avatar IV diffusion model for Google Cloud TPUs" (section
How it works); cloudcurated.com "How is HeyGen optimizing AI video on Google
Cloud TPUs" (Wall 2 and Wall 3).

Modules
  attention  dense fp64 masked softmax attention with an explicit boolean frame
             mask; a pure-Python brute force; a block-by-block evaluation over
             the attended intervals with the online running max or the fixed
             Cauchy-Schwarz shift.
  blocks     the query-tile / key-interval block list, derived from the dense
             boolean mask.
  norms      fp64 row norms, per-16-key maxima, per-head maxima, the per-row
             bound and the per-head eligibility test.
  producer   the Q/K producer that emits the norms in its epilogue: per-head
             RMS norm with a weight, rotary embedding of adjacent pairs, one
             bf16 rounding (straight from fp64), norms of the written rows.

Every function here is pinned by the ``-m "not gpu"`` tests in ``tests/`` to
something other than itself (brute force, closed forms, a library routine or
an invariant).  None is "parity unpinned".
"""
from . import attention, blocks, norms, producer  # noqa: F401
