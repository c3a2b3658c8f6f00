"""fp64 CPU oracle for exact attention: test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package.  The HIP library and its
Python binding never do, and this package imports nothing from them.
"""
from .ref import ref_bwd, ref_bwd_delta, ref_bwd_rows, ref_fwd, ref_fwd_rows, ref_probs  # noqa: F401
from .split import ref_fwd_keyrange, ref_lse_merge  # noqa: F401
from .masks import (ref_bwd_blocksparse, ref_bwd_visible, ref_bwd_window,  # noqa: F401
                    ref_fwd_blocksparse, ref_fwd_blocksparse_rows, ref_fwd_visible, ref_fwd_window,
                    ref_fwd_window_rows)
from .dropout import keep_mask, philox4x32, ref_bwd_dropout, ref_fwd_dropout  # noqa: F401
