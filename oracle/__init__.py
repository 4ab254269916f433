"""Oracle for the radix-tree prefix cache and its attention path.

TEST INFRASTRUCTURE ONLY: a plain CPU implementation (Python radix tree,
float64 numpy attention) that the tests compare the HIP library against.
Only tests/, the smoke check in __graft_entry__ and bench.py's CPU-baseline
leg may import it.  It shares no code with the library under
radix_tree_prefix_amd/ and imports nothing from it.
"""
from .tree import RadixTree, NoSpace, Stale, common_prefix_len  # noqa: F401
from .attention import attend, merge_states  # noqa: F401
from .admit import (admit, release, release_tail, admit_history, admit_batch,  # noqa: F401
                    prefill_no_sharing, prefill_sequential, prefill_fixed_prefix)
from .schedule import schedule, peek_match  # noqa: F401
from . import speculative  # noqa: F401
