"""CPU oracle for draft-tree verification -- test infrastructure, not product.

Only the tests, the smoke entry point and the benchmark's CPU-baseline leg may
import this package.  It shares no code with the HIP library.  ``ref`` holds
the verification step and the commit; ``eagle2`` the EAGLE-2 tree builder;
``draft_head`` the two-stage draft LM head.
"""
from .ref import (TREE_OK, TREE_E_ROOT, TREE_E_PARENT, TREE_E_COUNT, TREE_E_TOKEN,
                  TREE_E_NONFINITE, TREE_E_NOQ, TREE_E_SYNC, TREE_E_CACHE, TREE_E_PATH, SIB_WITHOUT_REPLACEMENT, SIB_IID, EXEMPT_MARGIN,
                  to_f64, check_tree, ancestors, tree_mask, tree_attention,
                  target_distribution, argmax_lowest, inverse_cdf, accept_walk,
                  spec_accept, commit_accepted, verify_step)
