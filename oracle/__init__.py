"""CPU oracle for the tree conv and tree Gated DeltaNet forward.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import anything from this package; the
product path never does.  It shares no code with the HIP library: it derives
root-to-leaf paths from the parent array on its own and runs the plain
definitions on every path.

Definitions followed ("Tree Training: Accelerating Agentic LLMs Training via
Shared Prefix Reuse", arXiv 2511.00413, section 3.1 Eq. 6 and section 3.2
Eq. 10-11; and the tree-recurrence 0.1.0 project page, "How a tree runs"):
every token's result equals the one a standalone forward over its own
root-to-leaf path produces.  So the oracle simply runs each path on its own:

* conv.py  -- causal depthwise conv1d over the path (zero left padding).
* gdn.py   -- token-by-token gated delta rule over the path.
* trie.py  -- parents -> children, leaves, paths, POR.
* brute.py -- independent fp64 brute forces used to pin the above.
* grad.py  -- gradients of the tree conv and tree gated delta rule: autograd
              of the token-by-token tree forward (fp64), siblings' gradients
              summed into their parent.
* ssd.py   -- token-by-token Mamba2 (SSD) recurrence over every path, the
              forked state of the tree Mamba2 forward.

Arithmetic is fp64 by default.  Parity status of every function is pinned by
tests (see tests/test_oracle_*.py); nothing here is "parity unpinned".
"""
from .trie import (  # noqa: F401
    segment_offsets, children_of, leaves_of, root_path, leaf_paths,
    path_token_index, path_token_count, por,
)
from .conv import conv_on_path, tree_conv_reference  # noqa: F401
from .gdn import gdn_on_path, tree_gdn_reference  # noqa: F401
