"""Tree conv + tree Gated DeltaNet forward for MI355X (gfx950), over a packed prefix trie.

    plan = tree_plan(parents, seg_lens, conv_width=4)   # host, once per forward
    y = tree_conv(x, w, plan)                            # [N, C]
    o = tree_gdn_scan(q, k, v, g, beta, plan)            # [N, H_v, d_v]

The kernels live in libtreegdn.so (C ABI in include/tree_gdn.h); this module
only marshals torch tensors into pointers and the current HIP stream.
"""
from ._lib import (  # noqa: F401
    TreeError,
    TreePlan,
    load,
    tree_conv,
    tree_conv_backward,
    tree_gdn_scan,
    tree_gdn_scan_backward,
    tree_plan,
    tree_ssd_scan,
)
