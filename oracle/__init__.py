"""CPU fp64 oracle for the hybrid gated-delta-rule + sink/sliding-window layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or link
this package: only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` use it.  It shares no code with the HIP library.

Parity status of each function (what pins it) is listed in ``oracle.hybrid``.
"""

from .hybrid import (  # noqa: F401
    in_softmax_set,
    in_linear_set,
    softmax_index_set,
    linear_index_set,
    gdn_linear_branch,
    gla_linear_branch,
    swa_branch,
    hybrid_prefill,
    cache_from_prefill,
    decode_step,
    rope,
    causal_depthwise_conv,
    l2norm,
    shortconv_qkv,
)
