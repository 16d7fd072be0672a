"""fp64 CPU oracle of the low-rank bottleneck block.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or execute anything in
this package. The GPU library never links or imports it, and the product
path fails loudly when its HIP library is missing instead of falling back
to anything here.
"""
from .lrblock import (  # noqa: F401
    ACTS,
    act_fn,
    act_grad,
    btp_consumer,
    btp_consumer_backward,
    btp_share_backward,
    btp_share_forward,
    lrblock_backward,
    lrblock_forward,
    lrmlp_backward,
    lrmlp_forward,
    rmsnorm,
    sigmoid,
    silu,
    silu_grad,
)
from .layer import (  # noqa: F401
    layer_backward,
    layer_forward,
    round_to_bf16,
    standin_backward,
    standin_forward,
)
