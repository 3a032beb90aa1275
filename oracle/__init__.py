"""Float64 CPU oracle for ReHyAt temporally chunked hybrid attention.

TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline
leg may import or call anything in this package. The library (hybrid_softmax_linear_amd)
never imports it, and this package imports nothing from the library: the two share no code.

What it computes and where each piece comes from is documented in rehyat_oracle.py.
"""
from .rehyat_oracle import (  # noqa: F401
    chunk_layout,
    phi,
    hybrid_attention,
    hybrid_recurrent,
    state_direct,
    recurrent_init,
    recurrent_step,
    EluFeatureMap,
    PolyMlpFeatureMap,
    feature,
    feature_dim,
    hybrid_attention_bwd,
)
