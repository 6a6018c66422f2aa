"""CPU oracles (fp64): document-masked causal grouped-query attention
(attention.py), its band-block formulation (band.py) and gated delta-rule
linear attention with a scalar gate (Gated DeltaNet, delta.py) and a
per-channel gate (Kimi Delta Attention, kimi_delta.py).

Test infrastructure: only tests/, the smoke check and the bench's CPU
baseline may import it.  The product path never does.
"""
from .attention import (attention_backward, attention_forward, attention_key, attention_row,
                        segments, visible_mask)

__all__ = ["attention_backward", "attention_forward", "attention_key", "attention_row",
           "segments", "visible_mask"]
