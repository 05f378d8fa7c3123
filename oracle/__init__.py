"""CPU float64 oracle (test infrastructure only; never on the product path)."""
from .naive_attention import (attention_forward, attention_rows, kv_head, merge_partials,  # noqa: F401
                              ROW_BLOCK)
from .naive_backward import attention_backward, backward_keys, backward_rows  # noqa: F401
from .naive_mla import (mla_absorb_q, mla_absorbed, mla_latent_attention, mla_naive,  # noqa: F401
                        mla_up_project)
