"""CPU float64 oracle (test infrastructure only; never on the product path)."""
from .naive_attention import attention_forward, attention_rows, kv_head, ROW_BLOCK  # noqa: F401
