"""KV-cache size formula (oracle; test infrastructure).

Per-token KV bytes = 2 (K and V) x layers x kv_heads x head_dim x bytes per element
(vLLM-PagedAttention与连续批处理技术拆解, section 一, the per-request memory ledger).
"""


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, bytes_per_elem: int) -> int:
    return 2 * layers * kv_heads * head_dim * bytes_per_elem


def kv_bytes_per_request(tokens: int, layers: int, kv_heads: int, head_dim: int,
                         bytes_per_elem: int) -> int:
    return tokens * kv_bytes_per_token(layers, kv_heads, head_dim, bytes_per_elem)
