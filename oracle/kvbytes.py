"""KV-cache bytes per token.

deepsonar "PagedAttention de vLLM …", §2.1 (how much memory the KV cache takes):
each token stores one key and one value vector per KV head per layer, so the
bytes per token are 2 x layers x KV heads x head dim x bytes per element.  The
page works it for an 80-layer, 8-KV-head, dim-128 fp16 model.
"""


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, dtype_bytes: int) -> int:
    for v in (layers, kv_heads, head_dim, dtype_bytes):
        if int(v) != v or v < 0:
            raise ValueError("sizes must be non-negative integers")
    return 2 * int(layers) * int(kv_heads) * int(head_dim) * int(dtype_bytes)


def kv_bytes(tokens: int, layers: int, kv_heads: int, head_dim: int, dtype_bytes: int) -> int:
    return int(tokens) * kv_bytes_per_token(layers, kv_heads, head_dim, dtype_bytes)
