"""KV-cache size formula — test infrastructure only.

"Генерация и KV-кэш", section "Сколько весит KV-кэш": the cache holds a key
and a value for every layer, every KV head, every position and every request:

    bytes = 2 * L * H_kv * d_h * T * B * (bytes per element)

(2 for K and V; 2 bytes in FP16/BF16, 1 in FP8).  With L = 1 and T = B = 1 this
is the per-token-per-layer figure 2 * H_kv * d_h * bytes; with H_kv = 1 it is
the per-head figure of "KV Cache, Flash Attention and Inference Optimization"
(section "The problem"/KV-cache sizing).  The decode kernels must read exactly
this many cache bytes per step (one pass over every cached token).
"""


def kv_cache_bytes(layers: int, kv_heads: int, head_dim: int, tokens: int,
                   batch: int = 1, bytes_per_elem: int = 2) -> int:
    return 2 * layers * kv_heads * head_dim * tokens * batch * bytes_per_elem


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, bytes_per_elem: int = 2) -> int:
    return kv_cache_bytes(layers, kv_heads, head_dim, 1, 1, bytes_per_elem)
