"""KV-cache size closed forms (exact integers).

Test infrastructure only (see the package docstring).
"""


def kv_bytes_per_token(layers: int, n_kv_heads: int, head_dim: int, bytes_per_elem: int = 2) -> int:
    """2 (K and V) x layers x n_kv_head x d_head x bytes.

    [注意力变体与MoE] "生成时的瓶颈", the bytes-per-token equation and kv_bytes().
    """
    return 2 * layers * n_kv_heads * head_dim * bytes_per_elem


def mla_kv_bytes_per_token(layers: int, d_latent: int, d_rope: int, bytes_per_elem: int = 2) -> int:
    """layers x (d_c + d_R) x bytes: one latent plus one shared RoPE key, no x2.

    [注意力变体与MoE] "MLA：缓存一个低秩的 latent" (the V3 check); [transformer架构]
    §2.3.5 table (the MLA row has no factor 2).
    """
    return layers * (d_latent + d_rope) * bytes_per_elem
