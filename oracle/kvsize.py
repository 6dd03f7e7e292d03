"""KV-cache byte accounting (oracle; test infrastructure only).

"The Reasoning Engine Meltdown", §2.1 "The Transformer Attention Mechanism &
KV-Cache Mechanics": a request of S tokens on a model with L layers, H heads of
dimension d_h stored with P bytes per element holds one key and one value
vector per token, per layer and per head, so it needs 2*L*H*d_h*S*P bytes.

Reading: H counts the heads that are *stored*, i.e. the KV heads under grouped
query attention; the printed example is multi-head (H = 64 for a 70B-class
model), where query and KV heads coincide.
"""


def kv_bytes(num_layers: int, num_heads: int, head_dim: int, seq_len: int, elem_bytes: int) -> int:
    """Memory_KV = 2 * L * H * d_h * S * P, exact integer bytes."""
    for name, v in (("num_layers", num_layers), ("num_heads", num_heads), ("head_dim", head_dim),
                    ("seq_len", seq_len), ("elem_bytes", elem_bytes)):
        if int(v) != v or v < 0:
            raise ValueError(f"{name} must be a non-negative integer, got {v!r}")
    return 2 * int(num_layers) * int(num_heads) * int(head_dim) * int(seq_len) * int(elem_bytes)


def kv_bytes_per_token(num_layers: int, num_heads: int, head_dim: int, elem_bytes: int) -> int:
    """The formula at S = 1 (the page's bytes/token figure)."""
    return kv_bytes(num_layers, num_heads, head_dim, 1, elem_bytes)
