"""Per-token KV-cache sizes of the layouts the pages compare (numbers, not bytes).

* "Multi-Head Latent Attention" (talalahmed.dev), "A concrete size comparison":
  MHA keeps a key and a value per head; the simplified MLA layout keeps the
  latent plus a RoPE key *per head*.
* "AI decoupled RoPE MLA" (operatorworld.com): MHA keeps 2 n_h d_h numbers;
  absorbed MLA keeps d_c; with decoupled RoPE it keeps d_c + d_r (one position
  key shared by all heads, as "Latent Attention Meets RoPE" also states).
"""


def mha(n_heads: int, d_k: int, d_v: int) -> int:
    return n_heads * d_k + n_heads * d_v


def mla_per_head_rope(d_latent: int, n_heads: int, d_rope: int) -> int:
    return d_latent + n_heads * d_rope


def mla_shared_rope(d_latent: int, d_rope: int) -> int:
    return d_latent + d_rope


def reduction(small: int, big: int) -> float:
    return 1.0 - small / big
