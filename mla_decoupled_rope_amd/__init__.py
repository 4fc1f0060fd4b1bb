"""MI355X-native Multi-head Latent Attention with decoupled RoPE (weight-absorbed form).

The computation lives in libmla.so (hand-written HIP kernels for gfx950 behind
the C ABI of include/mla.h).  This package is its Python binding plus the
device-side state that strings the five calls into decode and prefill steps.
Importing it without the built library raises ImportError.
"""

from .binding import (  # noqa: F401
    LIB, LIB_PATH, MLADims, MLAError, absorb_q, cache_write_per_head, decode, decode_noalloc, decode_per_head,
    decode_per_head_proj, decode_plan, decode_proj, decode_proj_workspace, decode_proj_workspace_size,
    decode_workspace, per_head_row,
    decode_workspace_size, fold_q_weights, front_workspace, front_workspace_size, kv_project, out_proj, prefill,
    prefill_mha, prefill_mha_workspace, prefill_mha_workspace_size, q_project, q_project_folded, rope_absorb_q,
    rope_apply,
)
from .pipeline import (  # noqa: F401
    DecodeStep, LatentCache, LayerDecodeStep, LayerPrefillStep, PerHeadDecodeStep, PrefillStep, choose_prefill_form,
)
