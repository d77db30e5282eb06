"""MI355X (gfx950) MLA decode with weight absorption: HIP kernels behind a C ABI.

The HIP library is libmla.so in this directory (built by
`python -m mla_latent_kv_08_amd.build`); `ops` binds its calls for torch tensors.
"""
from . import ops  # noqa: F401
from .ops import (LatentCache, MLAError, mla_absorb_q, mla_cache_append,  # noqa: F401
                  mla_decode_attn, mla_decode_workspace_size, mla_dequant_rows, mla_up_proj_v)
