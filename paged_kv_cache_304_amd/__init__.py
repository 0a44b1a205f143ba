"""MI355X (gfx950) paged KV cache kernels behind a C ABI.

The compute runs in ``libpagedkv.so`` (hand-written HIP, see ``csrc/``); this
package only marshals torch tensors into the C entry points declared in
``include/pagedkv.h``. PyTorch provides device memory and the current HIP
stream, nothing else. Importing the package fails loudly when the library has
not been built (``python paged_kv_cache_304_amd/build.py``): there is no
fallback implementation.
"""
from ._lib import LIB_PATH, PagedKVError, abi_version, lib  # noqa: F401
from .blocks import BlockManager, DeviceStep, StepStager  # noqa: F401
from .ops import (  # noqa: F401
    concat_and_cache_mla_k,
    concat_and_cast_mla_k,
    decode_attention,
    decode_attention_noalloc,
    decode_attention_workspace_size,
    decode_step,
    hbm_copy,
    hbm_read,
    mla_decode_attention,
    mla_decode_step,
    mla_decode_workspace_size,
    prefill_attention,
    reshape_and_cache,
)
