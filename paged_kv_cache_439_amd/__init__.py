"""MI355X (gfx950) library for attention over a block-paged KV cache.

The compute path is the C-ABI shared library ``libpagedattn.so`` built from
``csrc/`` (hand-written HIP kernels); ``binding`` marshals torch tensors into
its calls. ``workloads`` draws the seeded synthetic inputs.
"""

from .binding import (  # noqa: F401
    PagedAttnError,
    library_path,
    load_library,
    pa_decode,
    pa_decode_workspace_size,
    pa_prefill_chunk,
    pa_status_string,
    pa_store_kvcache,
)
