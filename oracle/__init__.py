"""CPU float64 oracle for GPT-OSS-style sink attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
its Python binding) may import, call or link anything under this directory;
only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the GPU path.
"""

from .append import append_mask_cols_ref, append_mask_ref, prefill_append_ref  # noqa: F401
from .paged import (decode_paged_fp8_multi_ref, decode_paged_fp8_ref, decode_paged_multi_ref, decode_paged_ref,  # noqa: F401
                    gather_pages)  # noqa: F401
from .rope import rope_qkv_append_ref, rope_ref, yarn_inv_freq_ref  # noqa: F401
from .oproj import oproj_ref  # noqa: F401
from .fp8 import decode_fp8_multi_ref, decode_fp8_ref, e4m3_to_float64  # noqa: F401
from .sink_attention import (  # noqa: F401
    LOG2E,
    decode_key_range,
    decode_ref,
    decode_split_partials_ref,
    merge_ref,
    prefill_mask_ref,
    prefill_varlen_ref,
    split_chunks_ref,
)
