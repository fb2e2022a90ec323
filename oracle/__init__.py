"""CPU oracle for paged KV attention (fp64, numpy).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``, never by the library.  See ``paged_attention.py``.
"""

from .paged_attention import (  # noqa: F401
    attention,
    bf16_to_f64,
    decode,
    gather,
    k_offset,
    kv_append,
    merge_partials,
    online_softmax_attention,
    page_bytes,
    partition_partials,
    prefill,
    v_offset,
)
from .rope import f64_to_bf16, positions, rope_freqs, rope_kv_append, rotate  # noqa: F401,E402
from .pages import copy_pages, cow_needs  # noqa: F401,E402
from .norm import residual_rmsnorm, silu_mul  # noqa: F401,E402
