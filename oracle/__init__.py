"""Float64 CPU oracle of the attention-KL primitive.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``, never by the library.
"""
from .streamkl_oracle import (  # noqa: F401
    allowed_keys,
    backward,
    finish,
    forward,
    head_backward,
    head_dk_cols,
    head_dq_rows,
    head_forward,
    merge_partials,
    online_forward,
    online_partials,
    row_logsumexp,
)
