"""Split-KV FP8 paged-attention decode for MI355X (gfx950).

The compute path is libpa.so (hand-written HIP kernels behind a C ABI, see
include/pa_decode.h); ``binding`` marshals torch tensors into it.
``workloads`` builds seeded synthetic inputs.
"""

from . import binding  # noqa: F401
from .binding import Plan, attend, load_library, pa_decode, pa_reduce, problem_of  # noqa: F401
