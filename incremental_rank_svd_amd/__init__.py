"""MI355X (gfx950) iS-KV compressed KV cache: block-incremental truncated SVD
of every K and V stream, with decode attention over the factors.

The compute path is libiskv.so (hand-written HIP, C ABI in include/iskv.h);
``iskv`` is its Python binding.
"""

from . import iskv  # noqa: F401
from .iskv import Cache, Config, ISKVError, config_from_workload, make_config, workspace_bytes  # noqa: F401
