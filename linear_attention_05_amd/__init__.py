"""MI355X-native Kimi Delta Attention (KDA) core.

The kernels (chunked prefill and single-token decode) live in libkda.so,
built from csrc/ by build.py for gfx950; include/kda.h is the C ABI. This
package is a thin torch front end over that ABI."""

from ._binding import KdaError, load as load_library, version  # noqa: F401
from ._binding import (FRONT_ALL, FRONT_BETA_SIGMOID, FRONT_GATE,  # noqa: F401
                       FRONT_L2NORM_QK)
from .api import (kda_decode_step, kda_prefill_chunked,  # noqa: F401
                  kda_prefill_chunked_at, kda_prefill_scan_segments,
                  kda_prefill_workspace_size)

decode_step = kda_decode_step
prefill = kda_prefill_chunked
