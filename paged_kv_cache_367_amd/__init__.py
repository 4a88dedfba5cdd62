"""MI355X-native paged attention (decode and multi-token queries): Python binding of
libpa.so.

The names mirror the C ABI in include/paged_attention.h. Each function only marshals
arguments (torch tensors -> device pointers, dtype codes, the current HIP stream) and
calls the library; every step of the computation runs in the HIP kernels. If the
library is not built the calls raise; there is no fallback path.
"""
from .binding import (  # noqa: F401
    PA_F32, PA_F16, PA_BF16, PA_FP8_E4M3, PaError, DecodeDesc, PrefillDesc, lib_path,
    load_library,
    pa_abi_version, pa_status_string, pa_decode_max_chunks, decode_workspace, pa_decode_workspace_bytes,
    pa_decode, pa_decode_noalloc, pa_prefill, pa_cache_write, pa_cache_write_fp8, pa_block_copy,
    pa_block_swap, pa_stream_read,
)
from .block_manager import BlockManager, PA_ERR_NO_BLOCKS, PA_ERR_UNKNOWN_SEQ  # noqa: F401
