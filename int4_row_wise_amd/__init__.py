"""Row-wise INT4/INT8 quantized embedding tables on MI355X (gfx950).

The compute lives in a HIP C-ABI library (``libqemb.so``, declared in
``include/qemb.h``); :mod:`int4_row_wise_amd.qemb` is a thin ctypes binding
over it that only marshals torch tensors and the current stream.  The
library loads on first use and raises if it was not built; there is no CPU
fallback.  :mod:`int4_row_wise_amd.synth` draws the seeded synthetic inputs.
"""
from .qemb import (  # noqa: F401
    RANGE, GREEDY, SUM, WEIGHTED_SUM, CODEBOOK_ITERS, SYMMETRIC, PERCENTILE, ACIQ, QembError,
    abi_version, bag_forward, quantize_baseline,
    bag_forward_codebook, codebook_row_stride, dequantize, dequantize_codebook, dot_interaction,
    interaction_width, l2_error,
    l2_error_codebook, load_library, quantize_codebook, quantize_rowwise, row_stride,
    COMPRESS_VERBATIM, compress_bound, compress_pooled, compress_record_bytes, compress_workspace_bytes,
    decompress_pooled, compress_pooled_noalloc, COMPRESS_NOALLOC_MAX_VECTORS,
)
