"""EXL3 decode-row projection for MI355X (gfx950): rot_in and the trellis linear.

The compute runs in libtf_exl3.so (hand-written HIP kernels behind the C ABI in
include/tf_exl3.h); this package only marshals torch tensors and streams into
those calls. Importing it does not touch the GPU; the first call loads the
library and raises if it has not been built.
"""

from ._lib import (  # noqa: F401
    TF_DT_BF16,
    TF_DT_F16,
    TF_DT_F32,
    Exl3Error,
    debug_decode_states,
    calib_copy,
    calib_stream_read,
    debug_decode_tiles,
    debug_linear_split,
    debug_linear_mfma_split,
    header_functions,
    linear,
    linear_plan,
    project,
    project_pass_rows,
    repack_strips,
    load,
    rot_in,
    status_string,
    trellis_bytes,
)

WIDTHS = (2, 3, 4, 5, 6, 8)
