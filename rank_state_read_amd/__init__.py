"""SketchSSM decode hot path for MI355X (gfx950): Python binding of libsketchssm.so.

The HIP library does all the work; this package only loads it and marshals
arguments.  Import fails loudly at first use if the library is not built.
"""
from .binding import (  # noqa: F401
    DTYPE,
    KIND,
    LIB_PATH,
    Plan,
    Shape,
    SketchSSMError,
    lib,
    make_shape,
    sketchssm_decode_read,
    sketchssm_decode_read_flush,
    sketchssm_decode_read_seq,
    sketchssm_dense_read,
    sketchssm_flush,
    sketchssm_flush_seq,
    sketchssm_rmw_step,
    sketchssm_stream_probe,
    status_string,
)
