"""Cache-aware streaming Conformer chunk step for MI355X (gfx950).

The work runs in ``libcac.so`` (HIP kernels behind the C ABI of ``include/cac.h`` for the
encoder chunk step, ``include/cac_decode.h`` for greedy decoding of its output and
``include/cac_mel.h`` for the streaming log-mel front and ``include/cac_beam.h`` for batched
beam search); ``binding`` is its thin ctypes wrapper.
"""
from .binding import (  # noqa: F401
    CAC_BF16,
    CAC_F32,
    CAC_FLAG_DRY_RUN,
    CAC_FLAG_POISON,
    BeamSearch,
    CacError,
    StreamingDecoder,
    StreamingEncoder,
    StreamingMel,
    load,
    make_config,
    pack_params,
    param_order,
)
