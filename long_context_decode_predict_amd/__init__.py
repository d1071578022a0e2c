"""MI355X-native Elastic Threshold Attention (ETA) block-sparse decode step.

The compute path is the HIP library ``libeta.so`` (C ABI in ``include/eta.h``);
this package holds its ctypes binding (``_lib``), a step driver (``decode``),
the seeded synthetic workloads (``workloads``), the closed-form threshold bias
(``calibrate``) and the in-tree build (``build``).
"""
from . import _lib  # noqa: F401
from ._lib import (EtaError, Meta, default_params, eta_admit_union, eta_append_meta,  # noqa: F401
                   eta_build_block_meta, eta_decode_attn, eta_decode_attn_combine,
                   eta_decode_attn_partial, eta_decode_attn_workspace_size, eta_predict_screen,
                   eta_predict_tau, eta_screen)
