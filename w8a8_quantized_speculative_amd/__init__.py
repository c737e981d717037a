"""MI355X-native hot path of Quasar's quantized verification.

The W8A8 SmoothQuant verify linear and the greedy/rejection accept step run as
hand-written gfx950 HIP kernels inside ``libquasar.so`` (C ABI in
``include/quasar.h``); ``binding`` marshals torch tensors into those calls.
``synth`` draws the seeded synthetic inputs.
"""
from .binding import (  # noqa: F401
    PackedWeights,
    QuasarError,
    lib,
    new_workspace,
    packed_weight_bytes,
    quasar_quantize_activations,
    quasar_quantize_weights,
    quasar_stream_copy,
    quasar_verify_accept,
    quasar_w8a8_linear,
    workspace_bytes_accept,
    w8a8_kernel_name,
    workspace_bytes_linear,
)
