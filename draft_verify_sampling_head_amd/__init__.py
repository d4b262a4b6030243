"""MI355X-native hot path of one DSpark speculative-decoding round.

The compute lives in libdspark.so (hand-written HIP kernels for gfx950, C ABI
in include/dspark.h).  This package is its binding: `_lib` marshals arguments
to the C entry points, `round` enqueues a whole round, `synth` draws seeded
synthetic inputs.  Importing the package loads the library and fails if it is
missing; there is no other execution path.
"""
from . import _lib
from ._lib import (DsparkError, acceptance_rate, acceptance_rate_features, async_schedule,
                   confidence, confidence_logits, draft_markov, draft_rnn, get_status, clear_status, pack, pack_tiered,
                   prefix_schedule, round_markov, schedule_pack, rnn_workspace, rnn_workspace_bytes, sts_fit, sts_workspace,
                   verify, verify_cap_accept, verify_cap_accept_features, verify_features,
                   w2_transpose, workspace, workspace_bytes)

_lib.load()

__all__ = ["DsparkError", "acceptance_rate", "acceptance_rate_features", "async_schedule",
           "confidence", "confidence_logits", "draft_markov", "draft_rnn", "get_status", "clear_status", "pack", "pack_tiered",
           "prefix_schedule", "round_markov", "schedule_pack", "rnn_workspace", "rnn_workspace_bytes", "sts_fit", "sts_workspace",
           "verify", "verify_cap_accept", "verify_cap_accept_features", "verify_features",
           "w2_transpose", "workspace", "workspace_bytes"]
