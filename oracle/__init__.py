"""CPU oracle for the DiffusionGemma canvas-denoise step (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import this package. The GPU library shares no code with it. See ``dg_oracle`` for
the method readings and the passages each function follows.
"""
from .dg_oracle import *  # noqa: F401,F403
from .dg_oracle import (  # noqa: F401
    from_bf16, to_bf16, temperature, canvas_attn, attention_rows, logits_entropy,
    entropy_fixed, entropy_accept, philox4x64_10, uniform_token, renoise, gelu_erf,
    selfcond, stop_test, commit_kv, run_canvas, STOP_GO, STOP_STOP, STOP_CAP,
    STREAM_INIT, STREAM_RENOISE, TWO32, H_LIMIT, Q_SENTINEL,
)
