"""Plain, slow, float64 CPU oracle for the cache-aware streaming Conformer chunk step.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from here. The HIP library and its
Python binding never import, call or link this package, and this package imports nothing from
them: the two share only the seeded draws in ``synth/``.

Sources (cited by page title and section):
- "True streaming encode — implementation spec" (fluidaudio-web STREAMING.md): the
  chunked-causal mask and the offline==streaming gate ("Why this is provably correct"), the
  per-stream state ("State"), the per-chunk flow ("Per-chunk flow", steps 1-4) and the
  provisional-tail lookahead variant ("Status", Nemotron bullet).
- "Parakeet-EOU-120M — Streaming ASR Model" (speech-swift model card): layer count, width and
  attention context ("Config"), the encoder cache tensors ("Architecture"), and the joint's
  class layout vocabulary + blank + EOU ("Joint", "Vocabulary").
- "Fast Accuracy-Preserving RNNT Beam Search on Apple Silicon": the encoder-side joint
  projection computed once per frame ("Delete Repeated Projection Work First").

Where the pages leave a step open the oracle takes the plainest reading; each such reading is
named where it is used (A1..A34 in the module docstrings).
"""
from .encoder import (  # noqa: F401
    Oracle,
    StreamState,
    layer_norm,
    silu,
    sinusoid_rows,
    relshift,
)
