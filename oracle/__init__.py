"""CPU oracle of the MoE decode step — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may import or
run anything under ``oracle/``.  It shares no code with the HIP library; see ``oracle/moe.py``.

Pinning status (each function is pinned by a ``-m "not gpu"`` test against something other than
itself — closed forms, hand-worked fixtures under ``tests/golden/``, brute force, library routines):
quantizer, packing, record layout, dequantization, router logits, top-k, gate weights, activations,
expert FFN, combine, RMSNorm, LFU policy.  Agreement with the real Gemma 4 / MLX numerics is unpinned
(no checkpoint or reference outputs exist here).
"""
from . import moe  # noqa: F401
