"""CPU oracle for one expert-parallel rank's share of an MoE layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package; only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the
HIP path: it is plain Python + NumPy, float64 for floating point, written from
the pages' description of the method and kept deliberately slow and obvious.

Source cited throughout ("the tile-signal notes"): the reading-notes page
"MoE 计算-通信细粒度重叠：用 Tile 级信号把 All-to-All 藏在 GEMM 背后" (Zhongzhu Zhou,
2026-08-06) on Cui, Wingkvist and Ericsson, "Fine-grained Computation-
Communication Overlap via Tile-level Signaling and Scheduling for Mixture-of-
Experts" (ICPP 2026).  Section numbers are the notes' own (§4.2 owner-aligned
row layout, §4.3 padding cost, §4.4 remote-first schedule and the layout +
schedule pseudo-code, §4.5 combine plan, §5.2 segments, §2.2 the five-step
MoE forward).

Modules
-------
``bf16``     round-to-nearest-even to bf16 from float64, and decoding.
``plan``     received rows, owner-aligned layout, remote-first schedule,
             combine plan, segments, owner-side slots.
``ffn``      SwiGLU expert FFN per layout row, float64 with bf16 rounding of
             the hidden activation and of the expert output.
``combine``  applying the combine plan to the expert output.
``scale``    gate-weighted top-k reduction at the owner.
``brute``    definition-level MoE output and a sort-based layout, for tiny
             inputs (independent of the histogram/scan route of ``plan``).
``invariants`` the properties the pages fix for layout, schedule and plan.

Pins: ``tests/test_oracle_*.py`` (marked ``not gpu``).  Every function here has
at least one pin that does not re-derive it with the same formula; see the
test module docstrings.
"""
from . import bf16, plan, ffn, combine, scale, brute, invariants  # noqa: F401

__all__ = ["bf16", "plan", "ffn", "combine", "scale", "brute", "invariants"]
