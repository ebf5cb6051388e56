"""Float64 CPU reference (the oracle) for prefix-shared attention forward.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, links or runs
this package: only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may use it.  It shares no code with the HIP library or its
Python binding; the only thing both sides share is the seeded input generator
in ``psattn_inputs``.

What it computes (PrefixSharing PR #50, "设计简介" / design summary): the
flat-packed layout ``[P | S1 | ... | SN]`` with a block-causal visibility is
claimed mathematically equal to the ``build_kv`` route, which copies the
provider prefix once per reuser so that every rollout becomes an ordinary
causal sequence ``[P | Si]``.  The oracle therefore *is* that expansion plus
ordinary causal softmax attention, in float64 (``attention.attn_flat``).  The
verify path (sglang PR #27382, "实现拆解" / implementation breakdown) is the
same causal attention of the draft rows over the request's paged prefix
followed by its own draft block (``attention.attn_paged``).

Modules:
  decode     -- exact byte -> float64 decoding (fp32, bf16, OCP fp8 e4m3fn)
  attention  -- build_kv expansion + causal attention (flat, paged)
  brute      -- scalar per-pair brute force over the visibility predicate
  plan       -- enumeration of the tile work items the library's planner emits

Every function is pinned by ``tests/test_oracle_*.py`` (brute force,
library special cases, closed forms, invariants); see each docstring.
"""
from .decode import decode, decode_bf16, decode_fp8_e4m3, fp8_e4m3_table  # noqa: F401
from .attention import attn_flat, attn_paged, causal_attention  # noqa: F401
