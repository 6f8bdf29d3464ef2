"""Plain CPU oracle (float64) for dynamic multi-LoRA and MoE-LoRA.

TEST INFRASTRUCTURE ONLY.  tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import it; the library (adapter_lora_amd) never does,
and the two share no code.  Every function cites the passage it follows.
Pins: tests/test_oracle_*.py (brute force, closed forms, invariants, an
integer worked case under tests/golden/).
"""
from . import lora, moe  # noqa: F401
