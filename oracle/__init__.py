"""CPU float64 oracle for the Mamba2 SSD varlen scan.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
benchmark's CPU-baseline leg, never by the product path. It shares no code with
the HIP library.
"""
from .oracle import (load, ssd_varlen, ssd_decode, causal_conv1d, varlen_metadata,  # noqa: F401
                     checkpoint_plan, num_threads, prefill_bites, prefill_schedule, gated_delta)
