"""CPU oracle for the decoder-only GPT training step — TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct NumPy implementation of what the device path
computes: forward, cross-entropy loss, hand-derived backward, global grad norm
and the AdamW update.  Only the tests, the smoke check and the CPU-baseline leg
of the benchmark may import it.  The device path never does, and this package
imports nothing from it.
"""

from .gpt_oracle import *  # noqa: F401,F403
