"""fp64 CPU oracle of the GPT-2 training step.

Test infrastructure only: the tests, the package smoke check and the bench's
CPU-baseline leg import it.  The HIP library never does.
"""
from .gpt_oracle import *  # noqa: F401,F403
