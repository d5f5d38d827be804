"""CPU oracle of the sparse MQA attention step (test infrastructure only).

Importable only by the tests, the smoke check and the benchmark's CPU-baseline
leg; the product path never touches it.
"""
from .dsa_oracle import *  # noqa: F401,F403
