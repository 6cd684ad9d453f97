"""fp64 CPU oracle for the LoLA hot path.  TEST INFRASTRUCTURE ONLY: the product path never imports it."""
from .lola_oracle import *  # noqa: F401,F403
