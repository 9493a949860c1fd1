"""fp64 CPU oracle (test infrastructure only; never imported by the product path)."""
from .hkv_oracle import *  # noqa: F401,F403
