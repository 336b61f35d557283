"""Float64 CPU oracle for exact attention: test infrastructure only (see sdpa_oracle)."""
from .sdpa_oracle import *  # noqa: F401,F403
