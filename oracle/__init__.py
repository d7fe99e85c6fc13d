"""Float64 CPU oracle (test infrastructure only; see prefix_sliding.py)."""
from .prefix_sliding import *  # noqa: F401,F403
from .prefix_sliding import KIND_FULL, KIND_PARTIAL  # noqa: F401
