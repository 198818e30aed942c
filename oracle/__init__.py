"""CPU oracle of the GR00T flow-matching DiT action head (test infrastructure only)."""
from . import gr00t_oracle  # noqa: F401
