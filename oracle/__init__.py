"""CPU oracle of the ReSA hot path (test infrastructure only; see resa_oracle)."""
from . import resa_oracle  # noqa: F401
