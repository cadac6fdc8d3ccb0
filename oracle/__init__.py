"""CPU oracle for MLA decoding -- test infrastructure only (see mla_oracle)."""
from . import mla_oracle  # noqa: F401
