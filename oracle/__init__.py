"""CPU oracle for the Fathom key scan -- test infrastructure only (see fathom_oracle)."""
from . import fathom_oracle  # noqa: F401
