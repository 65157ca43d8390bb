"""fp64 CPU oracle for attention-state memory.  Test infrastructure only: the
library never imports it."""
from . import asm_oracle  # noqa: F401
