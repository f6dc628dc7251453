"""fp64 CPU oracle for MARS structured-mask attention (test infrastructure only)."""
from .mars_oracle import *  # noqa: F401,F403
