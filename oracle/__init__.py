"""CPU oracle for SFI decode attention (test infrastructure only; see
``oracle.sfi_oracle``).  Only tests, the smoke check and the bench's CPU
baseline may import this package."""
from .sfi_oracle import *  # noqa: F401,F403
