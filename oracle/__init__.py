"""CPU oracle for W12 (test infrastructure only; see ``oracle.w12_oracle``)."""
from .w12_oracle import *  # noqa: F401,F403
from .w12_oracle import W12Logical, encode, decode, verify, choose_window, bits_per_weight  # noqa: F401
