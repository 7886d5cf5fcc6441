"""CPU fp64 oracle (test infrastructure only; see kata_oracle's docstring for who may use it)."""
from .kata_oracle import *  # noqa: F401,F403
from .kata_oracle import __all__  # noqa: F401
