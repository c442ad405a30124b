"""fp64 CPU oracle (test infrastructure only; the product path never imports it)."""
from . import layer, plan, compare  # noqa: F401
