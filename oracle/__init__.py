"""CPU oracle (test infrastructure only; see vit_oracle's header)."""

from . import vit_oracle  # noqa: F401
