"""CPU oracle for block-sparse decode attention -- test infrastructure only (see kvs_oracle)."""
from . import kvs_oracle  # noqa: F401
