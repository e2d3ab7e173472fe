"""CPU oracle (test infrastructure only; see sfag_oracle)."""
from .sfag_oracle import (backward, backward_rows, csr, decode, flops, forward, geometry,  # noqa: F401
                          scale32, token_terms)
