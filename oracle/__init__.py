"""Test infrastructure: the float64 CPU oracle of the token-sparse attention path.

Only the tests, the smoke check and the benchmark's CPU-baseline leg import this
package; the product library never does."""
from .tsa_oracle import *  # noqa: F401,F403
