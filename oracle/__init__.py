"""CPU oracle of the DSA path: test infrastructure only (tests, smoke check, CPU baseline).

The product library never imports this package.
"""
from . import dsa_oracle  # noqa: F401
