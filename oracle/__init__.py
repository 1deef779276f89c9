"""CPU oracle of the DSA hot path — test infrastructure only (tests, smoke check, CPU baseline).

Nothing in the product package imports this; see ``dsa_oracle`` for the definitions followed.
"""
from . import dsa_oracle, brute  # noqa: F401
