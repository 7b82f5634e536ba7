"""CPU oracle of the sparse-KV decode path: test infrastructure only.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package.  It imports nothing from the product package.
"""
from . import spc_oracle  # noqa: F401
from .decoder import OracleDecoder  # noqa: F401
