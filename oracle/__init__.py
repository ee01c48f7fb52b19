"""CPU oracle and checker for the sparse-attention indexer (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU baseline may use this
package; the GPU library neither imports nor links it.
"""
from . import indexer, check, prep  # noqa: F401
