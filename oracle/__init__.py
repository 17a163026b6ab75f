"""CPU fp64 oracle for document-masked causal GQA attention (one CP rank).

Test infrastructure only: imported by the tests, the package smoke check and
the benchmark's CPU-baseline leg, never by the GPU library.
"""
from .attention import *  # noqa: F401,F403
from .attention import __all__  # noqa: F401
