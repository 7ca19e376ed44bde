"""fp64 CPU oracle of the Titans neural long-term memory.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the GPU library never does.
"""
from .titans_oracle import (  # noqa: F401
    build, lib_path, param_count, memory_apply, memory_grad, forward, max_threads,
)
from .input_oracle import input_side  # noqa: F401
from .backward_oracle import backward, forward_torch  # noqa: F401
