"""MI355X-native Titans neural long-term memory: chunked test-time update and
retrieval behind the C ABI of include/titans_mem.h (libtitans_mem.so)."""
from . import workloads  # noqa: F401
from .titans_mem import (  # noqa: F401
    forward, retrieve, load, make_desc, param_count, select_path, workspace_bytes,
    TitansMemError,
)
