"""Cached seeded workloads shared by the GPU test modules (one draw per process)."""
import functools

import workloads


@functools.lru_cache(maxsize=None)
def get(name: str) -> workloads.Workload:
    return workloads.NAMED[name]()


ALL = ("tiny_fp32", "decode", "prefill", "long", "edge_fp16")
# further full-size workloads: the speculative verification step and a mixed decode/prefill batch
EXTRA = ("verify", "mixed")
