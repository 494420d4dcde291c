"""Seeded synthetic inputs shaped like the pages' workloads.

This package only draws random numbers and lays them out; it holds none of the
method's arithmetic (no rotation, no scoring, no selection, no attention, no
page summaries).  Both the oracle side (tests, cpu baseline) and the GPU side
(tests, bench) take their inputs from here.
"""
from .gen import (SPECS, Workload, aimed_dirs, dense_pool, draft_kv, make, make_device,  # noqa: F401
                  request_key, spec)
