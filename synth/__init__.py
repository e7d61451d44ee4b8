"""Seeded synthetic workloads for the KV-cache quantization path.

This module only *describes* the workloads (shapes, formats, value recipes)
and draws their random inputs.  It holds none of the quantization or attention
arithmetic: both the HIP library's tests and the CPU oracle take their inputs
from here, and nothing else is shared between them.
"""
from .workloads import (CONFIGS, Workload, make_workload, make_inputs, config_for,  # noqa: F401
                        make_prefill_queries, make_page_table)
