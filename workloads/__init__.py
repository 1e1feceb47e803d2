"""Seeded synthetic workloads: trie shapes and input tensors.

This package is shared by the oracle tests, the GPU tests and the benchmark.
It only draws random numbers and shapes them into the layouts the tree
conv, the tree Gated DeltaNet scan and the tree Mamba2 (SSD) scan consume;
it performs none of the method's arithmetic.
"""
from .gen import (  # noqa: F401
    CONFIGS,
    ConfigSpec,
    Workload,
    make_trie,
    make_conv_inputs,
    make_scan_inputs,
    make_ssd_inputs,
    SSD_SHAPE,
    make_workload,
)
