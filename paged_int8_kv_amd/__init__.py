"""Paged INT8-KV GQA attention for MI355X (gfx950).

The compute lives in a HIP shared library (libkv8.so, C ABI declared in
include/kv8.h).  `paged_int8_kv_amd.binding` marshals torch device tensors
into that ABI; `paged_int8_kv_amd.workloads` draws the seeded synthetic
inputs.  Importing the package loads nothing; the binding loads the library
on first use and raises if it is missing.
"""

__all__ = ["binding", "workloads", "build"]
