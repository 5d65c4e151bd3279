"""Tree-flattened ForkAttention and forked Gated DeltaNet for MI355X (gfx950).

The compute path is the HIP library ``libforkattn.so`` built from ``csrc/``;
``binding`` marshals arguments to its C-ABI. ``workloads`` holds the seeded
synthetic inputs. Importing the package loads nothing; the first call into the
binding loads the library and fails loudly if it is missing.
"""
__all__ = ["binding", "workloads", "metrics"]
