"""MI355X-native backward of the chunkwise gated delta rule (Gated DeltaNet).

The compute path is a C-ABI shared library (csrc/, header include/gdr.h) built
for gfx950; `binding` is a thin ctypes layer over it that marshals torch tensors
(device memory and streams only).  Import the binding explicitly:

    from chunked_gated_delta_08_amd import binding
"""
__all__ = ["binding", "workloads"]
