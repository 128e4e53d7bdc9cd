"""MI355X-native backward of the chunkwise gated delta rule (Gated DeltaNet).

The compute path is a C-ABI shared library (csrc/, header include/gdr.h) built
for gfx950; `binding` is a thin ctypes layer over it that marshals torch tensors
(device memory and streams only).  Import the binding explicitly:

    from chunked_gated_delta_08_amd import binding
    from chunked_gated_delta_08_amd.autograd import chunk_gated_delta_rule   # forward + backward
"""
__all__ = ["autograd", "binding", "workloads"]
