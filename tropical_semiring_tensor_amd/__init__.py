"""MI355X-native tropical GEMM, permute and diagonal gather (gfx950, HIP).

The compute path lives in the C-ABI library ``libtropical.so`` built from
``csrc/``; ``tropical_semiring_tensor_amd.binding`` marshals torch tensors
into it.  Importing this package loads nothing: the library is opened on
first use and a missing build raises an error instead of falling back.
"""
__all__ = ["binding", "inputs"]
