"""Exact IO-aware attention for AMD MI355X (gfx950).

`O = softmax(Q K^T * scale) V`, forward and backward, computed tile by tile
with an online softmax so that the N x N score matrix never reaches HBM.
The arithmetic runs in hand-written HIP kernels inside `libfa.so`, reached
through a C ABI (include/fa.h); `binding` marshals torch tensors into that
ABI and nothing more. The library is loaded on first use, so importing the
package (for example for `inputs`) does not need a GPU.
"""
__all__ = ["binding", "inputs"]
