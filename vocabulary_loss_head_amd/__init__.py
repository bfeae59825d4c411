"""cutloss: fused large-vocabulary classifier-head losses (BCE, softmax CE, fused SGD)
with hand-written HIP kernels for AMD Instinct MI355X (gfx950).

The compute path is the C-ABI shared library ``libcutloss.so`` (see include/cutloss.h);
``vocabulary_loss_head_amd.binding`` is its ctypes binding. Importing the binding
fails if the library has not been built (``python -m vocabulary_loss_head_amd.build``).
"""
__version__ = "0.1.0"
