"""Layer-streamed LoRA fine-tuning on MI355X (gfx950).

The compute path lives in a C-ABI shared library (``liblsq.so``, declared in
``include/ls.h``) built from ``csrc/``; ``binding`` wraps it with ctypes.  Nothing is
loaded at import time: ``binding.lib()`` loads the library on first use and raises if
it has not been built.
"""
