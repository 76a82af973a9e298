"""MI355X-native (gfx950) FlashAttention-2-style tiled attention.

The compute lives in hand-written HIP kernels behind a C ABI
(``include/fa.h``), built into ``libfa2tiles.so`` in this directory.  This
package only marshals arguments to that library (``attention_fa2_tiles_amd.lib``),
routes torch autograd and forward-mode AD to it
(``attention_fa2_tiles_amd.autograd``, which imports torch), and provides
seeded synthetic inputs (``attention_fa2_tiles_amd.inputs``).
Importing the package does not load the library; ``lib.load()`` does, and it
raises if the library is missing: there is no fallback path.
"""

__all__ = ["lib", "inputs", "autograd"]
