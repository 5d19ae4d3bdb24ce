"""MI355X (gfx950) GPT training-step library: HIP kernels behind a C ABI.

The compute path is the shared library ``libgptmi.so`` built from ``csrc/``;
``binding`` marshals torch tensors into its C entry points.  Importing this
package does not load the library; ``binding.lib()`` does, and raises if it
has not been built.
"""
__all__ = ["synth", "binding"]
