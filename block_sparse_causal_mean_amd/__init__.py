"""Block-sparse causal attention for long-context prefill on MI355X (gfx950).

The compute path is a C-ABI shared library of hand-written HIP kernels
(``csrc/`` -> ``libsparse_attn.so``); ``api`` is its thin Python binding.  Importing this
package loads nothing; the library is loaded on first use and its absence is an error.
"""

__all__ = ["api", "workloads"]
