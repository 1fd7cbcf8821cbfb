"""Frame-aligned attention for MI355X (gfx950).

The compute lives in libfa.so (hand-written HIP kernels behind the C ABI of
include/fa.h); `binding` marshals torch tensors and streams into it.  Import
`frame_aligned_attention_amd.binding` to use it; importing it fails if the
library has not been built.
"""
