"""MI355X-native Gated DeltaNet token mixer (gfx950).

The compute lives in ``libgdn.so`` (hand-written HIP kernels behind a C ABI);
this package only marshals arguments to it.
"""
