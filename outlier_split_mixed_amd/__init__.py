"""MI355X-native outlier-separated dual-path W4A4 GEMM (SQ-format / OSC).

``outlier_split_mixed_amd.sqf`` is the Python binding over the C-ABI library
``libsqf.so`` (HIP kernels for gfx950).  ``outlier_split_mixed_amd.synth``
draws the seeded synthetic workloads.  Importing this package loads nothing;
importing ``sqf`` loads the library and fails loudly if it is missing.
"""
