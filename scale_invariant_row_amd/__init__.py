"""Row-wise L2 normalisation on MI355X (gfx950): HIP kernels behind a C ABI.

``scale_invariant_row_amd.binding`` loads the compiled library and exposes its
entry points (``ds_l2_rows``, ``ds_slerp_rows``, ``ds_weight_rownorm_gain``);
``scale_invariant_row_amd.inputs`` builds the seeded synthetic workloads.
Importing the package itself loads nothing.
"""
