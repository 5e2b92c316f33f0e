"""MI355X (gfx950) MXFP4 expert-weight MoE decode layer.

The compute lives in ``libmoe_mxfp4.so`` (hand-written HIP kernels behind a C
ABI, declared in ``include/moe_mxfp4.h``).  ``mxfp4_expert_weight_amd.binding``
marshals arguments to it and raises if the library is missing -- there is no
CPU fallback.  ``mxfp4_expert_weight_amd.synth`` draws seeded synthetic inputs.
Submodules are imported explicitly (``from mxfp4_expert_weight_amd import
binding``); importing the package itself loads nothing.
"""
