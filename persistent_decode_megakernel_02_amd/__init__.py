"""Persistent decode megakernel for MI355X (gfx950).

The compute path is a C-ABI shared library (libmk.so) of hand-written HIP
kernels; `binding` marshals arguments to it.  `configs` and `synth` describe
and generate the seeded synthetic workloads.
"""
