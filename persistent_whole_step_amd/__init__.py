"""persistent_whole_step_amd: one persistent HIP kernel per training step on MI355X (gfx950).

The library (``libtk.so``, C ABI in ``include/tk.h``) compiles a static
whole-step program into a device-resident stage table and runs it with a
single grid-resident kernel.  ``persistent_whole_step_amd.tk`` is the thin
ctypes binding; ``programs`` and ``synth`` describe workloads and seeded inputs.
"""
