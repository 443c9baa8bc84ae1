"""MI355X-native expert-parallel dispatch/combine core (one GPU's share).

The four stages -- layout, notify, dispatch, combine -- are HIP kernels for
gfx950 behind the C ABI declared in ``include/ep.h`` (library ``libep.so``).
``combine_ep_get_02_amd.ep`` is the thin ctypes binding over that ABI;
``combine_ep_get_02_amd.inputs`` draws the seeded synthetic workloads.
"""
