"""MI355X-native deterministic MoE expert-parallel dispatch layout, dispatch and
combine on one GPU's share of the work.

* ``combine_ep_layout_07_amd.ep`` -- the Python binding of ``libep.so``
  (HIP kernels for gfx950 behind the C ABI in ``include/ep.h``); importing it
  raises ImportError when the library has not been built.
* ``combine_ep_layout_07_amd.workloads`` -- seeded synthetic inputs.
"""
