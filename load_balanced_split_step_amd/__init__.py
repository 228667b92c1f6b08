"""Dynamic split-KV paged decode attention for MI355X (gfx950).

The compute path lives in the HIP library ``libhda.so`` (C ABI, declared in
``include/hda.h``); :mod:`load_balanced_split_step_amd.hda` is its thin
ctypes binding and :mod:`load_balanced_split_step_amd.workloads` draws the
seeded synthetic inputs.
"""
