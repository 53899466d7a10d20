"""Microbenchmarks of the gfx950 facts the kernels' schedules rest on.

They are standalone HIP programs, not part of the library: nothing in the
library, the tests or the bench imports them.  Build them (on any machine with
hipcc) and run them on an MI355X with::

    python -m exact_tiled_attention_flash_amd.probes --build
    python -m exact_tiled_attention_flash_amd.probes coissue
    python -m exact_tiled_attention_flash_amd.probes ldsread
"""
