"""DyRA layer forward for AMD MI355X (gfx950).

Submodules:
  synth  -- seeded synthetic inputs (no method arithmetic)
  dyra   -- ctypes binding of the C-ABI library libdyra.so (loaded lazily)
"""
