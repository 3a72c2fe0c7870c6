"""MI355X-native Kimi Delta Attention (KDA) recurrent-state update.

The compute lives in ``libkda.so`` (hand-written HIP for gfx950 behind a C ABI,
declared in ``include/kda.h``); this package is its thin Python binding:

  api.py    the entry points, same names as the C ABI (argument marshalling)
  _lib.py   ctypes loader; fails loudly when the library is missing
  synth.py  seeded synthetic inputs (no method arithmetic)
  build.py  compiles libkda.so with hipcc for gfx950
"""
