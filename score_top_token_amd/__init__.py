"""MI355X (gfx950) Lightning Indexer forward pass: per-token scores
I[t,s] = sum_h w[t,h] * ReLU(q[t,h,:] . k[s,:]) and the fused per-token top-k,
behind the C ABI of include/li.h.

Submodules:
  binding -- ctypes binding of the C ABI (loads liblightning_indexer.so lazily,
             raises if it is missing)
  build   -- in-tree hipcc build of the library for gfx950
  synth   -- seeded synthetic inputs (no indexer arithmetic)
"""
