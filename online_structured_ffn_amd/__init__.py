"""POP (Partition-guided Online Pruning) channel-pruned gated-MLP path for
AMD Instinct MI355X (gfx950).

The compute path is the C-ABI HIP library ``libpop.so`` (declared in
``include/pop.h``); :mod:`online_structured_ffn_amd.pop` is its thin ctypes
binding.  :mod:`.configs` and :mod:`.synth` hold the workload table and the
seeded input generators.
"""
__all__ = ["configs", "synth"]
