"""CompKV block-sparse decode attention for AMD MI355X (gfx950).

The compute path is the HIP library ``libcknv.so`` (C ABI declared in
``include/cknv.h``); ``block_sparse_kv_stats_amd.cknv`` is its thin Python
binding. ``synth`` draws seeded synthetic inputs. Importing this package does
not load the library; the binding loads it on first use and raises if it is
missing.
"""
