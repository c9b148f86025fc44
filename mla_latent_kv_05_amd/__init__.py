"""Absorbed ("MQA mode") Multi-head Latent Attention decode for MI355X (gfx950).

The compute lives in ``libmla.so`` (hand-written HIP behind a C ABI, declared in
``include/mla_decode.h``); ``binding`` marshals torch tensors into it.
``inputs`` creates seeded synthetic workloads.  Submodules are imported on
demand (``from mla_latent_kv_05_amd import binding``)."""
