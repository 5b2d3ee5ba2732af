"""CPU oracle for OSCAR-style INT2 KV-cache quantize-append and decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package; only the tests, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP library (``long_context_decode_kvq_amd``) and imports nothing from it.
"""
from .kvq_oracle import *  # noqa: F401,F403
