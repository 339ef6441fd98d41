"""CPU oracle of the speculative-sampling verify step: TEST INFRASTRUCTURE ONLY.

Plain fp64 numpy (``spec_verify_oracle``) and an integer-exact Philox4x64-10
(``philox``).  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It never imports
the HIP library and the library never imports it.
"""
from . import philox, spec_verify_oracle  # noqa: F401
