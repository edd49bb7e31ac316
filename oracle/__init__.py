"""CPU oracle for the paged K/V write, the history-staging gather and paged attention.

TEST INFRASTRUCTURE, NOT PART OF THE LIBRARY.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import this package.  The HIP library under ``paged_kv_cache_174_amd/`` never
imports it, links it or calls it, and this package imports nothing from there.

Everything here is plain numpy in float64 (integer work in int64), written from
the four vllm-omni pages this project is built from:

* P1 "vllm_omni/experimental/ar_diffusion/kv_cache/paged_attention.py"
* P2 "tests/diffusion/ar_diffusion/test_paged_attention.py"
* P3 "vllm_omni/diffusion/attention/backends/utils/piecewise_attn.py"
* P4 "vllm_omni/diffusion/diffusion_kv/paged_attention_adapter.py"

Each function names the page and the function on it that it restates.  Parity
pins (checks against something other than the oracle itself) live in
``tests/test_oracle_*.py``; every function below has at least one.
"""

from .pkv_oracle import *  # noqa: F401,F403
from .pkv_oracle import __all__  # noqa: F401
