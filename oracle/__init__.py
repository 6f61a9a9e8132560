"""Plain fp64 CPU oracle for the Clebsch-Gordan tensor-product convolution.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
product (``clebsch_gordan_tensor_node_amd``) never imports it, and this package
never imports the product: the two share no code.

See ``oracle/cgtp_oracle.py`` for what each function follows and how it is pinned.
"""
from .cgtp_oracle import *  # noqa: F401,F403
