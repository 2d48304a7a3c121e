"""CPU oracle of the sparse MoE FFN forward -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import, call or execute anything in this package.  The HIP
library (``top_routing_expert_gate_amd``) never imports it, and it never
imports the HIP library: the two share no code.

* ``oracle.moe_oracle`` -- plain float64 NumPy statement of the layer.
* ``oracle.bruteforce`` -- pure-Python dense brute force for tiny inputs.
"""
