"""CPU oracle of the fused MoE expert layer (float64, NumPy).

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import, call or execute anything in this
package.  It shares no code with the HIP library (``moe_expert_layer_sigmoid_amd``)
and neither imports the other; both consume inputs from ``synth``.

Parity status of each function is listed in the module docstrings and in the
design notes; every function here is pinned by a CPU test under ``tests/``.
"""

from . import formats, moe  # noqa: F401
