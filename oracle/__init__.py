"""Plain, slow CPU oracle for the NCCL-style all-reduce data path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the HIP library under
``double_binary_tree_amd/`` and imports nothing from it.

The oracle follows the pages step by step, vectorised only over the elements
of one step, so that a reader can check every fold against the text:

* ``topology``  - node-level binary tree, double tree (mirror / shift), the
  intra-node chain and the head mapping per channel.
* ``partition`` - channel ranges, tree chunks, ring loops and rank-chunks.
* ``numerics``  - the reduction operators with per-hop rounding.
* ``ring``      - ring reduce-scatter + all-gather step simulator.
* ``tree``      - tree reduce-up / broadcast-down simulator.
* ``allreduce`` - the whole all-reduce over N virtual ranks, plus the fp64
  reference sum and the normwise tolerance check.

Parity status of every function is stated in its module header.
"""

from . import numerics, partition, topology, ring, tree, allreduce  # noqa: F401
