"""CPU oracle for chunk-wise block-causal wave attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
path (``block_causal_attention_wave_amd``) and imports nothing from it.

Contents
--------
``oracle.plan``
    Brute-force planner: builds the (chunk, level) update nodes, the context
    lists from the policy phi(j, r), refresh nodes, the serial and the
    pipelined ("wave") round assignment by round-by-round simulation, and a
    naive liveness-based physical slot allocation.
``oracle.attention``
    fp64 softmax attention under an explicit dense additive mask, and the
    round-to-nearest-even conversion of fp32 values to bfloat16.
``oracle.rollout``
    Serial rollout: executes a plan round by round against a dict cache keyed
    by logical slot, recomputing every node's context from phi.
``oracle.chain``
    The toy denoiser chain around the attention: seeded QKV projections with
    a per-token RMS scale, K/V into the node's own slot, and each chunk's next
    node consuming its previous node's last-layer attention output.

Pins (values this oracle is checked against, other than itself) live in
``tests/test_oracle_*.py`` and ``tests/golden/``: for the planner, closed-form
round counts, brute-force minimality, structural invariants and hand-worked
plans (pipelined, serial, same-level, clean, conditioned and history-capped)
down to physical slot ids; for attention, library routines, closed forms and
invariants.  Every function here is pinned; none is "parity unpinned".
"""
