"""CPU oracle for the deterministic attention backward.

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check in
__graft_entry__.py and the CPU-baseline leg of bench.py may import anything
here.  The product package never imports this package, and this package
never imports the product package: the two share no code.

Modules:
  attention  - fp64 numpy forward/backward from the definition
  schedules  - unit item lists and dQ rank tables, per schedule
  dag        - DAG / critical-path model and an event simulation
"""
