"""fp64 CPU oracle of the Hymba hybrid-head mixer: test infrastructure only.

Importable by the tests, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg; never by the product path.
"""
