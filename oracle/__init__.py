"""CPU oracle for the chunk-schedule collective executor.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this package.
The product library never reaches it: it shares no code with the HIP path and it
imports nothing from ``chunk_schedule_execution_amd``.

Three oracles live here, all plain numpy, written to be checked by eye:

* ``definitions`` (O1): the collectives by their definitions, sums in float64
  (int64 then wrapped for int32). These are the results the schedules must reach.
* ``schedule_order`` (O2): the textbook ring / hierarchical / two-dimensional
  algorithms the schedules follow, adding in the order each chunk travels, with
  the storage dtype's rounding at every store. This gives bit-exact expectations
  for floating-point reductions.
* ``program`` (O2, generic): a sequential interpreter of a chunk program given as
  plain tuples, plus a symbolic executor (multisets of contributors per chunk)
  that checks a program against a collective's postcondition.

Pins that tie these to something other than themselves are in
``tests/test_oracle_pins.py`` and ``tests/golden/``.
"""

from . import numerics, definitions, schedule_order, program  # noqa: F401
