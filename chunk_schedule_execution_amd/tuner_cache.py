"""Persistent cache of tuned points: the tuner's only state worth keeping across runs.

A JSON file maps a key -- a hash of the candidate programs' operations, the rank
count, dtype, the power-of-two bucket of the element count, the device name, the
search space and the base configuration's flags -- to the point ``ccl_tune`` returned.
Resuming tuning is loading the file: a key already present is answered without timing
anything. Host-side bookkeeping around ``capi.ccl_tune``; nothing here runs a
collective.
"""

from __future__ import annotations

import hashlib
import json
import os

from . import capi


def count_bucket(count: int) -> int:
    """The power of two at or above count (tuned points transfer within a bucket)."""
    b = 1
    while b < count:
        b <<= 1
    return b


def cache_key(progs, count: int, base: capi.ccl_plan_config, space: capi.ccl_tune_space, device: str) -> str:
    h = hashlib.sha256()
    for p in progs:
        h.update(repr((p.collective, p.nranks, p.in_chunks, p.out_chunks, p.scratch_chunks, p.group_size,
                       p.group_scope, [tuple(vars(o).values()) for o in p.ops])).encode())
    arrays = [[space.factors[i] for i in range(space.nfactors)], [space.nthreads[i] for i in range(space.nnthreads)],
              [space.slices[i] for i in range(space.nslices)]]
    h.update(repr((progs[0].nranks, base.dtype, count_bucket(count), device, arrays, space.protocols,
                   base.scheduler, base.wg_alloc, base.flags, base.num_cus)).encode())
    return h.hexdigest()[:32]


class TunerCache:
    def __init__(self, path: str, tune=None):
        self.path = path
        self._tune = tune or capi.ccl_tune  # the timing function (replaceable in host tests)
        self.entries = {}
        if os.path.exists(path):
            with open(path) as fh:
                self.entries = json.load(fh)
        self.hits = self.misses = 0

    def tune(self, progs, count: int, base: capi.ccl_plan_config, space: capi.ccl_tune_space, stream: int = 0,
             device: str | None = None) -> capi.ccl_tune_point:
        """The cached point for this key, else ccl_tune's, stored and saved."""
        if device is None:
            import torch
            device = torch.cuda.get_device_name(0)
        key = cache_key(progs, count, base, space, device)
        if key in self.entries:
            self.hits += 1
            e = self.entries[key]
            return capi.ccl_tune_point(e["variant"], e["parallel_factor"], e["nthreads"], e["slice_bytes"],
                                       e["protocol"], 0)
        self.misses += 1
        best, rep = self._tune([p.to_desc() for p in progs], count, base, space, stream)
        self.entries[key] = {"variant": best.variant, "parallel_factor": best.parallel_factor,
                             "nthreads": best.nthreads, "slice_bytes": best.slice_bytes, "protocol": best.protocol,
                             "best_score": rep.best_score, "evaluations": rep.evaluations, "count": count,
                             "device": device}
        tmp = self.path + ".tmp"
        with open(tmp, "w") as fh:
            json.dump(self.entries, fh, indent=1, sort_keys=True)
        os.replace(tmp, self.path)
        return best
