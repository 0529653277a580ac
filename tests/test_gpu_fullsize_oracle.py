"""Every element of every output of the five benchmark checkpoints, at full size, against the CPU
oracle, bit for bit.

Each checkpoint is written at its full size, staged from the file and decoded in the launch
configuration bench.py times (one st_materialize over the whole table, outputs in one arena, poisoned
first).  Then every output is copied back in 1 M-element pieces and compared with the unchanged
oracle's decode of the same element range.  The oracle is single-threaded NumPy; a pool of threads
runs it over different pieces at once (NumPy releases the GIL inside its elementwise loops), and
pieces stay small so that its temporaries reuse memory instead of faulting in fresh pages.  Large
checkpoints are split into parts (contiguous runs of outputs of about equal element counts), one test
each, so that no test runs long without reporting.  Each part logs "N of N elements bit-exact"; the
session summary lists the totals per checkpoint.
"""
import os
import shutil
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import synth
import device_checkpoint_dequantisation_amd as st
from tests import parity_log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
PIECE = 1 << 20                  # elements per oracle call
THREADS = max(1, min(16, os.cpu_count() or 1))
# parts per checkpoint, sized so that each part's oracle work takes about a minute on 16 threads
PARTS = {1: 1, 2: 1, 3: 2, 4: 3, 5: 1}
CASES = [(k, p) for k in sorted(PARTS) for p in range(PARTS[k])]

_cache = {}


@pytest.fixture(scope="module")
def workdir(tmp_path_factory):
    d = tmp_path_factory.mktemp("fullsize_oracle")
    yield str(d)
    _drop()
    shutil.rmtree(str(d), ignore_errors=True)


def _drop():
    for k in list(_cache):
        c = _cache.pop(k)
        del c["ck"]
        os.remove(c["path"])
    torch.cuda.empty_cache()


def _staged(k, d):
    """Config k written, staged and decoded once (kept while its parts run)."""
    if k in _cache:
        return _cache[k]
    _drop()
    path = os.path.join(d, f"c{k}.safetensors")
    t0 = time.perf_counter()
    print(f"full-size config {k}: writing", flush=True)
    synth.write_config(k, path)
    ix = st.SafeTensorIndex.open(path)
    ck = st.DeviceCheckpoint(ix, path, DEV)
    ck.arena.view(torch.int16).fill_(0x5A5A)    # poison: every element must be written
    ck.materialize()
    torch.cuda.synchronize()
    mm = np.memmap(path, dtype=np.uint8, mode="r")
    h, outs = oracle.plan(mm)
    couts = ix.outputs()
    assert [o.name for o in outs] == [c.name for c in couts]
    for o, c in zip(outs, couts):
        assert (o.kind, o.shape, o.numel) == (c.kind, c.shape, c.numel), o.name
    print(f"config {k}: {len(outs)} outputs staged and decoded in {time.perf_counter() - t0:.1f}s", flush=True)
    _cache[k] = {"path": path, "ck": ck, "outs": outs, "offsets": [c.offset // 2 for c in couts],
                 "data": mm[h.data_offset:]}
    return _cache[k]


def _part(outs, p, n_parts):
    """Output indices of part p: contiguous runs of about equal element counts."""
    total = sum(o.numel for o in outs)
    lo, hi = total * p / n_parts, total * (p + 1) / n_parts
    sel, pos = [], 0
    for j, o in enumerate(outs):
        mid = pos + o.numel / 2
        if lo <= mid < hi or (p == n_parts - 1 and mid >= hi):
            sel.append(j)
        pos += o.numel
    return sel


@pytest.mark.parametrize("k,part", CASES, ids=[f"c{k}-part{p}" for k, p in CASES])
def test_every_element_against_the_oracle(k, part, workdir):
    c = _staged(k, workdir)
    outs, data = c["outs"], c["data"]
    bits = c["ck"].arena.view(torch.int16)
    sel = _part(outs, part, PARTS[k])
    tasks = [(j, a, min(outs[j].numel, a + PIECE)) for j in sel for a in range(0, outs[j].numel, PIECE)]

    def run(t):
        j, a, b = t
        got = bits[c["offsets"][j] + a: c["offsets"][j] + b].cpu().numpy().view(np.uint16)
        want = oracle.decode(outs[j], data, np.arange(a, b, dtype=np.int64))
        return b - a, int(np.count_nonzero(got != want))

    t0 = time.perf_counter()
    with ThreadPoolExecutor(THREADS) as ex:
        res = list(ex.map(run, tasks))
    n = sum(r[0] for r in res)
    bad = sum(r[1] for r in res)
    dt = time.perf_counter() - t0
    msg = (f"c{k} part {part + 1}/{PARTS[k]}: {n - bad} of {n} elements bit-exact against the oracle "
           f"({len(sel)} outputs, {dt:.0f}s on {THREADS} threads)")
    print(msg, flush=True)
    parity_log.record(f"c{k}", n, n - bad, len(sel))
    assert bad == 0, msg
