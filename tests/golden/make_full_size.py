"""Write the fp64 oracle's per-row values at the full workload sizes.

The GPU parity tests at these sizes compare every row's log-normaliser and KL,
and the loss, with these values; computing them takes minutes of fp64 work on
the host (two projections of 2*S*H*V each at the 32K and 256K contexts), so
they are computed once here and stored. This script calls only the oracle and
the seeded input generator: no value comes from the GPU library.

  python tests/golden/make_full_size.py 32k_context 256k_context entropy_selective

Each output file holds, besides the arrays, a JSON string `meta` with the
workload, the seed, and the SHA-256 of the generated inputs (hidden, W, ids and
teacher-logit bits), which the tests check before using the values.
"""
from __future__ import annotations

import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from kd_synth import make_problem  # noqa: E402
from oracle import (oracle_entropy_rows, oracle_rows,  # noqa: E402
                    oracle_select_top_fraction)

HERE = os.path.dirname(os.path.abspath(__file__))

# name: (S, H, V, K, T, chunk, seed)
WORKLOADS = {
    "32k_context": (32768, 2880, 201088, 100, 1.0, 2048, 1003),
    "256k_context": (262144, 3072, 128256, 100, 2.0, 2048, 1004),
    "entropy_selective": (32768, 2048, 151936, 100, 1.0, 1024, 1005),
}
BLOCK = 1024


def input_digest(p) -> str:
    h = hashlib.sha256()
    for a in (p.hidden_bits, p.W_bits, np.ascontiguousarray(p.ids, dtype=np.int32), p.tl_bits):
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def path_of(name: str) -> str:
    return os.path.join(HERE, f"full_{name}.npz")


def load_problem(name: str):
    S, H, V, K, T, chunk, seed = WORKLOADS[name]
    return make_problem(S, H, V, K, T=T, chunk=chunk, seed=seed)


def _rows_fwd(p, Wd, rows):
    """The oracle's lse and KL of the given rows, in blocks (all rows treated as valid)."""
    lse = np.empty(len(rows))
    kl = np.empty(len(rows))
    for b0 in range(0, len(rows), BLOCK):
        r = rows[b0:b0 + BLOCK]
        out = oracle_rows(p.hidden[r], Wd, p.ids[r], p.tlogits[r], p.T, len(rows), grads=False)
        lse[b0:b0 + BLOCK] = out["lse"]
        kl[b0:b0 + BLOCK] = out["kl_rows"]
    return lse, kl


def make(name: str) -> str:
    t0 = time.time()
    p = load_problem(name)
    S, H, V, K, T, chunk, seed = WORKLOADS[name]
    Wd = p.W.astype(np.float64)
    meta = dict(workload=name, S=S, H=H, V=V, K=K, T=T, seed=seed, inputs_sha256=input_digest(p))
    arrays = {}
    if name == "entropy_selective":
        ent = np.empty(S)
        for b0 in range(0, S, BLOCK):
            ent[b0:b0 + BLOCK] = oracle_entropy_rows(p.hidden[b0:b0 + BLOCK].astype(np.float64) @ Wd.T)
        _, idx, k = oracle_select_top_fraction(ent, 20, 100)
        lse, kl = _rows_fwd(p, Wd, idx)
        arrays.update(entropy=ent, idx=idx, lse=lse, kl=kl)
        meta.update(num=20, den=100, kept=int(k), loss=math.fsum(kl) / k)
    else:
        rows = np.arange(S)
        lse, kl = _rows_fwd(p, Wd, rows)
        arrays.update(lse=lse, kl=kl)
        meta.update(loss=math.fsum(kl) / S)
    meta["seconds"] = round(time.time() - t0, 1)
    out = path_of(name)
    np.savez(out, meta=np.array(json.dumps(meta, sort_keys=True)), **arrays)
    return out


def load(name: str):
    """(meta dict, arrays dict) of a stored workload file."""
    with np.load(path_of(name), allow_pickle=False) as z:
        meta = json.loads(str(z["meta"]))
        arrays = {k: z[k] for k in z.files if k != "meta"}
    return meta, arrays


if __name__ == "__main__":
    for nm in sys.argv[1:] or list(WORKLOADS):
        print(nm, make(nm), flush=True)
