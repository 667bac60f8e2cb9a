"""Calibration artifacts: values computed once per model and reused across runs.

TEAL slides (method slide, slide 10): the per-projection thresholds come from
calibration data and the block-wise sparsity levels from a greedy search run once;
GLASS summary (section 2.2): the global prior and the resulting static neuron set
are reused from prompt to prompt.  This module stores such values (thresholds,
masks, index sets, seeds) as an ``.npz`` file of plain arrays beside a JSON record
holding the key they were computed for (configuration, seeds, sparsity, library
version) and the SHA-256 of the ``.npz``; ``load`` returns them only when the key
matches exactly and the file is the one recorded.  Arrays are written and read
without pickling (``numpy.load`` with ``allow_pickle=False``).  Host I/O only: no
arithmetic of the method happens here.
"""
from __future__ import annotations

import hashlib
import json
import os

import numpy as np


def _name(key: dict) -> str:
    """File stem of a key: the SHA-256 of its canonical JSON."""
    blob = json.dumps(key, sort_keys=True, separators=(",", ":")).encode()
    return hashlib.sha256(blob).hexdigest()[:24]


def _sha256(path: str) -> str:
    h = hashlib.sha256()
    with open(path, "rb") as f:
        for chunk in iter(lambda: f.read(1 << 20), b""):
            h.update(chunk)
    return h.hexdigest()


def save(directory: str, key: dict, arrays: dict, meta: dict | None = None) -> str:
    """Writes ``arrays`` (name -> array-like of numbers or booleans) under ``key``
    (a JSON-serialisable dict) into ``directory``; returns the path of the JSON record.
    An existing record of the same key is replaced."""
    os.makedirs(directory, exist_ok=True)
    stem = os.path.join(directory, _name(key))
    plain = {}
    for k, v in arrays.items():
        a = np.asarray(v)
        if a.dtype == object:
            raise TypeError(f"artifact {k!r}: object arrays are not stored")
        plain[k] = a
    npz = stem + ".npz"
    tmp = stem + ".tmp.npz"
    np.savez(tmp, **plain)
    os.replace(tmp, npz)
    rec = {"key": key, "arrays": sorted(plain), "npz": os.path.basename(npz), "npz_sha256": _sha256(npz),
           "meta": meta or {}}
    path = stem + ".json"
    with open(path + ".tmp", "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
    os.replace(path + ".tmp", path)
    return path


def load(directory: str, key: dict):
    """Returns ``(arrays, meta)`` saved under exactly ``key`` in ``directory``, or None
    when there is no record, the record's key differs, or the ``.npz`` is not the file
    the record describes (its SHA-256 differs)."""
    stem = os.path.join(directory, _name(key))
    path = stem + ".json"
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("key") != json.loads(json.dumps(key)):
        return None
    npz = os.path.join(directory, rec.get("npz", ""))
    if not os.path.exists(npz) or _sha256(npz) != rec.get("npz_sha256"):
        return None
    with np.load(npz, allow_pickle=False) as z:
        arrays = {k: z[k].copy() for k in rec.get("arrays", [])}
    return arrays, rec.get("meta", {})
