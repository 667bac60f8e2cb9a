"""Calibration artifacts (activation_sparse_gemv_amd.artifacts): values computed once
(thresholds, masks, index sets) round-trip exactly, are returned only for the key
they were saved under, and a changed file is refused."""
import json
import os

import numpy as np
import pytest

from activation_sparse_gemv_amd import artifacts


KEY = {"workload": "Llama-3-8B-shaped SwiGLU MLP", "sparsity": 0.5, "calib_seed": 20008, "library_version": 7}


def test_round_trip_is_exact(tmp_path):
    rng = np.random.default_rng(3)
    arrays = {"t_x": np.float32(0.6745), "t_h": np.float32(1.25e-3),
              "mask": rng.random(14336) < 0.5, "idx": np.sort(rng.choice(14336, 7168, replace=False)).astype(np.int32),
              "levels": np.array([4, 5, 5, 6], dtype=np.int32)}
    path = artifacts.save(str(tmp_path), KEY, arrays, {"note": "test"})
    assert os.path.exists(path)
    got, meta = artifacts.load(str(tmp_path), dict(KEY))
    assert meta == {"note": "test"}
    assert set(got) == set(arrays)
    for k, v in arrays.items():
        a = np.asarray(v)
        assert got[k].dtype == a.dtype and got[k].shape == a.shape
        assert np.array_equal(got[k], a)
    # bit patterns of the fp32 thresholds are kept
    assert got["t_x"].view(np.uint32) == np.float32(0.6745).view(np.uint32)


def test_other_key_or_missing_record_gives_none(tmp_path):
    artifacts.save(str(tmp_path), KEY, {"t_x": np.float32(1.0)})
    assert artifacts.load(str(tmp_path), {**KEY, "sparsity": 0.4}) is None
    assert artifacts.load(str(tmp_path), {**KEY, "library_version": 8}) is None
    assert artifacts.load(str(tmp_path / "nowhere"), KEY) is None


def test_changed_file_is_refused(tmp_path):
    path = artifacts.save(str(tmp_path), KEY, {"t_x": np.float32(1.0)})
    rec = json.load(open(path))
    npz = os.path.join(str(tmp_path), rec["npz"])
    np.savez(npz, t_x=np.float32(2.0))          # same name, other content
    assert artifacts.load(str(tmp_path), KEY) is None


def test_saving_again_replaces_and_objects_are_refused(tmp_path):
    artifacts.save(str(tmp_path), KEY, {"t_x": np.float32(1.0)})
    artifacts.save(str(tmp_path), KEY, {"t_x": np.float32(3.0)})
    got, _ = artifacts.load(str(tmp_path), KEY)
    assert float(got["t_x"]) == 3.0
    with pytest.raises(TypeError):
        artifacts.save(str(tmp_path), KEY, {"bad": np.array([{"a": 1}], dtype=object)})
