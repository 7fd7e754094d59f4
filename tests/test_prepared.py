"""Saving and loading the offline products (CPU): exact round trip, and refusal
of unknown names, wrong dtypes, disagreeing sizes and pickled objects."""
import numpy as np
import pytest
import torch

from w8a8_quantized_amd.prepared import load_prepared, save_prepared


def _prepared(rng, N=6, K=40, n_o=3):
    return {
        "s": torch.from_numpy(rng.uniform(0.1, 9, K).astype(np.float32)),
        "x_absmax": torch.from_numpy(rng.uniform(0, 90, K).astype(np.float32)),
        "w_absmax": torch.from_numpy(rng.uniform(0, 1, K).astype(np.float32)),
        "Wq": torch.from_numpy(rng.integers(-127, 128, (N, K), dtype=np.int8)),
        "Wq_fp8": torch.from_numpy(rng.integers(0, 256, (N, K), dtype=np.uint8)),
        "w_scale": torch.from_numpy(rng.uniform(1e-4, 1e-2, N).astype(np.float32)),
        "outlier_idx": torch.tensor([3, 17, 29], dtype=torch.int32),
        "outlier_mask": torch.from_numpy((np.arange(K) % 7 != 0).astype(np.float32)),
        "W_out": torch.from_numpy(rng.standard_normal((n_o, N)).astype(np.float32)),
        "alpha": 0.75,
    }


def test_round_trip(tmp_path):
    p = _prepared(np.random.default_rng(0))
    path = tmp_path / "layer.npz"
    save_prepared(path, **p)
    got = load_prepared(path, device="cpu")
    assert set(got) == set(p)
    assert got["alpha"] == 0.75
    for k, v in p.items():
        if k == "alpha":
            continue
        assert got[k].dtype == v.dtype and torch.equal(got[k], v), k


def test_partial_set_and_numpy_inputs(tmp_path):
    rng = np.random.default_rng(1)
    Wq = rng.integers(-127, 128, (4, 16), dtype=np.int8)
    ws = rng.uniform(0.01, 1, 4).astype(np.float32)
    path = tmp_path / "w.npz"
    save_prepared(path, Wq=Wq, w_scale=ws, s=None)
    got = load_prepared(path, device="cpu")
    assert set(got) == {"Wq", "w_scale"}
    assert np.array_equal(got["Wq"].numpy(), Wq) and np.array_equal(got["w_scale"].numpy(), ws)


@pytest.mark.parametrize("bad", [
    {"Wq": np.zeros((4, 16), np.int16), "w_scale": np.ones(4, np.float32)},     # dtype
    {"Wq": np.zeros((4, 16), np.int8), "w_scale": np.ones(5, np.float32)},      # N disagrees
    {"Wq": np.zeros((4, 16), np.int8), "s": np.ones(15, np.float32)},           # K disagrees
    {"Wq": np.zeros((4, 16), np.int8), "bias": np.ones(4, np.float32)},         # unknown name
    {"s": np.ones((2, 8), np.float32)},                                          # rank
])
def test_refused_on_save(tmp_path, bad):
    with pytest.raises(ValueError):
        save_prepared(tmp_path / "bad.npz", **bad)


def test_refused_on_load(tmp_path):
    # an archive written by other means is checked the same way on load
    path = tmp_path / "other.npz"
    np.savez(path, Wq=np.zeros((4, 16), np.int8), w_scale=np.ones(5, np.float32))
    with pytest.raises(ValueError):
        load_prepared(path, device="cpu")
    # object arrays would need unpickling: refused by the loader itself
    path2 = tmp_path / "objects.npz"
    np.savez(path2, s=np.array([{"a": 1}], dtype=object))
    with pytest.raises(ValueError):
        load_prepared(path2, device="cpu")
