"""Host checks of the seeded input generators (no GPU)."""
import numpy as np

from draft_head_step_amd.inputs import CONFIGS, from_tiled, make_head, make_workload, to_tiled


def test_make_head_matches_the_full_workload():
    cfg = CONFIGS["tiny"]
    head, full = make_head(cfg), make_workload(cfg)
    for k in ("W1", "W2", "anchors"):
        assert np.array_equal(head[k], full[k])


def test_workload_is_reproducible():
    a, b = make_workload(CONFIGS["tiny"]), make_workload(CONFIGS["tiny"])
    for k in ("W1", "W2", "base", "h", "w_conf", "anchors", "sps"):
        assert np.array_equal(a[k], b[k])


def test_tiled_roundtrip_ragged_tail():
    x = np.random.default_rng(0).standard_normal((3, 2, 70)).astype(np.float32)
    t = to_tiled(x)
    assert t.shape == (2, 3, 32, 3)
    assert np.array_equal(from_tiled(t, 70), x)
    assert np.all(t[:, 2, 6:, :] == 0)      # entries past V are zero
