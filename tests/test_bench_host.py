"""Host-side helpers of bench.py, checked on the CPU."""
import torch

import bench


def test_recall_vs_flat():
    # ascending lists with -1 padding after the ids
    h = torch.tensor([[[1, 3, 5, -1], [0, 2, 4, 6], [7, -1, -1, -1]]], dtype=torch.int32)
    f = torch.tensor([[[1, 2, 5, -1], [0, 2, 4, 6], [-1, -1, -1, -1]]], dtype=torch.int32)
    # 2 of 3, 4 of 4, and an empty flat list counts as 0 of 1
    assert abs(bench.recall_vs_flat(h, f) - (2 / 3 + 1 + 0) / 3) < 1e-12
    assert bench.recall_vs_flat(f, f) == (1 + 1 + 0) / 3
