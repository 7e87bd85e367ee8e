"""The selection-fidelity metrics (recall and IoU against the dense set) on
hand-worked rows: the definitions the sweep reports."""
import numpy as np

from long_context_sparse_05_amd.fidelity import set_metrics, to_markdown


def test_recall_and_iou_by_hand():
    # {1,2,3} vs {2,3,4}: two shared of three reference -> recall 2/3; union 4 -> IoU 2/4
    r, i = set_metrics([[1, 2, 3]], [[2, 3, 4]])
    assert r == 2 / 3 and i == 0.5
    # identical sets in any order
    assert set_metrics([[5, 1, 9]], [[9, 5, 1]]) == (1.0, 1.0)
    # disjoint
    assert set_metrics([[1, 2]], [[3, 4]]) == (0.0, 0.0)


def test_padding_is_dropped_and_rows_average():
    # a short prefix: both sides padded with -1; the padding is not a token
    r, i = set_metrics([[7, -1, -1], [1, 2, 3]], [[7, -1, -1], [1, 2, 4]])
    assert np.isclose(r, (1.0 + 2 / 3) / 2) and np.isclose(i, (1.0 + 0.5) / 2)
    # empty reference and empty selection agree perfectly
    assert set_metrics([[-1, -1]], [[-1, -1]]) == (1.0, 1.0)


def test_markdown_table():
    md = to_markdown([dict(method="MISA", B=128, h=8, kp=2048, recall=0.5, iou=0.25)], "t")
    assert "| MISA | 128 | 8 | 2048 | 0.5000 | 0.2500 |" in md
