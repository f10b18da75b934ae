import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD Instinct GPU (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running oracle statistics")


def pytest_collection_modifyitems(config, items):
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def load_worked_example(name):
    """Parse a worked-example fixture into numpy inputs of the accept step."""
    import numpy as np
    vocab, drafts, rows, exp_n, exp_tok = None, None, [], None, None
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *rest = line.split()
            if key == "vocab":
                vocab = rest
            elif key == "drafts":
                drafts = rest
            elif key in ("p", "q"):
                rows.append((key, [float(v) for v in rest]))
            elif key == "expect_n_acc":
                exp_n = int(rest[0])
            elif key == "expect_tokens":
                exp_tok = rest
    k = len(drafts)
    ps = [r for key, r in rows if key == "p"]
    qs = [r for key, r in rows if key == "q"]
    assert len(ps) == k + 1 and len(qs) == k
    with np.errstate(divide="ignore"):
        target = np.log(np.array(ps, dtype=np.float64))
        draft = np.log(np.array(qs, dtype=np.float64))
    tokens = np.array([vocab.index(d) for d in drafts], dtype=np.int64)
    return dict(vocab=vocab, target=target, draft=draft, tokens=tokens,
                expect_n_acc=exp_n, expect_tokens=[vocab.index(t) for t in exp_tok])
