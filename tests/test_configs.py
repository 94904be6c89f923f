"""The synthetic workloads against the benchmark configuration strings kept
at the repository root (the JSON file there that holds the metric and the
five configuration strings): latent, tile, window, batch, heads, head size,
dtype and value recipe of each configuration, parsed from the text and
compared with synthetic.WORKLOADS."""

import json
import os
import re

import pytest

from sliding_tile_attention_sta_amd.synthetic import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NAMES = ["tiny", "small", "720p", "mixed", "long"]


def triple(text):
    return tuple(int(x) for x in re.split(r"[×x,]", text))


def parse(cfg):
    out = {}
    m = re.search(r"latent (\d+[×x]\d+[×x]\d+)", cfg)
    out["video"] = triple(m.group(1))
    m = re.search(r"tile \((\d+,\s*\d+,\s*\d+)\)", cfg)
    out["tile"] = triple(m.group(1).replace(" ", "")) if m else None
    m = re.search(r"window (\d+[×x]\d+[×x]\d+) tiles", cfg)
    out["window"] = triple(m.group(1)) if m else None
    m = re.search(r"batch (\d+)", cfg)
    out["batch"] = int(m.group(1)) if m else None
    out["heads"] = int(re.search(r"(\d+) heads", cfg).group(1))
    out["head_dim"] = int(re.search(r"head_dim (\d+)", cfg).group(1))
    out["dtype"] = "f32" if "fp32" in cfg else "bf16"
    m = re.search(r"from (\d+(?:\.\d+)?)[–-](\d+(?:\.\d+)?)", cfg)
    out["magnitude"] = (float(m.group(1)), float(m.group(2))) if m else None
    m = re.search(r"\{([^}]*)\}", cfg)
    out["cycle"] = [triple(x.strip().split(" ")[0]) for x in m.group(1).split(",")] if m else None
    return out


@pytest.fixture(scope="module")
def configs():
    for name in sorted(os.listdir(ROOT)):
        if not name.endswith(".json"):
            continue
        try:
            doc = json.load(open(os.path.join(ROOT, name)))
        except (OSError, ValueError):
            continue
        if isinstance(doc, dict) and "metric" in doc and isinstance(doc.get("configs"), list):
            return doc["configs"]
    pytest.skip("no benchmark configuration file at the repository root")


def test_five_configurations(configs):
    assert len(configs) == 5


@pytest.mark.parametrize("i,name", list(enumerate(NAMES)))
def test_workload_matches_configuration(configs, i, name):
    c = parse(configs[i])
    w = WORKLOADS[name]
    assert w.video == c["video"], (name, w.video, c["video"])
    assert w.tile == (c["tile"] or WORKLOADS["720p"].tile)
    assert w.heads == c["heads"] and w.head_dim == c["head_dim"]
    assert w.batch == (c["batch"] or 1)
    assert w.dtype == c["dtype"]
    if c["cycle"]:
        assert [tuple(w.windows[h]) for h in range(4)] == c["cycle"]
        assert all(tuple(w.windows[h]) == c["cycle"][h % 4] for h in range(w.heads))
    else:
        assert all(tuple(x) == c["window"] for x in w.windows)
    assert w.magnitude == c["magnitude"]
