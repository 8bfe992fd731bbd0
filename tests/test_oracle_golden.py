"""The oracle against numbers the pages state (tests/golden/page_values.txt, each line citing its
page and section): FP4's 15 distinct values, the [0, 448*6] range of P's first level, the block
sizes and scale types of NVFP4 and MXFP4."""
import os

import numpy as np

import oracle as orc

HERE = os.path.dirname(os.path.abspath(__file__))


def page_values():
    vals = {}
    with open(os.path.join(HERE, "golden", "page_values.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            name, value = line.split(";", 1)[0].split()
            vals[name] = value
    return vals


def test_golden_file_is_complete():
    assert set(page_values()) == {"fp4_distinct_values", "p_first_level_max", "nvfp4_block", "nvfp4_scale_max",
                                  "mxfp4_block", "mxfp4_scale_kind", "e2m1_max"}


def test_fp4_distinct_values_and_max():
    v = page_values()
    table = [orc.lib().orc_e2m1_decode(c) for c in range(16)]
    assert len(set(table)) == int(v["fp4_distinct_values"])
    assert max(table) == float(v["e2m1_max"])


def test_block_sizes_and_scale_types():
    v = page_values()
    assert orc.blk(orc.NVFP4) == int(v["nvfp4_block"]) and orc.blk(orc.MXFP4) == int(v["mxfp4_block"])
    L = orc.lib()
    assert max(L.orc_e4m3_decode(b) for b in range(127)) == float(v["nvfp4_scale_max"])
    assert v["mxfp4_scale_kind"] == "power_of_two"
    for b in range(255):
        s = L.orc_e8m0_decode(b)
        assert s > 0 and np.frexp(s)[0] == 0.5  # an exact power of two


def test_p_first_level_range():
    """NVFP4 P of a tile: the maximal score maps to the top of [0, 448*6], which quantises exactly
    to the largest E2M1 code times the largest E4M3 scale; every other value lies below it."""
    v = page_values()
    top = float(v["p_first_level_max"])
    assert top == float(v["nvfp4_scale_max"]) * float(v["e2m1_max"])
    rng = np.random.default_rng(4)
    x = rng.standard_normal(128).astype(np.float32)
    vis = np.ones(128, np.uint8)
    E, codes, scales, t = orc.p_tile(orc.NVFP4, x, vis)
    smax = int(np.argmax(x))
    blk = smax // 16
    assert t == float(x.max()) and E[smax] == 1.0
    assert orc.lib().orc_e4m3_decode(int(scales[blk])) * orc.lib().orc_e2m1_decode(int(codes[smax])) == top
    assert np.all(2688.0 * E <= top)
