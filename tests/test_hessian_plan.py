"""The statistics kernel's token-split plan and work-item map (host logic),
checked on the CPU: the plan model against the library's workspace query,
and the item map covering every (upper super-tile, 32-token step) exactly
once -- at the workload shapes, including the 49152-feature fc2."""

import numpy as np
import pytest

import hessian_plan as hp
import post_weight_quantization_15_amd as gq

SHAPES = [(4096, 262144), (11008, 262144), (12288, 262144), (49152, 262144),
          (4096, 131072), (11008, 131072), (256, 512), (648, 3000), (1024, 20000),
          (136, 1000), (512, 6000)]


@pytest.fixture(scope="module")
def lib():
    return gq.load_library()


@pytest.mark.parametrize("d,n", SHAPES)
def test_plan_model_matches_library(lib, d, n):
    assert lib.gptq_hessian_workspace_bytes(d, n) == hp.workspace_bytes(d, n)


@pytest.mark.parametrize("d,n", [(49152, 262144), (4096, 262144), (648, 3000),
                                 (12288, 262144)])
def test_items_cover_every_tile_step_once(d, n):
    nt = -(-d // hp.SUP)
    steps = -(-n // hp.STEP)
    cover = np.zeros((nt, nt, steps), dtype=np.int16) if nt <= 64 else None
    count = {}
    ns, ks = hp.plan(d, n)
    for w, split, ti, tj, tb, cnt in hp.items(d, n):
        assert 0 <= ti <= tj < nt
        assert tb % hp.STEP == 0 and cnt > 0
        key = (ti, tj)
        count.setdefault(key, []).append((tb, cnt))
    assert len(count) == hp.upper_tiles(nt)
    for key, spans in count.items():
        spans.sort()
        assert len(spans) == ns, key
        pos = 0
        for tb, cnt in spans:
            assert tb == pos, (key, spans)
            pos += cnt
        assert pos == n, (key, pos)


def test_fc2_chain_length():
    """d = 49152: three token splits of 2732, 2732 and 2728 steps (the
    16 GiB partial-tile bound caps the split count)."""
    ns, ks = hp.plan(49152, 262144)
    assert (ns, ks) == (3, 2732 * 32)
    assert hp.chain_steps(49152, 262144) == 2732
