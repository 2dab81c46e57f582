"""The tile-choice cost model in bench.py against the library's own choice.

bench.py fits the model from a sweep, writes the table the library compiles
in (tg_tile_model.inc) and, for profiles/tile_sweep.md, predicts which
configuration the library will pick (model_choice, a copy of the host's
auto_tiles rule).  These CPU tests read the committed table back, check that
writing it again reproduces the file, and that model_choice picks what the
library's host-only tg_gemm_tiles_plan picks over a grid of shapes and CU
counts, so the summary's `auto` column is the library's choice.
"""
import os
import re

import pytest

import bench
import tiled_dense_gemm_tg_amd as tg

FIELDS = ("a1", "b1", "a2", "b2", "kappa", "phi", "rho")


def committed_model():
    rows = {}
    names = {v: k for k, v in bench.TILE_ENUM.items()}
    with open(bench.TILE_MODEL_INC) as fh:
        for line in fh:
            m = re.match(r"\s*\{(TG_TILES_\w+),\s*(.*)\},\s*$", line)
            if not m:
                continue
            vals = [float(v) for v in m.group(2).split(",")]
            rows[names[m.group(1)]] = dict(zip(FIELDS, vals[3:]))
    return rows


def test_table_lists_every_configuration_in_library_order():
    assert list(committed_model()) == list(bench.TILE_ENUM)
    assert set(bench.TILE_ENUM) == set(tg.TILES_NAMES[c] for c in tg.TILES_AXES)


def test_writing_the_table_again_reproduces_it(tmp_path):
    out = tmp_path / "model.inc"
    bench.write_tile_model({"model": committed_model()}, str(out))
    with open(bench.TILE_MODEL_INC) as fh:
        assert out.read_text() == fh.read()


@pytest.fixture(scope="module")
def lib():
    return tg.load_library()


SIZES = [1, 100, 128, 256, 257, 512, 1000, 2048, 3000, 4000, 4096, 4093, 8192, 11008]


@pytest.mark.parametrize("cus", [256, 304, 80])
def test_model_choice_is_the_library_choice(lib, cus):
    model = committed_model()
    checked = 0
    for M in SIZES[1:]:
        for N in SIZES:
            for K in (64, 1000, 4096, 4111, 8192):
                st, tiles = tg.tg_gemm_tiles_plan(M, N, K, cus)
                assert st == tg.TG_OK
                mine = bench.model_choice(model, M, N, K, cus, aligned=K % 8 == 0 and N % 8 == 0)
                assert mine == tg.TILES_NAMES[tiles], (M, N, K, cus)
                checked += 1
    assert checked == 13 * 14 * 5
