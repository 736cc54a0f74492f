"""Host logic of the fused forward's tiling choice (lfm2sc_fused_prefill_plan, no GPU): the expected plans are
worked out by hand from the cost model, rounds of 256 resident workgroups x a tile's cost relative to a wide
overlapping tile (split tiles 0.30 at 32 channels and 0.45 at 64, mid tiles 0.60, wide halo tiles 1.21, the
4-wave tile 0.80), e.g. T = 1024 at H = D = 2048: mid tiles 8 x 32 = 256 (one round, 0.60) against 64-channel
split tiles 16 x 32 = 512 (two rounds, 0.90) and 5 x 16 = 80 overlapping wide tiles (one round, 1.00)."""
import pytest

from gated_short_causal_amd import lfm2sc_fused_prefill_plan as plan

WIDE, HALO, MAIN, MID = 1, 2, 3, 128
ENV = ("LFM2SC_FUSED_SPLIT", "LFM2SC_FUSED_HALO", "LFM2SC_FUSED_WIDE")


@pytest.fixture(autouse=True)
def _clean_env(monkeypatch):
    for k in ENV:
        monkeypatch.delenv(k, raising=False)


@pytest.mark.parametrize("T,expected", [
    (64, 32),          # 64-row split tiles: 1 x 64 tiles of 32 channels, one round at 0.30
    (256, 32),         # 4 x 64 = 256 split tiles of 32 channels: one round at 0.30
    (512, 64),         # 32 channels: 512 tiles, two rounds (0.60); 64 channels: 256 tiles, one round (0.45)
    (768, MID),        # mid: 6 x 32 = 192 tiles (0.60) against two rounds of split tiles (0.90)
    (1024, MID),
    (1536, WIDE),      # 7 x 16 = 112 overlapping wide tiles, one round (1.00); mid two rounds (1.20)
    (2048, WIDE),
    (4096, HALO),      # halo: 16 x 16 = 256 tiles, one round (1.21); overlapping: 17 x 16 = 272, two rounds
    (8192, HALO),      # halo 512 tiles, 2 x 1.21; overlapping 528 tiles, three rounds
    (65536, WIDE),     # overlapping 259 x 16 = 4144 tiles, 17 rounds; halo 4096 tiles, 16 x 1.21
])
def test_lfm2_shape(T, expected):
    assert plan(2048, 3, 2048, T) == expected


def test_other_shapes():
    assert plan(192, 3, 1024, 65536) == MAIN      # H % 128 != 0: 4-wave tiles, 259 x 3 = 777 (4 rounds, 3.2)
    assert plan(192, 3, 1024, 256) == 32          # split tiles 4 x 6 = 24 (0.30) against the 4-wave tile (0.80)
    assert plan(128, 3, 384, 100) == MAIN         # D outside {1024, 1536, 2048}: the 4-wave tile's loop form
    assert plan(2048, 1, 2048, 4096) == WIDE      # K = 1: 256-row tiles overlap by nothing, 256 tiles, one round
    assert plan(2048, 3, 2048, 0) == 0            # no token, nothing launched


@pytest.mark.parametrize("args", [(100, 3, 2048, 10), (2048, 5, 2048, 10), (2048, 0, 2048, 10), (2048, 3, 100, 10),
                                  (2048, 3, 2048, -1), (2048, 3, 2048, 1 << 31), (32, 3, 1024, 10)])
def test_rejected_sizes(args):
    assert plan(*args) < 0


def test_environment_overrides(monkeypatch):
    monkeypatch.setenv("LFM2SC_FUSED_SPLIT", "0")
    assert plan(2048, 3, 2048, 256) == WIDE       # 2 x 16 overlapping tiles vs 1 x 16 halo tiles: one round each
    monkeypatch.setenv("LFM2SC_FUSED_HALO", "1")
    assert plan(2048, 3, 2048, 65536) == HALO
    monkeypatch.setenv("LFM2SC_FUSED_WIDE", "0")
    assert plan(2048, 3, 2048, 65536) == MAIN
    monkeypatch.delenv("LFM2SC_FUSED_HALO")
    monkeypatch.delenv("LFM2SC_FUSED_WIDE")
    for v, expected in (("32", 32), ("64", 64), ("128", MID)):
        monkeypatch.setenv("LFM2SC_FUSED_SPLIT", v)
        assert plan(2048, 3, 2048, 65536) == expected
    monkeypatch.setenv("LFM2SC_FUSED_SPLIT", "1")  # always, the cheapest of the three: mid tiles, 64 rounds x 0.60
    assert plan(2048, 3, 2048, 65536) == MID
