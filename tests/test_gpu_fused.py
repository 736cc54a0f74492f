"""GPU parity of the fused in_proj + ShortConv forward (lfm2sc_fused_prefill, through the C ABI) against the fp64
oracle (oracle.fused_prefill: the in_proj dot products, then the ShortConv prefill).

B, C and xv stay in fp32 inside the kernel, so y, the final states and the optional in_proj output carry one bf16
rounding of an fp32 result: they are compared within the bf16 tolerance (abs-or-rel 2e-2), and slots the call must
not touch are compared bit for bit."""
import pytest
import torch

import oracle
from gated_short_causal_amd import (lfm2sc_fused_prefill, lfm2sc_fused_prefill_workspace_bytes,
                                    lfm2sc_prefill_ragged)
from gated_short_causal_amd import workloads as wl
from tests.parity_util import assert_bits, assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda"
BF = torch.bfloat16

# For D in {1024, 1536, 2048} the library picks a tile form per call by expected span: wide tiles (H % 128 == 0)
# overlapping by K-1 rows, wide tiles with K-1 halo rows, split tiles (64 rows x 32 or 64 channels, each of the
# 4 waves reducing a quarter of D, K-1 halo rows) or mid tiles (128 rows x 64 channels, 8 waves, two halves of
# D, K-1 halo rows); the 4-wave tile (256 rows x 64 channels, "narrow") serves the other shapes.
# LFM2SC_FUSED_SPLIT, LFM2SC_FUSED_HALO and LFM2SC_FUSED_WIDE force one.
FORMS = {"overlap": {"LFM2SC_FUSED_SPLIT": "0", "LFM2SC_FUSED_HALO": "0"},
         "halo": {"LFM2SC_FUSED_SPLIT": "0", "LFM2SC_FUSED_HALO": "1"},
         "split32": {"LFM2SC_FUSED_SPLIT": "32"},
         "split64": {"LFM2SC_FUSED_SPLIT": "64"},
         "mid": {"LFM2SC_FUSED_SPLIT": "128"},
         "narrow": {"LFM2SC_FUSED_SPLIT": "0", "LFM2SC_FUSED_WIDE": "0"}}


@pytest.fixture(params=sorted(FORMS))
def form(request, monkeypatch):
    for k in ("LFM2SC_FUSED_SPLIT", "LFM2SC_FUSED_HALO", "LFM2SC_FUSED_WIDE"):
        monkeypatch.delenv(k, raising=False)
    for k, v in FORMS[request.param].items():
        monkeypatch.setenv(k, v)
    return request.param


def _say(msg):
    print(msg, flush=True)


def _nan(shape):
    return torch.full(shape, float("nan"), dtype=BF, device=DEV)


def _run(c, with_io=False, y_pad=0, io_pad=0):
    g = c.to(DEV)
    rows = c.x.shape[0]
    N = c.cu.numel() - 1
    y = _nan((rows, c.H + y_pad))[:, : c.H] if y_pad else _nan((rows, c.H))
    io = None
    if with_io:
        io = _nan((rows, 3 * c.H + io_pad))[:, : 3 * c.H] if io_pad else _nan((rows, 3 * c.H))
    ws = None
    if c.pool is not None:
        ws = torch.empty(max(16, lfm2sc_fused_prefill_workspace_bytes(BF, c.H, c.K, N, True)), dtype=torch.uint8,
                         device=DEV)
    x = g.x[:, : c.D] if g.x.shape[1] != c.D else g.x
    lfm2sc_fused_prefill(x, g.W_in, g.cu, g.w, y, g.pool, g.slot_idx, bias=g.bias, in_proj_out=io, workspace=ws)
    torch.cuda.synchronize()
    return y.cpu(), (None if io is None else io.cpu()), (None if g.pool is None else g.pool.cpu())


def _check(c, y, io, pool, what):
    x = c.x[:, : c.D]
    y_ref, p_ref, ip_ref = oracle.fused_prefill(x, c.W_in, c.cu, c.w, c.pool, c.slot_idx, bias=c.bias)
    covered = int(c.cu[-1])
    assert_close(y[:covered], y_ref[:covered], BF, f"{what}: y")
    if covered < y.shape[0]:
        assert torch.isnan(y[covered:].float()).all(), f"{what}: rows outside every sequence were written"
    if io is not None:
        assert_close(io[:covered], ip_ref[:covered], BF, f"{what}: in_proj_out")
    if pool is not None:
        assert_close(pool, p_ref, BF, f"{what}: final states")
        lens = (c.cu[1:] - c.cu[:-1]).tolist()
        touched = {int(s) for s, n in zip(c.slot_idx.tolist(), lens) if n > 0}
        for s in range(pool.shape[0]):
            if s not in touched:
                assert_bits(pool[s], c.pool[s], f"{what}: slot {s} must be untouched")


@pytest.mark.parametrize("K", [1, 2, 3, 4])
def test_fused_ragged_pool_bias(K):
    lens = [37, 1, 0, 300, 5, 2]
    _say(f"case: fused ragged K={K} lens={lens} H=128 D=384 pool+bias")
    c = wl.fused_case(500 + K, lens, H=128, K=K, D=384, slots=9, bias=True)
    y, io, pool = _run(c, with_io=True)
    _check(c, y, io, pool, f"K={K}")


def test_fused_training_shape_no_pool():
    """One sequence over several row tiles, no pool (zero initial state, no state out), in_proj kept."""
    _say("case: fused one sequence T=1000 H=256 D=256 no pool")
    c = wl.fused_case(510, [1000], H=256, K=3, D=256)
    y, io, pool = _run(c, with_io=True)
    _check(c, y, io, pool, "train")


def test_fused_short_sequences_and_tail_rows():
    """Many sequences shorter than K in one tile and across a tile boundary, rows after the last sequence,
    padded x / y / in_proj rows."""
    lens = [1, 2, 1, 0, 3, 1] * 50
    _say(f"case: fused {len(lens)} short sequences, tail rows, padded strides")
    c = wl.fused_case(511, lens, H=64, K=3, D=128, slots=len(lens) + 4, bias=True, x_pad=8, tail_rows=7)
    y, io, pool = _run(c, with_io=True, y_pad=8, io_pad=16)
    _check(c, y, io, pool, "short")


def test_fused_out_of_range_slots():
    lens = [4, 9, 2]
    _say("case: fused out-of-range slot ids")
    c = wl.fused_case(512, lens, H=64, K=3, D=128, slots=5)
    c.slot_idx = torch.tensor([1, 5, -2], dtype=torch.int32)
    y, io, pool = _run(c)
    # sequences 1 and 2 start from a zero state and write nothing
    zero = c.pool.clone()
    zero[:] = 0
    y_ref_ok, p_ok, _ = oracle.fused_prefill(c.x, c.W_in, c.cu, c.w, c.pool, torch.tensor([1, 2, 3]))
    y_ref_zero, _, _ = oracle.fused_prefill(c.x, c.W_in, c.cu, c.w, zero, torch.tensor([0, 1, 2]))
    assert_close(y[:4], y_ref_ok[:4], BF, "valid slot rows")
    assert_close(y[4:], y_ref_zero[4:], BF, "rows of out-of-range slots")
    assert_close(pool[1], p_ok[1], BF, "valid slot state")
    for s in (0, 2, 3, 4):
        assert_bits(pool[s], c.pool[s], f"slot {s} untouched")


@pytest.mark.parametrize("nc", ["32", "64", "128"])
def test_fused_split_out_of_range_slots(nc, monkeypatch):
    """Split tiles with slot ids outside the pool: those sequences start from a zero state and write no state;
    a valid slot still gets its final state; the other slots stay untouched."""
    monkeypatch.setenv("LFM2SC_FUSED_SPLIT", nc)
    lens = [4, 70, 2, 1]
    _say(f"case: fused split{nc} out-of-range slot ids H=128 D=1024")
    c = wl.fused_case(516, lens, H=128, K=3, D=1024, slots=6)
    c.slot_idx = torch.tensor([1, 6, -2, 4], dtype=torch.int32)
    y, io, pool = _run(c)
    zero = c.pool.clone()
    zero[:] = 0
    y_ok, p_ok, _ = oracle.fused_prefill(c.x, c.W_in, c.cu, c.w, c.pool, torch.tensor([1, 2, 3, 4]))
    y_zero, _, _ = oracle.fused_prefill(c.x, c.W_in, c.cu, c.w, zero, torch.tensor([0, 1, 2, 3]))
    assert_close(y[:4], y_ok[:4], BF, "valid slot rows")
    assert_close(y[4:76], y_zero[4:76], BF, "rows of out-of-range slots")
    assert_close(y[76:], y_ok[76:], BF, "valid slot rows after them")
    assert_close(pool[1], p_ok[1], BF, "valid slot state")
    assert_close(pool[4], p_ok[4], BF, "valid slot state")
    for s in (0, 2, 3, 5):
        assert_bits(pool[s], c.pool[s], f"slot {s} untouched")


def test_fused_lfm2_shape_sampled_channels(form):
    """LFM2-1.2B layer shape (H = D = 2048) over 4096 tokens in 3 ragged sequences with a pool; the oracle
    computes 24 sampled channels (channels are independent once in_proj is formed)."""
    lens = [1500, 7, 2589]
    _say(f"case: fused H=2048 D=2048 T=4096 ragged, sampled channels, {form} tiles")
    c = wl.fused_case(513, lens, H=2048, K=3, D=2048, slots=6, bias=True)
    y, io, pool = _run(c, with_io=True)
    chans = torch.tensor([0, 1, 31, 32, 63, 64, 100, 511, 512, 777, 1023, 1024, 1300, 1535, 1536, 1600, 1800,
                          1983, 2000, 2014, 2031, 2040, 2046, 2047])
    H = c.H
    rows = torch.cat([chans, chans + H, chans + 2 * H])
    y_ref, p_ref, ip_ref = oracle.fused_prefill(c.x, c.W_in[rows], c.cu, c.w[chans], c.pool[:, chans, :],
                                                c.slot_idx, bias=c.bias[chans])
    assert_close(y[:, chans], y_ref, BF, "y (sampled)")
    assert_close(io[:, rows], ip_ref, BF, "in_proj_out (sampled)")
    assert_close(pool[:, chans, :], p_ref, BF, "final states (sampled)")


def test_fused_in_proj_matches_torch_gemm():
    """The in_proj the fused call hands to the backward against torch's GEMM of the same bf16 operands (fp32
    accumulation, rounded to bf16).  y is not compared with the unfused path (a bf16 GEMM followed by
    lfm2sc_prefill_ragged): that path rounds B, C and xv before the conv, so it is itself an approximation whose
    distance from the fused result is not bounded by one bf16 tolerance; both are checked against the oracle."""
    lens = [700, 0, 333, 64]
    _say("case: fused in_proj_out vs torch GEMM")
    c = wl.fused_case(514, lens, H=512, K=3, D=1024, slots=5, bias=True)
    y, io, pool = _run(c, with_io=True)
    g = c.to(DEV)
    ip = torch.matmul(g.x.float(), g.W_in.float().t()).to(BF).cpu()
    assert_close(io, ip.double(), BF, "in_proj_out vs torch GEMM")
    _check(c, y, io, pool, "vs oracle")


def test_fused_deterministic():
    c = wl.fused_case(515, [400, 90], H=128, K=3, D=256, slots=3)
    a = _run(c, with_io=True)
    b = _run(c, with_io=True)
    for u, v, n in zip(a, b, ("y", "in_proj", "pool")):
        assert_bits(u, v, f"rerun {n}")


@pytest.mark.parametrize("K", [1, 2, 3, 4])
@pytest.mark.parametrize("H", [128, 256])
def test_fused_wide_tiles(K, H, form):
    """Channel counts that are multiples of 128 with D = 1024 run the 8-wave wide tile (256 rows x 128 channels):
    ragged sequences, ones shorter than K, a sequence across several row tiles, rows after the last sequence,
    padded x / y / in_proj rows, a pool and a bias."""
    lens = [37, 1, 0, 300, 5, 2, 1, 2, 3, 600]
    _say(f"case: fused wide tile K={K} H={H} D=1024 lens={lens} padded, tail rows, {form} tiles")
    c = wl.fused_case(520 + K + H, lens, H=H, K=K, D=1024, slots=len(lens) + 2, bias=True, x_pad=8, tail_rows=5)
    y, io, pool = _run(c, with_io=True, y_pad=8, io_pad=16)
    _check(c, y, io, pool, f"wide K={K} H={H}")


@pytest.mark.parametrize("D", [1536, 2048])
def test_fused_wide_other_depths(D, form):
    """The wide tile's straight-line reductions for the other LFM2 hidden sizes, no pool."""
    _say(f"case: fused wide tile D={D} H=128 one sequence, {form} tiles")
    c = wl.fused_case(530 + D, [777], H=128, K=3, D=D)
    y, io, pool = _run(c, with_io=True)
    _check(c, y, io, pool, f"wide D={D}")


def test_fused_graph_replays_match_eager():
    """The fused call with a pool (tile kernel + state install kernel) and the in_proj output, captured in a
    HIP graph: each replay, with eager work and syncs in between and the pool restored first, must reproduce
    the eager results bit for bit."""
    lens = [300, 1, 0, 77, 2]
    _say(f"case: fused graph capture lens={lens} H=256 D=1024")
    c = wl.fused_case(540, lens, H=256, K=3, D=1024, slots=7, bias=True)
    g = c.to(DEV)
    T, N = c.x.shape[0], len(lens)
    pool0 = g.pool.clone()
    y = torch.empty(T, c.H, dtype=BF, device=DEV)
    io = torch.empty(T, 3 * c.H, dtype=BF, device=DEV)
    ws = torch.empty(lfm2sc_fused_prefill_workspace_bytes(BF, c.H, c.K, N, True), dtype=torch.uint8, device=DEV)

    def call():
        lfm2sc_fused_prefill(g.x, g.W_in, g.cu, g.w, y, g.pool, g.slot_idx, bias=g.bias, in_proj_out=io,
                             workspace=ws)

    call()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (y, io, g.pool)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        g.pool.copy_(pool0)
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    g.pool.copy_(pool0)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        call()
    for rep in range(3):
        y.fill_(float("nan"))
        io.fill_(float("nan"))
        g.pool.copy_(pool0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("y", "in_proj_out", "pool"), (y, io, g.pool), ref):
            assert_bits(a, b, f"replay {rep}: {name}")
    _check(c, ref[0].cpu(), ref[1].cpu(), ref[2].cpu(), "graph")


@pytest.mark.parametrize("K", [2, 3, 4])
def test_fused_wide_tile_boundaries(K, form):
    """Tile boundaries in both forms (halo tiles start at multiples of 256 and take the history of their first
    K-1 rows from the halo rows): sequences that end exactly at a 256-row boundary, one row before it, and a
    2-token sequence across it (its second token is row 0 of a halo tile, its first is a halo row)."""
    lens = [256, 255, 2, 254, 1, 300]
    _say(f"case: fused wide tile boundaries K={K} lens={lens} H=128 D=1024 pool, {form} tiles")
    c = wl.fused_case(550 + K, lens, H=128, K=K, D=1024, slots=len(lens) + 1, bias=True)
    y, io, pool = _run(c, with_io=True)
    _check(c, y, io, pool, f"boundaries K={K}")


@pytest.mark.parametrize("nc", ["32", "64", "128"])
@pytest.mark.parametrize("K", [1, 2, 3, 4])
@pytest.mark.parametrize("H", [64, 192])
def test_fused_split_tiles(K, H, nc, monkeypatch):
    """Split tiles of 32 and 64 channels and mid tiles (nc = 128: 128 rows x 64 channels) also serve channel
    counts that are not multiples of 128.  A split tile starts at a multiple of 64 rows (a mid tile at a
    multiple of 128) and takes the history of its first K-1 rows from halo rows: sequences that end exactly at
    such a boundary, one row before and one row after it, a 2-token sequence across it, sequences shorter than
    K, an empty one, a sequence over several tiles, rows after the last sequence, padded rows, a pool, a bias."""
    monkeypatch.setenv("LFM2SC_FUSED_SPLIT", nc)
    lens = [64, 63, 2, 65, 1, 0, 190, 5, 1, 2]
    _say(f"case: fused split tiles nc={nc} K={K} H={H} D=1024 lens={lens} padded, tail rows")
    c = wl.fused_case(560 + K + H, lens, H=H, K=K, D=1024, slots=len(lens) + 2, bias=True, x_pad=8, tail_rows=9)
    y, io, pool = _run(c, with_io=True, y_pad=8, io_pad=16)
    _check(c, y, io, pool, f"split{nc} K={K} H={H}")


def test_fused_one_token_sequences_lfm2_shape():
    """256 one-token sequences at the LFM2-1.2B layer shape (H = D = 2048) with a pool: every conv history comes
    from the slots.  The library's own choice of tile form (split tiles for inputs this short); the oracle
    computes sampled channels."""
    lens = [1] * 256
    _say("case: fused 256 one-token sequences H=2048 D=2048 pool, default tile form")
    c = wl.fused_case(570, lens, H=2048, K=3, D=2048, slots=300, bias=True)
    y, io, pool = _run(c, with_io=True)
    chans = torch.tensor([0, 5, 63, 64, 127, 640, 1023, 1024, 1999, 2047])
    H = c.H
    rows = torch.cat([chans, chans + H, chans + 2 * H])
    y_ref, p_ref, ip_ref = oracle.fused_prefill(c.x, c.W_in[rows], c.cu, c.w[chans], c.pool[:, chans, :],
                                                c.slot_idx, bias=c.bias[chans])
    assert_close(y[:, chans], y_ref, BF, "y (sampled)")
    assert_close(io[:, rows], ip_ref, BF, "in_proj_out (sampled)")
    assert_close(pool[:, chans, :], p_ref, BF, "final states (sampled)")


@pytest.mark.parametrize("seed", [580, 581, 582])
def test_fused_random_ragged_all_forms(seed, form):
    """Seeded random ragged batches (1-40 sequences, lengths 0-300 with many short ones, a pool with out-of-range
    slots mixed in, a bias, padded rows) through every tile form at H = 128, D = 1024, K drawn from 1-4."""
    g = torch.Generator().manual_seed(seed)
    N = int(torch.randint(1, 41, (1,), generator=g))
    short = torch.randint(0, 4, (N,), generator=g)
    long_ = torch.randint(0, 301, (N,), generator=g)
    pick = torch.rand(N, generator=g) < 0.4
    lens = torch.where(pick, short, long_).tolist()
    K = int(torch.randint(1, 5, (1,), generator=g))
    _say(f"case: fused random ragged seed={seed} N={N} K={K} T={sum(lens)} {form} tiles")
    c = wl.fused_case(seed, lens, H=128, K=K, D=1024, slots=N + 3, bias=True, x_pad=8, tail_rows=3)
    bad = torch.rand(N, generator=g) < 0.15
    c.slot_idx = torch.where(bad, torch.full_like(c.slot_idx, -1), c.slot_idx)
    y, io, pool = _run(c, with_io=True, y_pad=8)
    zero_for_bad = c.pool.clone()
    # the oracle's reading of an out-of-range slot: zero initial state, nothing written; give those sequences
    # spare slots filled with zeros and compare the states of the valid slots only
    spare = [s for s in range(N + 3) if s not in set(c.slot_idx.tolist())]
    sl = c.slot_idx.clone()
    for i in torch.nonzero(bad).flatten().tolist():
        sl[i] = spare.pop()
        zero_for_bad[sl[i]] = 0
    y_ref, p_ref, ip_ref = oracle.fused_prefill(c.x[:, : c.D], c.W_in, c.cu, c.w, zero_for_bad, sl, bias=c.bias)
    covered = int(c.cu[-1])
    assert_close(y[:covered], y_ref[:covered], BF, "y")
    assert_close(io[:covered], ip_ref[:covered], BF, "in_proj_out")
    for i in range(N):
        s = int(c.slot_idx[i])
        if s >= 0:
            if lens[i] > 0:
                assert_close(pool[s], p_ref[s], BF, f"state of sequence {i}")
            else:
                assert_bits(pool[s], c.pool[s], f"slot of empty sequence {i} untouched")
    named = {int(s) for s in c.slot_idx.tolist() if s >= 0}
    for s in range(N + 3):
        if s not in named:
            assert_bits(pool[s], c.pool[s], f"slot {s} untouched")


def test_fused_plan_on_the_device(monkeypatch):
    """On MI355X the occupancy query behind the tiling choice gives one workgroup per CU for each tile form, so
    the plans match the ones worked out for 256 resident workgroups (tests/test_fused_plan.py)."""
    from gated_short_causal_amd import lfm2sc_fused_prefill_plan as plan
    for k in ("LFM2SC_FUSED_SPLIT", "LFM2SC_FUSED_HALO", "LFM2SC_FUSED_WIDE"):
        monkeypatch.delenv(k, raising=False)
    assert torch.cuda.get_device_properties(0).multi_processor_count == 256
    expected = {64: 32, 256: 32, 512: 64, 768: 128, 1024: 128, 1536: 1, 2048: 1, 4096: 2, 8192: 2, 65536: 1}
    assert {T: plan(2048, 3, 2048, T) for T in expected} == expected


def test_fused_wider_channels_sampled(form):
    """H = 4096 channels (twice LFM2-1.2B's) at D = 2048 over ragged sequences with a pool, every tile form;
    the oracle computes sampled channels, including the last tile's."""
    lens = [900, 3, 1200, 1]
    _say(f"case: fused H=4096 D=2048 lens={lens} pool, sampled channels, {form} tiles")
    c = wl.fused_case(590, lens, H=4096, K=3, D=2048, slots=6, bias=True)
    y, io, pool = _run(c, with_io=True)
    chans = torch.tensor([0, 31, 32, 127, 128, 2047, 2048, 3000, 4031, 4032, 4095])
    H = c.H
    rows = torch.cat([chans, chans + H, chans + 2 * H])
    y_ref, p_ref, ip_ref = oracle.fused_prefill(c.x, c.W_in[rows], c.cu, c.w[chans], c.pool[:, chans, :],
                                                c.slot_idx, bias=c.bias[chans])
    assert_close(y[:, chans], y_ref, BF, "y (sampled)")
    assert_close(io[:, rows], ip_ref, BF, "in_proj_out (sampled)")
    assert_close(pool[:, chans, :], p_ref, BF, "final states (sampled)")
