"""GPU parity of the grouped launch (w12_gemm_group / w12_gemm_group_q): several independent
W12 products of one M in one stream-K launch.

Every product's Y is checked against the FP64 oracle within 2^-12 * sum|x w| (the exact pass
against W, the Q pass against the oracle's Q view), bitwise repeatable, and compared with the
single-product launch.  Small work-group counts force work-group ranges that cross product
boundaries and tiles split over many work-groups.  The full decoder-layer group is checked on
sampled channels at the sizes and launch configuration the benchmark uses.
"""
import numpy as np
import pytest
import torch

import lossless_bit_weight_encode_amd as w12
import w12_synth as S
from oracle import w12_oracle as O
from gpu_util import say, to_dev

pytestmark = pytest.mark.gpu

# mixed shapes, every K a multiple of 16: tiny case with infs, a 40-binade mix, heavy tails,
# a channel of zeros only, a single row block, a ragged N
MEMBERS = {
    "tiny_256x512": lambda: S.tiny_weights(0),
    "gauss_300x4096": lambda: S.layer_matrix(torch.Generator().manual_seed(5), 300, 4096),
    "heavy_64x2048": lambda: S.heavy_tail_weights(1000, 64, 2048),
    "wide_37x1008": lambda: S.random_bits_matrix(np.random.default_rng(11), 37, 1008, "wide"),
    "all_escapes_20x96": lambda: np.zeros((20, 96), dtype=np.uint16),
    "single_1x16": lambda: S.random_bits_matrix(np.random.default_rng(4), 1, 16, "wide"),
    "gauss_130x640": lambda: S.layer_matrix(torch.Generator().manual_seed(6), 130, 640),
    "wide_70x272": lambda: S.random_bits_matrix(np.random.default_rng(12), 70, 272, "wide"),
    "no_escapes_64x512": lambda: S.to_bf16_bits(1.0 + torch.rand(64, 512, generator=torch.Generator().manual_seed(8))),
}
_cache = {}


def counter_bytes():
    """The counter region at the start of every GEMM workspace (the same for every plan)."""
    return w12.gemm_plan(1, 16, 16)["counter_bytes"]


def member(name):
    if name not in _cache:
        w = MEMBERS[name]()
        _cache[name] = (w, w12.encode(to_dev(w)), O.encode(w))
    return _cache[name]


def run_group(names, m, seed, qpass=False, repeats=2):
    ws_, ts, xs = [], [], []
    for i, nm in enumerate(names):
        w, t, _ = member(nm)
        ws_.append(w)
        ts.append(t)
        xs.append(S.activations(m, w.shape[1], 7000 + seed + 31 * i + m))
    xd = [to_dev(x) for x in xs]
    ws = w12.gemm_group_workspace(m, ts)
    ys = w12.gemm_group(xd, ts, ws=ws, qpass=qpass)
    torch.cuda.synchronize()
    for _ in range(repeats - 1):
        ys2 = w12.gemm_group(xd, ts, ws=ws, qpass=qpass)
        torch.cuda.synchronize()
        for a, b in zip(ys, ys2):
            assert torch.equal(a, b), "grouped GEMM output is not bitwise repeatable"
    # every call leaves the arrival counters (a region of the same size for every plan) zero
    assert int(ws[:counter_bytes()].count_nonzero()) == 0
    for i, nm in enumerate(names):
        yh = ys[i].cpu().numpy()
        if qpass:
            bad, worst = O.gemm_q_check(xs[i], member(nm)[2], yh)
        else:
            bad, worst = O.gemm_check(xs[i], ws_[i], yh)
        assert bad == 0, f"{nm} (item {i}) M={m}: {bad} outputs outside tolerance (worst rel {worst:.3g})"
    return xs, xd, ys


# eight members (a full group of the kernel-argument form), the no-escape one included; the size
# test cycles over all of them
ALL = [nm for nm in MEMBERS if nm != "wide_70x272"]
assert len(ALL) == w12.GROUP_INLINE


def many(count, step=5):
    """count items cycling over every member (groups past GROUP_INLINE keep their arguments in
    the workspace)."""
    every = list(MEMBERS)
    return [every[(step * i + i // len(every)) % len(every)] for i in range(count)]


@pytest.mark.parametrize("m", [1, 2, 3, 8, 16, 17, 32, 33, 48, 64])
def test_group_within_tolerance(m):
    say(f"[group] M={m} members={len(ALL)}")
    run_group(ALL, m, seed=0)


@pytest.mark.parametrize("grid", [1, 2, 3, 7, 50])
@pytest.mark.parametrize("m", [1, 16, 40])
def test_group_small_grids(monkeypatch, grid, m):
    """Few work-groups: ranges cross product boundaries and tiles split over many segments."""
    monkeypatch.setenv("W12_MAX_GRID", str(grid))
    run_group(ALL[:5], m, seed=100 + grid)


@pytest.mark.parametrize("m", [3, 5, 8])
def test_group_gemv_path(monkeypatch, m):
    monkeypatch.setenv("W12_GEMV_MAX_M", "8")
    run_group(ALL, m, seed=200)


@pytest.mark.parametrize("m", [1, 16, 33, 64])
def test_group_qpass_within_tolerance(m):
    run_group(ALL, m, seed=300, qpass=True)


def test_group_sizes_one_to_past_inline():
    for count in range(1, w12.GROUP_INLINE + 4):
        every = list(MEMBERS)
        names = [every[(3 * i) % len(every)] for i in range(count)]
        say(f"[group] count={count} M=16")
        run_group(names, 16, seed=400 + count, repeats=1)


@pytest.mark.parametrize("count", [9, 33])
@pytest.mark.parametrize("m", [1, 2, 16, 32, 40, 64])
def test_large_group_within_tolerance(m, count):
    """More products than the kernel arguments hold: the argument blocks go to the workspace."""
    say(f"[group] count={count} M={m}")
    run_group(many(count), m, seed=700 + count)


@pytest.mark.parametrize("grid", [1, 2, 3, 7, 50])
@pytest.mark.parametrize("m", [1, 16])
def test_large_group_small_grids(monkeypatch, grid, m):
    """Few work-groups over 20 products: one work-group's range walks across many products."""
    monkeypatch.setenv("W12_MAX_GRID", str(grid))
    say(f"[group] count=20 M={m} grid={grid}")
    run_group(many(20), m, seed=800 + grid)


@pytest.mark.parametrize("m", [5, 8])
def test_large_group_gemv_path(monkeypatch, m):
    monkeypatch.setenv("W12_GEMV_MAX_M", "8")
    run_group(many(12), m, seed=850)


@pytest.mark.parametrize("m", [1, 16, 33])
def test_large_group_qpass_within_tolerance(m):
    run_group(many(17), m, seed=900, qpass=True)


def test_group_of_the_maximum_count():
    """W12_GROUP_MAX products (small members) in one launch, twice, bitwise repeatable."""
    small = ["single_1x16", "all_escapes_20x96", "wide_70x272", "wide_37x1008", "no_escapes_64x512"]
    names = [small[i % len(small)] for i in range(w12.GROUP_MAX)]
    say(f"[group] count={len(names)} M=16")
    run_group(names, 16, seed=950)
    with pytest.raises(w12.W12Error):
        w12.gemm_group([to_dev(S.activations(1, 16, 1))] * (w12.GROUP_MAX + 1), [member("single_1x16")[1]] * (w12.GROUP_MAX + 1))


@pytest.mark.parametrize("m", [1, 16, 64])
def test_group_matches_single_launch(m):
    """Grouped and single launches agree up to the FP32 summation order (each is within 2^-12 of
    the exact sum, so they differ by at most 2^-11 * sum|x w|)."""
    xs, xd, ys = run_group(ALL, m, seed=500, repeats=1)
    for i, nm in enumerate(ALL):
        w, t, _ = member(nm)
        y1 = w12.gemm(xd[i], t).cpu().numpy().astype(np.float64)
        _, a_ref = O.gemm_reference(xs[i], w)
        fin = np.isfinite(y1)
        assert (np.abs(y1[fin] - ys[i].cpu().numpy()[fin]) <= 2.0 ** -11 * a_ref[fin]).all(), nm


def test_group_rejects_unsupported():
    w, t, _ = member("gauss_300x4096")
    x = to_dev(S.activations(65, w.shape[1], 1))
    with pytest.raises(w12.W12Error):
        w12.gemm_group([x], [t])
    wr = S.random_bits_matrix(np.random.default_rng(3), 17, 33, "wide")
    tr = w12.encode(to_dev(wr, 40))
    with pytest.raises(w12.W12Error):
        w12.gemm_group([to_dev(S.activations(4, 33, 1), 40)], [tr])


# ---- full size: one dense decoder layer in one launch, sampled channels ---------------------

@pytest.mark.timeout(600)
@pytest.mark.parametrize("m", [1, 16, 32, 64])
def test_group_layer_full_size(m):
    say(f"[group] layer seed 0, M={m}")
    lay = S.layer(0)
    names = list(S.LAYER_ORDER)
    ts = [w12.encode(to_dev(lay[nm])) for nm in names]
    xs = [S.activations(m, S.LAYER_SHAPES[nm][1], S.x_seed(m, S.LAYER_SHAPES[nm][1])) for nm in names]
    xd = [to_dev(x) for x in xs]
    ws = w12.gemm_group_workspace(m, ts)
    ys = w12.gemm_group(xd, ts, ws=ws)
    torch.cuda.synchronize()
    ys2 = w12.gemm_group(xd, ts, ws=ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(m)
    for i, nm in enumerate(names):
        assert torch.equal(ys[i], ys2[i]), f"{nm}: not bitwise repeatable"
        n = S.LAYER_SHAPES[nm][0]
        rows = np.array(sorted(set(range(64)) | set(range(n - 64, n)) |
                               set(rng.choice(n, 128, replace=False).tolist())))
        yh = ys[i].cpu().numpy()
        bad, worst = O.gemm_check(xs[i], lay[nm][rows], yh[:, rows])
        assert bad == 0, f"{nm} M={m}: {bad} sampled outputs outside tolerance (worst rel {worst:.3g})"
        assert np.isfinite(yh).all()


@pytest.mark.timeout(900)
def test_group_whole_model_full_size():
    """The launch the benchmark times for a 64-layer model at M=32: 256 products of decoder-layer
    shapes in one launch (here layer 0's four matrices 64 times over, each with its own Y), on
    sampled channels of every product, twice, bitwise repeatable."""
    m, n_layers = 32, 64
    lay = S.layer(0)
    names = list(S.LAYER_ORDER)
    enc = {nm: w12.encode(to_dev(lay[nm])) for nm in names}
    xs = {nm: S.activations(m, S.LAYER_SHAPES[nm][1], S.x_seed(m, S.LAYER_SHAPES[nm][1])) for nm in names}
    xd = {nm: to_dev(xs[nm]) for nm in names}
    order = [nm for _ in range(n_layers) for nm in names]
    ts = [enc[nm] for nm in order]
    say(f"[group] whole model: {len(ts)} products M={m}")
    ws = w12.gemm_group_workspace(m, ts)
    ys = w12.gemm_group([xd[nm] for nm in order], ts, ws=ws)
    torch.cuda.synchronize()
    ys2 = w12.gemm_group([xd[nm] for nm in order], ts, ys=None, ws=ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(77)
    for i, nm in enumerate(order):
        assert torch.equal(ys[i], ys2[i]), f"item {i} ({nm}): not bitwise repeatable"
        n = S.LAYER_SHAPES[nm][0]
        rows = np.array(sorted(set(rng.choice(n, 24, replace=False).tolist()) | {0, n - 1}))
        yh = ys[i].cpu().numpy()
        bad, worst = O.gemm_check(xs[nm], lay[nm][rows], yh[:, rows])
        assert bad == 0, f"item {i} ({nm}): {bad} sampled outputs outside tolerance (worst rel {worst:.3g})"
        assert np.isfinite(yh).all()


@pytest.mark.parametrize("m", [1, 16, 40])
@pytest.mark.parametrize("count", [5, 13])
def test_group_deterministic_poisoned_workspace_and_canaries(monkeypatch, m, count):
    """20 grouped launches bitwise identical, with the partial region of the workspace (and the
    argument blocks of a large group) NaN-poisoned before every launch (a read of a partial never
    written would show) and canary values around every Y (nothing written outside Y).  A small
    grid makes most tiles split."""
    monkeypatch.setenv("W12_MAX_GRID", "7")
    names = many(count)
    ws_, ts, xs = [], [], []
    for i, nm in enumerate(names):
        w, t, _ = member(nm)
        ws_.append(w)
        ts.append(t)
        xs.append(S.activations(m, w.shape[1], 9000 + 17 * i + m))
    xd = [to_dev(x) for x in xs]
    canary = -12345.678
    bufs = [torch.full((m + 3, t.n + 11), canary, dtype=torch.float32, device="cuda") for t in ts]
    ys = [b[:m, :t.n] for b, t in zip(bufs, ts)]
    ws = w12.gemm_group_workspace(m, ts)
    cb = counter_bytes()
    outs = []
    for _ in range(20):
        ws[cb:].view(torch.uint8).fill_(0xFF)   # NaN patterns in every partial slot
        w12.gemm_group(xd, ts, ys, ws=ws)
        torch.cuda.synchronize()
        outs.append([y.cpu().numpy().view(np.uint32).copy() for y in ys])
        assert int(ws[:cb].count_nonzero()) == 0, "arrival counters must return to zero"
    for o in outs[1:]:
        for a, b in zip(o, outs[0]):
            assert np.array_equal(a, b)
    for i, (b, t) in enumerate(zip(bufs, ts)):
        bh = b.cpu().numpy()
        assert (bh[:m, t.n:] == np.float32(canary)).all(), f"item {i}: write past N"
        assert (bh[m:, :] == np.float32(canary)).all(), f"item {i}: write past M"
        bad, worst = O.gemm_check(xs[i], ws_[i], outs[0][i].view(np.float32))
        assert bad == 0, f"item {i}: {bad} outputs outside tolerance"


def test_workspace_reused_across_plans():
    """One workspace serves products whose plans differ (wide tiles, MFMA tiles, the wavefront
    GEMV, a grouped launch, then wide tiles again): the counter region is the same for every
    plan, so partial sums of one plan never land where another reads its counters.  Every
    output is checked against the oracle and the counters are zero after every call."""
    w, t, _ = member("gauss_300x4096")
    names = ALL[:4]
    gts = [member(nm)[1] for nm in names]
    need = max([w12.gemm_workspace_size(m, t.n, t.k) for m in (1, 16, 256)] +
               [w12.gemm_group_workspace_size(16, gts)])
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    w12.gemm_workspace_init(ws)
    cb = counter_bytes()
    plans = []
    for step, m in enumerate([256, 16, "group", 1, 256, 33]):
        say(f"[reuse] step {step} M={m}")
        if m == "group":
            xs = [S.activations(16, member(nm)[0].shape[1], 500 + i) for i, nm in enumerate(names)]
            ys = w12.gemm_group([to_dev(x) for x in xs], gts, ws=ws)
            torch.cuda.synchronize()
            for i, nm in enumerate(names):
                bad, worst = O.gemm_check(xs[i], member(nm)[0], ys[i].cpu().numpy())
                assert bad == 0, f"group item {nm}: {bad} outputs outside tolerance (worst rel {worst:.3g})"
        else:
            plans.append(w12.gemm_plan(m, t.n, t.k)["path"])
            # partial slots of the previous plan hold stale sums; poison them too
            ws[cb:].fill_(0xFF)
            x = S.activations(m, t.k, 600 + step)
            y = w12.gemm(to_dev(x), t, ws=ws)
            torch.cuda.synchronize()
            bad, worst = O.gemm_check(x, w, y.cpu().numpy())
            assert bad == 0, f"step {step} M={m}: {bad} outputs outside tolerance (worst rel {worst:.3g})"
        assert int(ws[:cb].count_nonzero()) == 0, f"step {step}: arrival counters must return to zero"
    assert sorted(set(plans)) == [1, 2, 3], plans   # GEMV, MFMA tiles and wide tiles all ran
