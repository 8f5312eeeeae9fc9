"""Every attention dispatch path on peaked scores, and the bitwise invariants on each (needs an MI355X).

Paths (kernel x schedule), each asserted with wf_chunk_attn_plan before it runs:
  pp_tile      bf16 cache, pages >= 64: LDS-DMA kernel, one workgroup per query tile
  pp_split     the same kernel under the split schedule (key parts + tails, LSE merge)
  fp8_tile     E4M3FN cache, pages >= 64: fp8-MFMA kernel, per tile
  fp8_split    the fp8-MFMA kernel under the split schedule
  staged_bf16  bf16 cache, pages of 40: register-staged kernel
  staged_fp8   E4M3FN cache, pages of 40: staged kernel dequantising to bf16

Peaked inputs.  The online softmax (Wave Forcing abstract: chunk-wise causal
attention; each kernel keeps a running reference point m for the exponentials)
has a branch that only runs when a later key tile scores well above the earlier
ones.  synth.staircase lifts dimension 0 of Q and K so that the scores climb by
up to 16 log2 units every 4 key tiles; before any kernel runs, the test shows
from the inputs alone (gpu_util.rescale_events) that this path's rescale rule
must fire at a dozen or more distinct tiles.  A "Q x 16" case (flat K, scores
with a standard deviation of about 5.8 log2 units) adds rows dominated by a
few keys.

Bars (against the float64 oracle on the same seeded inputs).
  bf16 caches: O max-abs 1e-2, mean-abs 1e-3, rel-L2 1e-2; LSE 4e-3 (the row sum
  is taken from the bf16-rounded weights, relative error <= 2^-8, and
  ln(1 + 2^-8) < 3.9e-3).
  E4M3FN caches: O rel-L2 6e-2 and max-abs max(5e-2, (eps_p + 2 Delta) max|V|),
  LSE 1e-3 + Delta_row (+ 3.9e-3 for the staged kernel's bf16 row sums), derived
  from the kernels' arithmetic:
    Delta_row = 2^-8 * scale * max_j sum_d |q_d k_jd| bounds the score error of a
    row -- the fp8-MFMA kernel carries Q as two E4M3FN terms (within 2^-8 |q|),
    the staged kernel rounds the dequantised K to bf16 (within 2^-8 |k|);
    a score error of at most Delta changes any softmax weight by a factor in
    [e^-2Delta, e^2Delta];
    eps_p is the relative rounding of the weights that multiply V: 2^-4 for
    E4M3FN weights (fp8 MFMA), 2^-7 for bf16 weights times bf16-rounded V
    (staged).
  Once a few keys dominate a row, the weight rounding is a fraction of one V
  row rather than an average over thousands, which is what the eps_p max|V|
  term covers.
"""
import numpy as np
import pytest
import torch

import chunk_causal_dit_wf_amd as wf
import synth
from gpu_util import Pair, dev, errors, host_codes, host_values, rescale_events, score_error_bounds, values_of

pytestmark = pytest.mark.gpu

H, D = 2, 128
N_KEYS = 6400
Q_OFF = [0, 37, 300, 301]
KB = [5, 0, 0]           # chunk 0 starts off the 8-key grid
KE = [6395, 6400, 6340]  # every chunk spans 100 key tiles; chunks 0 and 2 end inside a tile
STEP_KEYS = 256

SPEC = {
    "pp_tile": dict(dtype="bf16", P=256, ws=False, kernel="dma_bf16", sched="per_tile", kind="max11"),
    "pp_split": dict(dtype="bf16", P=256, ws=True, kernel="dma_bf16", sched="split", kind="max11"),
    "fp8_tile": dict(dtype="fp8", P=256, ws=False, kernel="dma_fp8", sched="per_tile", kind="max"),
    "fp8_split": dict(dtype="fp8", P=256, ws=True, kernel="dma_fp8", sched="split", kind="max"),
    "staged_bf16": dict(dtype="bf16", P=40, ws=False, kernel="staged_bf16", sched="per_tile", kind="max"),
    "staged_fp8": dict(dtype="fp8", P=40, ws=False, kernel="staged_fp8", sched="per_tile", kind="max"),
}
PATHS = list(SPEC)
BF16_MAX, BF16_MEAN, BF16_REL = 1e-2, 1e-3, 1e-2
FP8_MAX, FP8_REL = 5e-2, 6e-2


def say(*a):
    print(*a, flush=True)


class Case:
    """A cache holding N_KEYS keys for one path, the query codes, and the launch arguments."""

    def __init__(self, path, seed, peaked=True, q_mult=1.0, v_ones=False, table=None, fill=True, d=D):
        sp = SPEC[path]
        self.D = d
        self.path, self.sp = path, sp
        self.dtype = sp["dtype"]
        P = sp["P"]
        T = N_KEYS // P
        rng = np.random.default_rng(seed)
        num_pages = T + 3
        if table is None:
            table = rng.permutation(num_pages)[:T]
        std = 0.5 if self.dtype == "bf16" else 1.0
        q = synth.normal_f32((Q_OFF[-1], H, d), std, 77, seed, 0)
        k = synth.normal_f32((N_KEYS, H, d), std, 77, seed, 1)
        v = synth.normal_f32((N_KEYS, H, d), std, 77, seed, 2)
        if peaked:
            q, k = synth.staircase(q, k, np.arange(N_KEYS), 0, STEP_KEYS, 16.0, seed_words=(77, seed, 3))
        q[:, :, (1 if peaked else 0):] *= np.float32(q_mult)
        if v_ones:
            v[:] = 1.0
        self.pair = Pair(num_pages, P, H, d, self.dtype, table, fill_seed=seed + 1 if fill else None)
        if self.dtype == "fp8":
            kc, ks = synth.quantize_e4m3_pages(k, P)
            vc, vs = synth.quantize_e4m3_pages(v, P)
            self.pair.append(0, kc, vc, ks, vs)
        else:
            self.pair.append(0, synth.bf16_codes(k), synth.bf16_codes(v))
        self.q = synth.bf16_codes(q)
        self.qd = dev(self.q, "bf16")
        self.ws = wf.workspace_for(self.pair.gpu, "cuda") if sp["ws"] else None

    def check_plan(self, q_off=Q_OFF, kb=KB, ke=KE):
        wsb = 0 if self.ws is None else self.ws.numel()
        pl = wf.wf_chunk_attn_plan(self.pair.gpu, q_off, kb, ke, "bf16", wsb)
        say("%s plan: %s" % (self.path, pl))
        assert pl["kernel"] == self.sp["kernel"] and pl["schedule"] == self.sp["sched"], pl
        return pl

    def attend(self, q_off=Q_OFF, kb=KB, ke=KE, qd=None):
        return self.pair.attend(self.qd if qd is None else qd, q_off, kb, ke, workspace=self.ws)

    def events(self):
        """Tiles (over chunks 0 and 1, both heads) at which this path's rescale rule must fire."""
        K, _ = self.pair.ref.gather(0, N_KEYS)
        qv = values_of(self.q, "bf16")
        ev = set()
        for c in (0, 1):
            for h in range(H):
                rows = qv[Q_OFF[c]:Q_OFF[c + 1], h]
                ev |= set(rescale_events(rows, K[KB[c]:KE[c], h], KB[c], KE[c], self.sp["kind"]))
        return sorted(ev)


def check_bars(kernel_dtype, staged, got, ref, lse, rl, what, q_vals=None, K=None, V=None, args=None):
    """Compare with the oracle at the bars of the module docstring."""
    mx, mean, rel = errors(got, ref)
    lerr = np.abs(lse - rl)
    say("%s: max-abs %.3e mean-abs %.3e rel-L2 %.3e LSE %.3e (|ref| max %.3f)" % (what, mx, mean, rel, lerr.max(),
                                                                                  np.abs(ref).max()))
    assert np.isfinite(got).all()
    if kernel_dtype == "bf16":
        assert mx <= BF16_MAX and mean <= BF16_MEAN and rel <= BF16_REL, (what, mx, mean, rel)
        assert lerr.max() < 4e-3, (what, lerr.max())
        return
    delta = score_error_bounds(q_vals, K, *args)
    eps_p = 2.0 ** -7 if staged else 2.0 ** -4
    vmax = float(np.abs(V).max())
    bound = max(FP8_MAX, (eps_p + 2.0 * delta.max()) * vmax * 1.01)
    say("%s: fp8 max-abs bound %.3e (Delta max %.2e, max|V| %.2f)" % (what, bound, delta.max(), vmax))
    assert rel <= FP8_REL and mx <= bound, (what, mx, rel, bound)
    lbound = 1e-3 + delta + (3.9e-3 if staged else 0.0)
    assert np.all(lerr <= lbound), (what, float((lerr - lbound).max()))


def check_case(case, o, lse, q_off=Q_OFF, kb=KB, ke=KE, what=""):
    qv = values_of(case.q, "bf16")[:q_off[-1]]
    ro, rl = case.pair.reference(qv, q_off, kb, ke)
    K, V = case.pair.ref.gather(min(kb), max(ke))
    check_bars(case.dtype, case.path.startswith("staged"), host_values(o), ro, lse.cpu().numpy(), rl,
               "%s %s" % (case.path, what), qv, K, V, (q_off, kb, ke, min(kb)))


@pytest.mark.parametrize("path", PATHS)
def test_peaked_scores_every_path(path):
    say("case: peaked staircase, path", path)
    case = Case(path, seed=40)
    case.check_plan()
    ev = case.events()
    say("%s: %d tiles force a rescale (%s ...)" % (path, len(ev), ev[:8]))
    assert len(ev) >= 12 and ev[-1] >= 90, ev
    o, lse = case.attend()
    check_case(case, o, lse, what="staircase")


@pytest.mark.parametrize("path", PATHS)
def test_sharp_queries_every_path(path):
    """Flat K, Q scaled so that the scores have a standard deviation of about 4 nats (x16 on the
    N(0, 0.5^2) bf16 inputs, x4 on the N(0, 1) E4M3FN inputs): a handful of keys dominate each row."""
    say("case: sharp Q, path", path)
    mult = 16.0 if SPEC[path]["dtype"] == "bf16" else 4.0
    case = Case(path, seed=41, peaked=False, q_mult=mult)
    case.check_plan()
    o, lse = case.attend()
    qv = values_of(case.q, "bf16")
    K, _ = case.pair.ref.gather(0, N_KEYS)
    s = (qv[:37, 0] @ K[5:6395, 0].T) / np.sqrt(D)
    w = np.exp(s - s.max(axis=1, keepdims=True))
    top = (w.max(axis=1) / w.sum(axis=1))
    say("%s: score std %.2f nats, median largest softmax weight %.3f" % (path, s.std(), np.median(top)))
    assert np.median(top) > 0.2
    check_case(case, o, lse, what="sharp Q x%g" % mult)


@pytest.mark.parametrize("path", PATHS)
def test_head_dim_64_every_path(path):
    """head_dim 64 (the kernels' other instantiation) on every path: the peaked staircase against
    the oracle, and two runs bitwise equal."""
    say("case: D = 64, peaked staircase, path", path)
    case = Case(path, seed=46, d=64)
    case.check_plan()
    assert len(case.events()) >= 12
    o, lse = case.attend()
    check_case(case, o, lse, what="D64 staircase")
    o2, l2 = case.attend()
    assert np.array_equal(host_codes(o), host_codes(o2))
    assert np.array_equal(lse.cpu().numpy(), l2.cpu().numpy())


# ----------------------------------------------------------------------------- invariants on every path

@pytest.mark.parametrize("path", [p for p in PATHS if SPEC[p]["sched"] == "per_tile"])
def test_single_visible_key_returns_its_value(path):
    """Windows of one key: O = V[j] bitwise for bf16 caches; for E4M3FN caches the value
    decode(code) * scale rounded to bf16, to within one bf16 ulp (the kernel divides by a row sum
    that is 1 up to float32 rounding)."""
    say("case: single key, path", path)
    case = Case(path, seed=42)
    q_off, kb, ke = [0, 70, 75], [123, 4000], [124, 4001]
    case.check_plan(q_off, kb, ke)
    o, _ = case.attend(q_off, kb, ke, qd=case.qd[:75])
    got = host_codes(o)
    for c in range(2):
        kc, vc = case.pair.ref.gather_codes(kb[c], ke[c])
        if case.dtype == "bf16":
            want = np.broadcast_to(vc[0], (q_off[c + 1] - q_off[c], H, D))
            assert np.array_equal(got[q_off[c]:q_off[c + 1]], want)
        else:
            _, V = case.pair.ref.gather(kb[c], ke[c])
            want = V[0].astype(np.float32)
            g = host_values(o)[q_off[c]:q_off[c + 1]]
            ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(want), 1e-30))) - 7)
            assert np.all(np.abs(g - want) <= ulp * 1.0001), np.abs(g - want).max()


@pytest.mark.parametrize("path", PATHS)
def test_constant_values_give_ones_on_peaked_scores(path):
    """V = 1 everywhere: every output is 1 (rows of softmax sum to 1), on inputs whose scores
    force rescales.  bf16 MFMA kernels (bf16 caches, and E4M3FN caches dequantised to bf16):
    exactly 1.0 (the row sum is taken from the same bf16 weights the P.V product uses).  fp8-MFMA
    kernel: within 2^-4 (the weights are rounded to E4M3FN for the product, the row sum is not)."""
    say("case: V = 1, path", path)
    case = Case(path, seed=43, v_ones=True)
    case.check_plan()
    assert len(case.events()) >= 12
    o, lse = case.attend()
    got = host_values(o)
    d = np.abs(got - 1.0).max()
    say("%s: max |O - 1| = %.3e" % (path, d))
    assert d <= (2.0 ** -4 if case.path.startswith("fp8") else 0.0)


def poison_outside(case, lo, hi):
    """NaN codes on every stored key outside [lo, hi): evict (with poison) up to lo, and rewrite the
    keys from hi on (for E4M3FN caches the page holding hi is rewritten whole, keeping the codes and
    scales of its keys below hi)."""
    pair = case.pair
    nan_code = {"bf16": np.uint16(0x7FC0), "fp8": np.uint8(0x7F)}[case.dtype]
    if case.dtype == "bf16":
        n = pair.gpu.end - hi
        nan = np.full((n, H, D), nan_code, np.uint16)
        pair.append(hi, nan, nan)
    else:
        P = case.sp["P"]
        p0 = (hi // P) * P
        kc, vc = pair.ref.gather_codes(p0, pair.gpu.end)
        kc, vc = kc.copy(), vc.copy()
        kc[hi - p0:] = nan_code
        vc[hi - p0:] = nan_code
        pages = [int(pair.ref.table[(t // P) % pair.ref.T]) for t in range(p0, pair.gpu.end, P)]
        ks = np.stack([pair.ref.k_scale[pg] for pg in pages])
        vs = np.stack([pair.ref.v_scale[pg] for pg in pages])
        pair.append(p0, kc, vc, ks, vs)
    pair.evict(lo, poison=True)


@pytest.mark.parametrize("path", PATHS)
def test_nan_outside_windows_never_read(path):
    """NaN codes before every window (evicted with poison) and after it (rewritten), inside the
    windows' first and last key tiles, leave the output and LSE bitwise unchanged: keys outside
    [kv_begin, kv_end) are never used."""
    say("case: NaN outside, path", path)
    case = Case(path, seed=44)
    kb, ke = [405, 408, 408], [6125, 6140, 6140]  # 90 key tiles each: the split schedule still applies
    case.check_plan(Q_OFF, kb, ke)
    o1, l1 = case.attend(Q_OFF, kb, ke)
    poison_outside(case, 405, 6140)
    o2, l2 = case.attend(Q_OFF, kb, ke)
    assert not np.isnan(host_values(o2)).any()
    assert np.array_equal(host_codes(o1), host_codes(o2))
    assert np.array_equal(l1.cpu().numpy(), l2.cpu().numpy())


@pytest.mark.parametrize("path", PATHS)
def test_deterministic_and_paged_equals_contiguous(path):
    """Three runs on a randomly paged cache and one on an identity-table cache holding the same
    keys give bitwise identical outputs and LSE."""
    say("case: determinism + paging, path", path)
    a = Case(path, seed=45)
    T = N_KEYS // SPEC[path]["P"]
    b = Case(path, seed=45, table=np.arange(T))
    outs = [a.attend() for _ in range(3)] + [b.attend()]
    for o, l in outs[1:]:
        assert np.array_equal(host_codes(o), host_codes(outs[0][0]))
        assert np.array_equal(l.cpu().numpy(), outs[0][1].cpu().numpy())


# ----------------------------------------------------------------------------- full-size windows

def full_window_pair(cfg, layer, variant):
    """A paged ring (P 1560, T 21, permuted table) holding a full 32760-key window of the round
    workload, K and Q peaked as `variant` says.  Returns the pair, the query codes and the window."""
    H_, D_, P, L = cfg["H"], cfg["D"], cfg["page_size"], cfg["chunk"]
    table = synth.permuted_table(cfg["workload"], layer, cfg["table_len"])
    pair = Pair(cfg["num_pages"], P, H_, D_, cfg["dtype"], table)
    q = synth.queries(cfg, layer, L, stream=11)
    for c in range(7):
        k, v = synth.chunk_kv(cfg, layer, c)
        if variant == "staircase":
            _, k = synth.staircase(q[:1], k, np.arange(c * L, (c + 1) * L), 0, 1024, 16.0, seed_words=(78, layer))
        if cfg["dtype"] == "fp8":
            kc, ks = synth.quantize_e4m3_pages(k, P)
            vc, vs = synth.quantize_e4m3_pages(v, P)
            pair.append(c * L, kc, vc, ks, vs)
        else:
            pair.append(c * L, synth.bf16_codes(k), synth.bf16_codes(v))
    if variant == "staircase":
        q, _ = synth.staircase(q, np.zeros((1, H_, D_), np.float32), np.zeros(1), 0, 1024, 16.0,
                               seed_words=(78, layer, 1))
    else:
        q = q * np.float32(16.0)
    return pair, synth.bf16_codes(q), 0, 7 * L


@pytest.mark.parametrize("variant", ["staircase", "sharp16"])
def test_peaked_full_window_round_shape(variant):
    """Wan-1.3B round shape (4680 query rows over a 32760-key paged window, 12 heads) on peaked
    scores, the kernel and schedule the forward round runs; 256 sampled rows against the oracle."""
    cfg = synth.WAN_ROUND
    say("case: full window, bf16 round shape,", variant)
    pair, q, kb, ke = full_window_pair(cfg, 5, variant)
    L = cfg["chunk"]
    ws = wf.workspace_for(pair.gpu, "cuda")
    pl = wf.wf_chunk_attn_plan(pair.gpu, [0, L], [kb], [ke], "bf16", ws.numel())
    say("plan:", pl)
    assert pl["kernel"] == "dma_bf16" and pl["schedule"] == "per_tile"
    rows = np.sort(np.random.default_rng(12).choice(L, size=256, replace=False))
    qv = values_of(q, "bf16")
    if variant == "staircase":
        K, _ = pair.ref.gather(kb, ke, heads=[0])
        ev = rescale_events(qv[rows, 0], K[:, 0], kb, ke, "max11")
        say("%d tiles force a rescale" % len(ev))
        assert len(ev) >= 20
    o, lse = pair.attend(dev(q, "bf16"), [0, L], [kb], [ke], workspace=ws)
    ro, rl = pair.reference(qv[rows], [0, len(rows)], [kb], [ke])
    check_bars("bf16", False, host_values(o)[rows], ro, lse.cpu().numpy()[:, rows], rl, "full window " + variant)


def test_peaked_full_window_fp8_14b_shape():
    """14B shape (40 heads, E4M3FN K/V, 32760-key paged window) on staircase scores; 128 sampled
    rows x 6 heads against the oracle."""
    cfg = synth.FP8_14B
    say("case: full window, fp8 14B shape, staircase")
    pair, q, kb, ke = full_window_pair(cfg, 0, "staircase")
    L = cfg["chunk"]
    pl = wf.wf_chunk_attn_plan(pair.gpu, [0, L], [kb], [ke], "bf16", 0)
    assert pl["kernel"] == "dma_fp8"
    heads = [0, 9, 17, 26, 33, 39]
    rows = np.sort(np.random.default_rng(13).choice(L, size=128, replace=False))
    qv = values_of(q, "bf16")
    K, V = pair.ref.gather(kb, ke, heads=heads)
    ev = rescale_events(qv[rows, heads[0]], K[:, 0], kb, ke, "max")
    say("%d tiles force a rescale" % len(ev))
    assert len(ev) >= 20
    o, lse = pair.attend(dev(q, "bf16"), [0, L], [kb], [ke], workspace=None)
    qh = qv[rows][:, heads]
    ro, rl = pair.reference(qh, [0, len(rows)], [kb], [ke], heads=heads)
    got = host_values(o)[rows][:, heads]
    check_bars("fp8", False, got, ro, lse.cpu().numpy()[heads][:, rows], rl, "full window fp8", qh, K, V,
               ([0, len(rows)], [kb], [ke], kb))
