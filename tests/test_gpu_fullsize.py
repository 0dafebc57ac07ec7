"""GPU parity at the full prefill-shaped workloads (T4604 and the Zipf-skewed
T16384, H7168 I2048 E256 top-8), stratified so that every token tile of every
used expert is compared with the oracle, on both expert paths:

* per (token, slot) pair, through the oracle's per-pair entry: the requantised
  SwiGLU output h (bytes, in sorted order) and the down projection O.  Rows
  are chosen per 192-row token tile of each expert (the prefill GEMM's tile
  height): one row per tile at a rotating 16-row sub-tile index and position
  in it (so every sub-tile index 0-11 and every row-in-sub-tile 0-15 is hit),
  the last row of each expert (the ragged tile), and the rows on both sides
  of each tile boundary for the first and last tiles of multi-tile experts.
  Every work item of the persistent GEMMs (a token tile times a feature tile)
  holds at least one compared row, whatever the items' XCD partition;
* the down GEMM isolated: O of the GPU's own h bytes against the oracle's down
  projection of those bytes, to bf16 rounding;
* the two expert paths (weight streaming and the MFMA-tiled GEMMs) on every
  token of the layer.

Also: the W2 identity probe's negative controls through the GPU (a W2 with
rows or K columns permuted before the prepack must fail the probe, while the
GPU still computes the permuted layer faithfully), the prepacked layout read
back bit for bit at the full weight shape, and the device MXFP8 quantiser on
an adversarial table of bf16 blocks."""
import time

import numpy as np
import pytest
import torch

import fp4_routed_expert_amd as moe
import oracle
import synth
from gpu_cases import Case, check_y, get_case, log, sample_tokens, to_dev, unpack_layout

pytestmark = pytest.mark.gpu

PATHS = {"decode": moe.MOE_FLAG_FORCE_DECODE, "prefill": moe.MOE_FLAG_FORCE_PREFILL}
TILE = 192


def stratified_rows(offsets: np.ndarray, edge_tiles: int = 4) -> np.ndarray:
    rows = []
    n = 0
    for e in range(offsets.size - 1):
        o0, o1 = int(offsets[e]), int(offsets[e + 1])
        if o1 == o0:
            continue
        tiles = list(range(o0, o1, TILE))
        for i, m0 in enumerate(tiles):
            r = min(o1 - m0, TILE)
            rows.append(m0 + min(r - 1, 16 * (n % 12) + (7 * n + 3) % 16))
            n += 1
            if i > 0 and (i <= edge_tiles or i >= len(tiles) - edge_tiles):
                rows += [m0 - 1, m0]               # rows 191 and 0 of neighbouring tiles
        rows.append(o1 - 1)                         # the expert's last row (ragged tile)
    return np.unique(np.array(rows, dtype=np.int64))


_pairs_cache: dict = {}


def _oracle_pairs(c, name):
    """Oracle per-pair h and O for the stratified rows (cached per workload)."""
    if name not in _pairs_cache:
        _pairs_cache.clear()
        rows = stratified_rows(c.offsets)
        pairs = c.sorted_pair[rows]
        t0 = time.time()
        ex, h, hq, hs, O = oracle.layer_pairs(c.inp, pairs)
        log(f"[{name}] oracle: {rows.size} pairs in {time.time() - t0:.1f} s")
        _pairs_cache[name] = (rows, pairs, ex, hq, hs, O)
    return _pairs_cache[name]


def _stages(c, flags):
    sh = c.sh
    ids, gates = moe.route_topk(c.logits, sh.k)
    counts, offsets, sp, pp = moe.sort_permute(ids, sh.E)
    xq, xs = moe.quant_act_mxfp8(c.x)
    hq, hs = moe.expert_up(c.pw, xq, xs, offsets, sp, sh.T, sh.k, flags)
    O = moe.expert_down(c.pw, hq, hs, offsets, sh.T, sh.k, flags)
    torch.cuda.synchronize()
    return hq, hs, O


@pytest.mark.parametrize("path", ["prefill", "decode"])
@pytest.mark.parametrize("name", ["c3", "c4"])
def test_stratified_pairs_every_tile(name, path, dev):
    c = get_case(name, dev)
    sh = c.sh
    rows, pairs, ex, hq_ref, hs_ref, O_ref = _oracle_pairs(c, name)
    log(f"[{name}/{path}] {rows.size} stratified rows over {int((c.counts > 0).sum())} used experts")
    hq, hs, O = _stages(c, PATHS[path])
    # the expert of each sorted row is the one whose segment holds it
    assert np.array_equal(ex, np.searchsorted(c.offsets, rows, side="right") - 1)
    idx = torch.from_numpy(rows).to(dev)
    hq_g = hq.index_select(0, idx).cpu().numpy()
    hs_g = hs.index_select(0, idx).cpu().numpy()
    O_g = O.index_select(0, idx).float().cpu().numpy().astype(np.float64)
    check_h_bytes(hq_g, hs_g, hq_ref, hs_ref, f"{name}/{path}", c, pairs, ex)
    # O against the oracle's pairs (each side from its own h): the layer tolerance
    check_y(O_g, O_ref, f"{name}/{path}/O")
    row_err = np.abs(O_g - O_ref).max(axis=1) / np.abs(O_ref).max(axis=1)
    log(f"[{name}/{path}] worst row err/ref {row_err.max():.3e} (row {rows[row_err.argmax()]})")
    # the down GEMM isolated: O from the GPU's own h bytes against the exact
    # (float64) product of the same decoded operands, within O's bf16 rounding
    # (8 significant bits: at most 2^-8 relative) plus the bound of an fp32 accumulation of
    # I exact products in any rounding mode, gamma_(I-1) * sum |h_i W_ri| with
    # u = 2^-23
    hd = oracle.decode_mxfp8(hq_g, hs_g)
    I = sh.I
    gam = (I - 1) * 2.0 ** -23 / (1 - (I - 1) * 2.0 ** -23)
    worst, at = 0.0, None
    rel_abs = 0.0
    for e in np.unique(ex):
        sel = np.nonzero(ex == e)[0]
        W2 = oracle.decode_fp4_matrix(c.inp.w2[e], c.inp.s2[e])
        exact = hd[sel] @ W2.T
        absum = np.abs(hd[sel]) @ np.abs(W2).T
        err = np.abs(O_g[sel] - exact)
        lim = 2.0 ** -8 * np.abs(exact) + gam * absum * (1 + 2.0 ** -7)
        over = err / lim
        rel_abs = max(rel_abs, float((np.maximum(err - 2.0 ** -8 * np.abs(exact), 0) / absum).max()))
        if over.max() > worst:
            i, j = np.unravel_index(over.argmax(), over.shape)
            worst = float(over.max())
            at = (int(e), int(rows[sel[i]]), int(j), float(O_g[sel][i, j]), float(exact[i, j]),
                  float(absum[i, j]), float(lim[i, j]))
    log(f"[{name}/{path}] down GEMM: worst |err| / bound {worst:.3f} at (expert, row, col, gpu, exact, "
        f"sum|terms|, bound) = {at}; max (|err| - bf16 rounding) / sum|terms| = {rel_abs:.3e}")
    assert worst <= 1, f"O off its bf16 + fp32 summation bound: {at}"


def _e4m3_codes_between(lo: float, hi: float) -> set:
    """The e4m3 codes (sign included) a value in [lo, hi] can round to."""
    a, b = oracle.e4m3_rne_sat(lo), oracle.e4m3_rne_sat(hi)
    def rank(cd):  # codes in value order: negatives descending, then positives
        return -(cd & 0x7F) if cd & 0x80 else (cd & 0x7F)
    ra, rb = sorted((rank(a), rank(b)))
    out = set()
    for r in range(ra, rb + 1):
        out.add(r if r > 0 else (0x80 | -r) if r < 0 else 0)
    if ra <= 0 <= rb:
        out |= {0x00, 0x80}
    return out


def check_h_bytes(hq_g, hs_g, hq_r, hs_r, what, c, pairs, ex):
    """h is requantised from fp32 sums that the GPU and the oracle take in
    different orders, so a code may land on the other side of a rounding
    boundary; the codes are then not unique, and the check is that each is
    valid.  Scales must be equal (a scale flip needs an amax crossing 2^n;
    none occurs on these workloads).  Where the codes differ, the GPU's code
    must be one that the exact h can round to once its fp32 uncertainty is
    allowed: G and U are sums of H exact products, each within gamma_(H-1) *
    sum |x_h W_ih| of its exact value (u = 2^-23, any rounding mode), which
    SwiGLU carries to h through |dh/dG| <= 1.1 |U| and |dh/dU| = |silu(G)|,
    plus 8 fp32 ulps of h for the exp and reciprocal.  The exact G and U come
    from float64 dot products of the decoded row of x and the decoded weight
    rows.  Differing codes must also be rare."""
    sg, sr = hs_g.astype(np.int32), hs_r.astype(np.int32)
    assert np.array_equal(sg, sr), (what, "h scales differ", np.argwhere(sg != sr)[:5].tolist())
    diff = hq_g != hq_r
    rate = diff.mean()
    log(f"[{what}] h codes differing {rate:.2e} ({int(diff.sum())} codes)")
    assert rate <= 1e-3, f"{what}: h code flips {rate}"
    sh = c.sh
    H = sh.H
    gam = (H - 1) * 2.0 ** -23 / (1 - (H - 1) * 2.0 ** -23)
    steps = 0
    for n, i in np.argwhere(diff):
        t, e = int(pairs[n]) // sh.k, int(ex[n])
        xd = oracle.decode_mxfp8(c.xq[t:t + 1], c.xs[t:t + 1])[0]
        w1 = oracle.decode_fp4_matrix(c.inp.w1[e, i:i + 1], c.inp.s1[e, i:i + 1])[0]
        w3 = oracle.decode_fp4_matrix(c.inp.w3[e, i:i + 1], c.inp.s3[e, i:i + 1])[0]
        G, U = float(xd @ w1), float(xd @ w3)
        dG, dU = gam * float(np.abs(xd) @ np.abs(w1)), gam * float(np.abs(xd) @ np.abs(w3))
        silu = G / (1 + np.exp(-G))
        h = silu * U
        dh = 1.1 * abs(U) * dG + (abs(silu) + 1.1 * dG) * dU + 8 * 2.0 ** -24 * abs(h)
        mul = 2.0 ** (127 - int(sg[n, i // 32]))
        ok = _e4m3_codes_between((h - dh) * mul, (h + dh) * mul)
        assert int(hq_g[n, i]) in ok, (f"{what}: h code {hq_g[n, i]:#x} at pair {int(pairs[n])} col {int(i)} "
                                       f"is not a rounding of h = {h!r} +- {dh!r} (valid {sorted(ok)})")
        assert int(hq_r[n, i]) in ok, f"{what}: the oracle's h code at pair {int(pairs[n])} col {int(i)}"
        steps = max(steps, abs((int(hq_g[n, i]) & 0x7F) - (int(hq_r[n, i]) & 0x7F)))
    log(f"[{what}] every differing h code is a valid rounding (largest code distance {steps})")


@pytest.mark.parametrize("name", ["c3", "c4"])
def test_paths_agree_on_every_token(name, dev):
    c = get_case(name, dev)
    log(f"[{name}] both paths, all {c.sh.T} tokens")
    y_d = moe.moe_layer(c.pw, c.x, c.logits, c.sh.k, flags=PATHS["decode"])
    y_p = moe.moe_layer(c.pw, c.x, c.logits, c.sh.k, flags=PATHS["prefill"])
    torch.cuda.synchronize()
    yd, yp = y_d.cpu().numpy(), y_p.cpu().numpy()
    check_y(yp, yd, f"{name}/prefill-vs-decode")
    per_tok = np.abs(yp.astype(np.float64) - yd).max(axis=1) / np.abs(yd).max()
    log(f"[{name}] worst token {int(per_tok.argmax())}: {per_tok.max():.3e}")
    assert per_tok.max() <= 1e-2
    toks = sample_tokens(c.sh.T, 6, seed=11)
    check_y(yp[toks], oracle.layer_tokens(c.inp, toks), f"{name}/prefill/oracle")


def _probe_closed_form(inp, toks, hq, hs):
    sh = inp.shape
    ids, gates = oracle.route(inp.logits, sh.k)
    hd = oracle.decode_mxfp8(hq, hs)
    r = np.arange(sh.H)
    out = np.zeros((toks.size, sh.H))
    for n, t in enumerate(toks):
        for j in range(sh.k):
            out[n] += float(gates[t, j]) * hd[n * sh.k + j, (r + ids[t, j]) % sh.I]
    return out


@pytest.mark.parametrize("path", ["decode", "prefill"])
@pytest.mark.parametrize("mistake", ["none", "swap_rows", "swap_k_columns"])
def test_w2_probe_negative_controls_on_gpu(mistake, path, dev):
    """The identity W2 probe passes with the canonical W2 and FAILS when W2's
    rows (output features) or K columns were permuted before the prepack --
    the layout mistake the probe exists to catch -- while the GPU still equals
    the oracle's layer for the permuted weights."""
    inp = synth.make_inputs(synth.Shape(T=64, H=512, I=256, E=8, k=2, seed=41), probe_w2=True)
    w2 = inp.w2.copy()
    if mistake == "swap_rows":
        w2[:, [5, 300]] = w2[:, [300, 5]]
    elif mistake == "swap_k_columns":     # K bytes 1 and 70 of every row: columns 2-3 <-> 140-141
        w2[:, :, [1, 70]] = w2[:, :, [70, 1]]
    inp.w2 = np.ascontiguousarray(w2)
    c = Case(inp, dev)
    y = moe.moe_layer(c.pw, c.x, c.logits, c.sh.k, flags=PATHS[path])
    torch.cuda.synchronize()
    toks = np.arange(c.sh.T, dtype=np.int32)
    ref, _, hq, hs = oracle.layer_tokens(c.inp, toks, want_pairs=True)
    check_y(y.cpu().numpy(), ref, f"w2/{mistake}/{path}")
    closed = _probe_closed_form(c.inp, toks, hq, hs)
    err = np.abs(y.cpu().numpy() - closed).max() / np.abs(closed).max()
    log(f"[w2/{mistake}/{path}] probe err/ref {err:.3e}")
    if mistake == "none":
        assert err <= 1e-2
    else:
        assert err > 5e-2, "the probe missed a permuted W2"


def test_prepack_roundtrip_full_weight_shape(dev):
    """The packed tile layout read back into canonical W1/W3/W2 and scales,
    bit for bit, at the H7168 I2048 expert shape (3 experts)."""
    c = get_case(synth.Shape(T=4, H=7168, I=2048, E=3, k=2, seed=31), dev)
    packed = c.pw.buffer.cpu().numpy()
    got = unpack_layout(packed, 3, 7168, 2048)
    for g, name in zip(got, ("w1", "s1", "w3", "s3", "w2", "s2")):
        assert np.array_equal(g, getattr(c.inp, name)), name


def _adversarial_bf16_rows():
    """Rows of 32-element blocks: zero and -0 blocks, bf16 subnormals, maxima at
    2^n - ulp, 2^n, 1.75 * 2^n, elements that scale to 448 / 464 / 480 and to
    e4m3 midpoints, the largest finite bf16, mixed signs and magnitudes."""
    rng = np.random.default_rng(17)
    blocks = [np.zeros(32, np.float32), -np.zeros(32, np.float32)]
    sub = (np.arange(1, 33, dtype=np.uint32)).astype(np.uint16)          # bf16 subnormal bit patterns
    blocks.append(synth.bf16_bits_to_f32(sub))
    blocks.append(-synth.bf16_bits_to_f32(sub[::-1]))
    mixed = synth.bf16_bits_to_f32(sub).copy()
    mixed[::3] = 0
    blocks.append(mixed)
    for n in (-126, -100, -30, -7, -1, 0, 1, 8, 20, 60, 120, 127):
        base = np.float32(2.0 ** n)
        for lead in (base * np.float32(1 - 2.0 ** -8), base, np.float32(1.75) * base):
            if not np.isfinite(lead):
                continue
            b = (rng.normal(0, 0.25, 32) * base).astype(np.float32)
            b[rng.integers(32)] = lead
            blocks.append(b)
        if n > 118:
            continue
        unit = 2.0 ** (n - 8)
        b = np.array([1.5 * 2 ** 8, 448, 464, 480, 500, 504, 17, 18, 19, 36, 38, 272, 288, 304, 240, 248,
                      -448, -464, -480, -17, -19, 2.0 ** -6, 2.0 ** -9, 3 * 2.0 ** -10, -2.0 ** -10,
                      100, 104, 108, 0, 1, -1, 0.5], dtype=np.float64) * unit
        blocks.append(b.astype(np.float32))
    big = np.full(32, 1.0, np.float32)
    big[3] = synth.bf16_bits_to_f32(np.array([0x7F7F], np.uint16))[0]          # largest finite bf16
    blocks.append(big)
    blocks += [(rng.normal(0, 1, 32) * 2.0 ** rng.integers(-40, 40)).astype(np.float32) for _ in range(40)]
    bits = synth.f32_to_bf16_bits(np.concatenate(blocks))
    assert np.isfinite(synth.bf16_bits_to_f32(bits)).all()
    return bits


@pytest.mark.parametrize("K", [32, 96, 7168])
def test_device_mxfp8_adversarial_table(K, dev):
    bits = _adversarial_bf16_rows()
    n = (bits.size // K + 1) * K
    bits = np.resize(bits, n).reshape(-1, K)          # wraps the table to whole rows of K
    x = to_dev(bits.view(np.int16), dev).view(torch.bfloat16)
    q, s = moe.quant_act_mxfp8(x)
    torch.cuda.synchronize()
    wq, ws = oracle.quant_mxfp8_bf16(bits)
    assert np.array_equal(s.cpu().numpy(), ws)
    assert np.array_equal(q.cpu().numpy(), wq)
