"""GPU parity of qmoe_grouped (route, grouped gate/up + SwiGLU, grouped down,
weighted combine) against the CPU oracle, through the C ABI.

Checked stage by stage, as the oracle's contract rounds (h is bf16):
  * h (SwiGLU output) against the oracle's within the propagated bound
    |dh| <= |u| silu'max 2e-3 mag_g + |silu(g)| 2e-3 mag_u + half a bf16 ulp;
  * y against the oracle run on the GPU's own h, within 2e-3 * sum_k |w_k| mag(d_k)
    (plus half a bf16 ulp when y is bf16)."""

import numpy as np
import pytest
import torch

import oracle
from synth import formats as F
from synth import quant, routing

pytestmark = pytest.mark.gpu
TOL = 2e-3
SILU_SLOPE_MAX = 1.1  # |d silu / dg| <= 1.0998


def _q():
    import gemm_dequant_gemv_amd as q
    return q


def _dev_bf16(bits):
    return torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).cuda()


def make_case(fmt_gu, fmt_dn, E, S, H, I, T, topk, tag):
    gu = quant.synthetic_weight(fmt_gu, 2 * I, H, batch=E + S, name=f"{tag}/gu")
    dn = quant.synthetic_weight(fmt_dn, H, I, batch=E + S, name=f"{tag}/dn")
    x = quant.synthetic_bf16(T, H, name=f"{tag}/x")
    ids, w = routing.random_routing(T, E, topk, name=f"{tag}/r")
    return gu, dn, x, ids, w


def _u32(ws, off, count):
    return ws[off:off + 4 * count].view(torch.int32).cpu().numpy().view(np.uint32).astype(np.int64)


def run_gpu(q, gu, dn, x, ids, w, E, S, shared_w=None, y_dtype=torch.float32, wdev=None):
    """Run the layer; return y (float64) and the workspace's intermediates."""
    T, topk = ids.shape
    gud, dnd = wdev if wdev is not None else (q.Weight.from_host(gu), q.Weight.from_host(dn))
    L = q.moe_workspace_layout(gud, dnd, E, S, T, topk)
    assert L["bytes"] == q.moe_workspace_size(gud, dnd, E, S, T, topk)
    ws = torch.empty(L["bytes"], dtype=torch.uint8, device="cuda")
    sw = None if shared_w is None else torch.from_numpy(shared_w).cuda()
    y = q.moe(gud, dnd, _dev_bf16(x), torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda(),
              E, S, shared_w=sw, y_dtype=y_dtype, workspace=ws)
    torch.cuda.synchronize()
    I = gu.n // 2
    rows = T * (topk + S)
    r = {"slot_rows": bool(L["slot_rows"]), "tile_rows": int(L["tile_rows"])}
    r["err"] = int(_u32(ws, L["scalars"], 3)[2])
    if r["slot_rows"]:
        # decode form: h / d row s is token slot s, shared slots after the routed
        routed = T * topk
        valid = (ids >= 0) & (ids < E)
        r["row_of_slot"] = np.where(valid, np.arange(routed).reshape(T, topk), 0xFFFFFFFF)
        r["row_of_shared"] = routed + np.arange(S * T)
    else:
        r["counts"] = _u32(ws, L["counts"], E + S)
        r["offsets"] = _u32(ws, L["offsets"], E + S + 1)
        r["row_of_slot"] = _u32(ws, L["row_of_slot"], T * topk).reshape(T, topk)
        r["row_of_shared"] = _u32(ws, L["row_of_shared"], S * T)
        r["token_of_row"] = _u32(ws, L["token_of_row"], rows)
        r["slot_of_row"] = _u32(ws, L["slot_of_row"], rows)
        n_active, n_tiles, _ = _u32(ws, L["scalars"], 3)
        r["active"] = _u32(ws, L["active"], n_active)
        r["tiles"] = _u32(ws, L["tiles"], 3 * n_tiles).reshape(-1, 3)
    r["h"] = ws[L["h"]:L["h"] + rows * I * 2].view(torch.int16).cpu().numpy().view(np.uint16).reshape(rows, I)
    H = dn.n
    r["d"] = ws[L["d"]:L["d"] + rows * H * 4].view(torch.float32).cpu().numpy().reshape(rows, H)
    if y.dtype == torch.bfloat16:
        yh = oracle.bf16(y.view(torch.int16).cpu().numpy().view(np.uint16))
    else:
        yh = y.cpu().numpy().astype(np.float64)
    return yh, r


def check_grouping(r, ids, E, S):
    """Bit-exact on what the grouping fixes (counts, offsets, active experts,
    tile table, error flag); valid on what it leaves open (the order of a
    group's rows): every slot lands inside its expert's rows, once."""
    # the library's routing-tile height (its grouped GEMMs' activation tile) is
    # part of the layout it reports; the tiles themselves must match exactly
    assert r["tile_rows"] in (32, 64, 128, 192, 256)
    g = oracle.moe_grouping(ids, E, S, tile_rows=r["tile_rows"])
    T, topk = ids.shape
    assert r["err"] == g["err"]
    if r["slot_rows"]:  # the decode form builds no grouping tables
        return
    assert np.array_equal(r["counts"], g["counts"])
    assert np.array_equal(r["offsets"], g["offsets"])
    assert np.array_equal(r["active"], g["active"])
    assert np.array_equal(r["tiles"], g["tiles"])
    assert r["err"] == g["err"]
    ros = r["row_of_slot"]
    assert (ros[~g["valid"]] == 0xFFFFFFFF).all()
    e = ids[g["valid"]].astype(np.int64)
    rv = ros[g["valid"]]
    assert ((g["offsets"][e] <= rv) & (rv < g["offsets"][e + 1])).all()
    tok = np.nonzero(g["valid"])[0]
    assert np.array_equal(r["token_of_row"][rv], tok)
    rs = r["row_of_shared"].reshape(S, T)
    for s in range(S):
        assert ((g["offsets"][E + s] <= rs[s]) & (rs[s] < g["offsets"][E + s + 1])).all()
        assert np.array_equal(r["token_of_row"][rs[s]], np.arange(T))
    every = np.concatenate([rv, rs.ravel()])
    assert len(np.unique(every)) == len(every) == g["offsets"][-1]
    # each grouped row knows its token slot (the row of d it writes)
    slots = np.arange(T * topk).reshape(T, topk)[g["valid"]]
    assert np.array_equal(r["slot_of_row"][rv], slots)
    for s in range(S):
        assert np.array_equal(r["slot_of_row"][rs[s]], T * topk + s * T + np.arange(T))


def gpu_h_dict(r, T, topk, S, tokens):
    h, ros, rsh = r["h"], r["row_of_slot"], r["row_of_shared"]
    d = {}
    for t in tokens:
        for j in range(topk):
            if ros[t, j] != 0xFFFFFFFF:
                d[(t, j)] = h[ros[t, j]]
        for s in range(S):
            d[(t, topk + s)] = h[rsh[s * T + t]]
    return d


def check_h(gu, x, ids, E, S, hd, tokens):
    """GPU h against the oracle's SwiGLU of exact gate/up outputs."""
    I = gu.n // 2
    cache = {}
    for t in tokens:
        experts = [(int(ids[t, j]), j) for j in range(ids.shape[1])]
        experts += [(E + s, ids.shape[1] + s) for s in range(S)]
        xt = oracle.bf16(x[t])
        for e, slot in experts:
            if e not in cache:
                cache[e] = oracle.dequant(gu, e)
            wgu = cache[e]
            gu_v = wgu @ xt
            mag = np.abs(wgu) @ np.abs(xt)
            g, u, mg, mu = gu_v[:I], gu_v[I:], mag[:I], mag[I:]
            sg = oracle.silu(g)
            href = sg * u
            bound = (np.abs(u) * SILU_SLOPE_MAX * TOL * mg + np.abs(sg) * TOL * mu
                     + 2 * oracle.bf16_half_ulp(href) + 1e-30)
            got = oracle.bf16(hd[(t, slot)])
            bad = np.abs(got - href) > bound
            assert not bad.any(), f"token {t} expert {e}: {bad.sum()} h values out of bound"


def check_y(gu, dn, x, ids, w, E, S, yh, hd, tokens, shared_w=None, bf16_out=False):
    yref, mag, _ = oracle.moe(gu, dn, x, ids, w, E, S, shared_w=shared_w, tokens=tokens,
                              h_given=hd)
    got = yh[np.asarray(tokens)]
    ok = (oracle.within_tolerance_bf16(got, yref, mag, TOL) if bf16_out
          else oracle.within_tolerance(got, yref, mag, TOL))
    assert ok.all(), (f"{(~ok).sum()} of {ok.size} outside; worst "
                      f"{np.max(np.abs(got - yref) / mag):.3e} of mag")


SMALL = dict(E=16, S=1, H=256, I=128, topk=4)


def decode_form(T, topk, S):
    """Whether a call takes the decode form (one grouped GEMV per projection
    over the token slots), as the header states for activations that fit in
    LDS (every case here)."""
    return T <= 16 and T * (topk + S) <= 128


@pytest.mark.parametrize("T", [1, 4, 8, 16, 17, 37, 100, 200, 300])
@pytest.mark.parametrize("fmts", [(F.NVFP4, F.NVFP4), (F.AFFINE4_G64, F.MXFP4), (F.Q6_K, F.AFFINE4_G64)])
def test_moe_parity_small(T, fmts):
    q = _q()
    c = SMALL
    gu, dn, x, ids, w = make_case(*fmts, c["E"], c["S"], c["H"], c["I"], T, c["topk"],
                                  f"moe{fmts}{T}")
    yh, r = run_gpu(q, gu, dn, x, ids, w, c["E"], c["S"])
    assert r["slot_rows"] == decode_form(T, c["topk"], c["S"])
    check_grouping(r, ids, c["E"], c["S"])
    tokens = list(range(T)) if T <= 40 else list(range(0, T, 7))
    hd = gpu_h_dict(r, T, c["topk"], c["S"], tokens)
    check_h(gu, x, ids, c["E"], c["S"], hd, tokens)
    check_y(gu, dn, x, ids, w, c["E"], c["S"], yh, hd, tokens)


@pytest.mark.parametrize("T,rows", [(17, 32), (200, 64), (300, 128), (600, 192), (800, 256)])
def test_moe_every_tile_height(T, rows):
    """The grouped form at each routing tile height (32 to 256 rows; the
    height follows the mean rows per routed expert), so that every tile
    configuration of the gate/up and down GEMMs, and their mapping of
    workgroups to (tile, column block), meets the oracle stage by stage."""
    q = _q()
    c = SMALL
    gu, dn, x, ids, w = make_case(F.NVFP4, F.AFFINE4_G64, c["E"], c["S"], c["H"], c["I"], T,
                                  c["topk"], f"moeth{T}")
    yh, r = run_gpu(q, gu, dn, x, ids, w, c["E"], c["S"])
    assert not r["slot_rows"] and r["tile_rows"] == rows
    check_grouping(r, ids, c["E"], c["S"])
    tokens = list(range(0, T, 5)) + [T - 1]
    hd = gpu_h_dict(r, T, c["topk"], c["S"], tokens)
    check_h(gu, x, ids, c["E"], c["S"], hd, tokens)
    check_y(gu, dn, x, ids, w, c["E"], c["S"], yh, hd, tokens)


def test_moe_no_shared_weighted_shared_and_bf16_out():
    q = _q()
    E, H, I, T, topk = 8, 256, 128, 50, 2
    gu, dn, x, ids, w = make_case(F.NVFP4, F.NVFP4, E, 0, H, I, T, topk, "moens")
    yh, r = run_gpu(q, gu, dn, x, ids, w, E, 0, y_dtype=torch.bfloat16)
    tokens = list(range(T))
    hd = gpu_h_dict(r, T, topk, 0, tokens)
    check_y(gu, dn, x, ids, w, E, 0, yh, hd, tokens, bf16_out=True)
    # one shared expert with a per-token weight
    gu, dn, x, ids, w = make_case(F.NVFP4, F.NVFP4, E, 1, H, I, T, topk, "moesw")
    sw = (np.arange(T, dtype=np.float32) / T - 0.3).astype(np.float32)
    yh, r = run_gpu(q, gu, dn, x, ids, w, E, 1, shared_w=sw)
    hd = gpu_h_dict(r, T, topk, 1, tokens)
    check_y(gu, dn, x, ids, w, E, 1, yh, hd, tokens, shared_w=sw)


def test_moe_single_expert_equals_dense_chain():
    """E = 1, topk = 1, weight 1, no shared expert: the layer is down(SwiGLU(gate_up x))."""
    q = _q()
    H, I, T = 512, 256, 130
    gu, dn, x, _, _ = make_case(F.AFFINE4_G64, F.NVFP4, 1, 0, H, I, T, 1, "moe1")
    ids = np.zeros((T, 1), np.int32)
    w = np.ones((T, 1), np.float32)
    yh, r = run_gpu(q, gu, dn, x, ids, w, 1, 0)
    tokens = list(range(T))
    hd = gpu_h_dict(r, T, 1, 0, tokens)
    # the oracle's down stage on the GPU's h is exactly two dense products
    hb = np.stack([hd[(t, 0)] for t in tokens])
    yref, mag = oracle.gemv(dn, hb)
    assert oracle.within_tolerance(yh, yref, mag, TOL).all()
    check_h(gu, x, ids, 1, 0, hd, tokens)


@pytest.mark.parametrize("T", [3, 6])
def test_moe_invalid_expert_ids_contribute_nothing(T):
    q = _q()
    E, H, I, topk = 8, 256, 128, 3
    gu, dn, x, ids, w = make_case(F.NVFP4, F.NVFP4, E, 1, H, I, T, topk, f"moebad{T}")
    ids = ids.copy()
    bad = [(0, 1), (T - 1, 0)]
    ids[bad[0]] = E + 5
    ids[bad[1]] = -1
    yh, r = run_gpu(q, gu, dn, x, ids, w, E, 1)
    assert all(r["row_of_slot"][b] == 0xFFFFFFFF for b in bad)
    assert r["err"] == 1
    check_grouping(r, ids, E, 1)
    w2 = w.copy()
    for b in bad:
        w2[b] = 0.0
    ids2 = np.where(ids < 0, 0, np.where(ids >= E, 0, ids)).astype(np.int32)
    tokens = list(range(T))
    hd = gpu_h_dict(r, T, topk, 1, tokens)
    # the dropped slots get a placeholder h (their weight is zero in the reference)
    for b in bad:
        hd[b] = np.zeros(I, np.uint16)
    check_y(gu, dn, x, ids2, w2, E, 1, yh, hd, tokens)


@pytest.mark.parametrize("T", [1638, 1700, 4000, 14000])
def test_moe_many_slots_route(T):
    """Calls with more than 16384 routed slots group them over many workgroups
    (per-workgroup counts, one scan, placement); 1638 x 10 slots is the largest
    call of the one-workgroup route, and 14000 x 10 slots take 69 workgroups
    (the scan reads their counts in two batches of up to 64).  Dropped ids sit in the first, a middle
    and the last (ragged) chunk; the tables must still match the oracle's."""
    q = _q()
    E, S, H, I, topk = 64, 1, 256, 128, 10
    gu, dn, x, ids, w = make_case(F.NVFP4, F.AFFINE4_G64, E, S, H, I, T, topk, f"moemany{T}")
    ids = ids.copy()
    bad = [(0, 3), (T // 2, 0), (T - 1, topk - 1)]
    ids[bad[0]] = E
    ids[bad[1]] = -7
    ids[bad[2]] = 1 << 20
    yh, r = run_gpu(q, gu, dn, x, ids, w, E, S)
    assert not r["slot_rows"]
    assert all(r["row_of_slot"][b] == 0xFFFFFFFF for b in bad)
    assert r["err"] == 1
    check_grouping(r, ids, E, S)
    w2 = w.copy()
    for b in bad:
        w2[b] = 0.0
    ids2 = np.where((ids < 0) | (ids >= E), 0, ids).astype(np.int32)
    tokens = [0, 1, T // 2, T // 2 + 1, T - 2, T - 1]
    hd = gpu_h_dict(r, T, topk, S, tokens)
    clean = [1, T // 2 + 1, T - 2]
    check_h(gu, x, ids, E, S, {k: v for k, v in hd.items() if k[0] in clean}, clean)
    for b in bad:
        hd[b] = np.zeros(I, np.uint16)
    check_y(gu, dn, x, ids2, w2, E, S, yh, hd, tokens)


def _fma_f32(a, b, c):
    """fma(a, b, c) in float32: the exact a * b + c rounded once to nearest
    even (exact rational arithmetic, then the nearest float32)."""
    from fractions import Fraction
    exact = Fraction(float(a)) * Fraction(float(b)) + Fraction(float(c))
    f = np.float32(float(exact))
    best = None
    for cand in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        err = abs(Fraction(float(cand)) - exact)
        key = (err, int(np.array(cand, np.float32).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, cand)
    return np.float32(best[1])


@pytest.mark.parametrize("T", [1, 4, 8])
@pytest.mark.parametrize("y_dtype", [torch.float32, torch.bfloat16])
def test_moe_decode_combine_is_the_fixed_fma_chain(T, y_dtype):
    """The decode form runs the combine inside its down launch: each output is
    the float32 chain acc = fma(w_j, d_j, acc) over the token's terms (routed
    slots in list order, skipping dropped ids, then the shared experts), from
    0, the chain the grouped form's combine kernel runs.  Checked bit for bit
    against that chain evaluated exactly on the d rows the launch wrote."""
    q = _q()
    E, S, H, I, topk = 12, 2, 256, 128, 4
    gu, dn, x, ids, w = make_case(F.NVFP4, F.AFFINE4_G64, E, S, H, I, T, topk, f"moefc{T}")
    ids = ids.copy()
    ids[0, 2] = E + 3  # a dropped slot
    sw = np.linspace(0.5, 1.5, T).astype(np.float32)
    yh, r = run_gpu(q, gu, dn, x, ids, w, E, S, shared_w=sw, y_dtype=y_dtype)
    assert r["slot_rows"]
    d = r["d"]
    for t in range(T):
        terms = [(t * topk + j, w[t, j]) for j in range(topk) if 0 <= ids[t, j] < E]
        terms += [(T * topk + s * T + t, sw[t]) for s in range(S)]
        acc = np.zeros(H, np.float32)
        for row, wt in terms:
            acc = np.array([_fma_f32(wt, d[row, n], acc[n]) for n in range(H)], np.float32)
        if y_dtype == torch.bfloat16:
            want = oracle.bf16(oracle.bf16_round(acc))
        else:
            want = acc.astype(np.float64)
        assert np.array_equal(yh[t], want), f"token {t}"


@pytest.mark.parametrize("T", [4, 300])
def test_moe_deterministic(T):
    q = _q()
    E, H, I, topk = 16, 256, 128, 4
    gu, dn, x, ids, w = make_case(F.NVFP4, F.NVFP4, E, 1, H, I, T, topk, f"moedet{T}")
    wdev = (q.Weight.from_host(gu), q.Weight.from_host(dn))
    ys = [run_gpu(q, gu, dn, x, ids, w, E, 1, wdev=wdev)[0] for _ in range(3)]
    for y in ys[1:]:
        assert np.array_equal(ys[0], y)


# The full layer: 512 routed experts plus one shared expert, hidden 2048,
# expert intermediate 512, NVFP4, top-10 of softmaxed N(0, 1) logits.
FULL = dict(E=512, S=1, H=2048, I=512, topk=10)


@pytest.fixture(scope="module")
def full_layer():
    q = _q()
    c = FULL
    gu = quant.synthetic_weight(F.NVFP4, 2 * c["I"], c["H"], batch=c["E"] + c["S"],
                                name="moe_full/gate_up")
    dn = quant.synthetic_weight(F.NVFP4, c["H"], c["I"], batch=c["E"] + c["S"],
                                name="moe_full/down")
    return gu, dn, (q.Weight.from_host(gu), q.Weight.from_host(dn))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("T,y_dtype", [(4, torch.float32), (8192, torch.bfloat16)])
def test_moe_full_layer(full_layer, T, y_dtype):
    q = _q()
    c = FULL
    gu, dn, wdev = full_layer
    x = quant.synthetic_bf16(T, c["H"], name=f"moe_full/x{T}")
    ids, w = routing.random_routing(T, c["E"], c["topk"], name=f"moe_full/r{T}")
    print(f"moe full layer T={T}", flush=True)
    yh, r = run_gpu(q, gu, dn, x, ids, w, c["E"], c["S"], y_dtype=y_dtype, wdev=wdev)
    assert r["slot_rows"] == decode_form(T, c["topk"], c["S"])
    check_grouping(r, ids, c["E"], c["S"])
    tokens = list(range(T)) if T <= 16 else [0, 1, 2047, 4096, 6000, T - 1]
    hd = gpu_h_dict(r, T, c["topk"], c["S"], tokens)
    check_h(gu, x, ids, c["E"], c["S"], hd, tokens)
    check_y(gu, dn, x, ids, w, c["E"], c["S"], yh, hd, tokens,
            bf16_out=y_dtype == torch.bfloat16)
    assert np.isfinite(yh).all()


# ------------------------------------------------------------ router

def _router_case(T, E, k, kind):
    if kind == "normal":
        lg = routing.router_logits(T, E, name=f"rt{T}/{E}")
    elif kind == "ties":  # few distinct values: many equal logits per token
        lg = np.floor(routing.router_logits(T, E, name=f"rtt{T}/{E}") * 2.0).astype(np.float32)
    else:  # signed zeros among negative logits
        lg = -np.abs(routing.router_logits(T, E, name=f"rtz{T}/{E}"))
        lg[:, ::3] = 0.0
        lg[:, 1::3] = -0.0
        lg = lg.astype(np.float32)
    return np.ascontiguousarray(lg, dtype=np.float32)


@pytest.mark.parametrize("T,E,k,kind", [(1, 512, 10, "normal"), (4, 512, 10, "normal"),
                                        (37, 512, 10, "normal"), (8192, 512, 10, "normal"),
                                        (5, 64, 1, "normal"), (3, 4096, 64, "normal"),
                                        (7, 100, 7, "normal"), (6, 130, 5, "ties"),
                                        (9, 512, 10, "ties"), (5, 300, 12, "zeros"),
                                        (3, 1, 1, "normal"), (4, 65, 64, "normal"),
                                        (2, 4096, 10, "ties")])
def test_router_parity(T, E, k, kind):
    """Expert ids exactly as the oracle orders them (both sides compare the same
    float32 logits); weights within 2e-6 relative of the float64 softmax."""
    q = _q()
    lg = _router_case(T, E, k, kind)
    ids, w = q.moe_router(torch.from_numpy(lg).cuda(), k)
    torch.cuda.synchronize()
    rid, rw = oracle.router(lg, k)
    assert np.array_equal(ids.cpu().numpy(), rid)
    wg = w.cpu().numpy().astype(np.float64)
    assert (np.abs(wg - rw) <= 2e-6 * rw + 1e-12).all()
    # repeatable bits
    ids2, w2 = q.moe_router(torch.from_numpy(lg).cuda(), k)
    assert torch.equal(ids, ids2) and torch.equal(w, w2)


@pytest.mark.parametrize("T", [1, 4, 16, 100])
def test_moe_from_logits_is_router_then_layer(T):
    """qmoe_grouped_logits gives the bits of qmoe_router followed by
    qmoe_grouped: the decode form (up to 16 tokens here) with the router folded
    into its first launch, the grouped form (100 tokens) with the router as
    its own launch."""
    q = _q()
    c = SMALL
    gu, dn, x, _, _ = make_case(F.NVFP4, F.AFFINE4_G64, c["E"], c["S"], c["H"], c["I"], T,
                                c["topk"], f"moelg{T}")
    lg = torch.from_numpy(routing.router_logits(T, c["E"], name=f"moelg{T}/r")).cuda()
    gud, dnd = q.Weight.from_host(gu), q.Weight.from_host(dn)
    xd = _dev_bf16(x)
    y1, ids1, w1 = q.moe_from_logits(gud, dnd, xd, lg, c["topk"], c["E"], c["S"])
    ids2, w2 = q.moe_router(lg, c["topk"])
    y2 = q.moe(gud, dnd, xd, ids2, w2, c["E"], c["S"])
    torch.cuda.synchronize()
    assert torch.equal(ids1, ids2) and torch.equal(w1, w2)
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))
    rid, _ = oracle.router(lg.cpu().numpy(), c["topk"])
    assert np.array_equal(ids1.cpu().numpy(), rid)


def test_router_argument_errors():
    q = _q()
    lg = torch.zeros((2, 8), dtype=torch.float32, device="cuda")
    with pytest.raises(q.QmmError):
        q.moe_router(lg, 9)  # topk > experts
    with pytest.raises(q.QmmError):
        q.moe_router(lg, 0)


def test_moe_from_logits_full_layer_decode(full_layer):
    """The 512-expert layer at 4 tokens from router logits (router folded into
    the first launch) against qmoe_router + qmoe_grouped, bit for bit, and the
    routing against the oracle's."""
    q = _q()
    c = FULL
    gu, dn, wdev = full_layer
    T = 4
    x = _dev_bf16(quant.synthetic_bf16(T, c["H"], name="moe_full/xlg"))
    lg = torch.from_numpy(routing.router_logits(T, c["E"], name="moe_full/lg")).cuda()
    y1, ids1, w1 = q.moe_from_logits(wdev[0], wdev[1], x, lg, c["topk"], c["E"], c["S"])
    ids2, w2 = q.moe_router(lg, c["topk"])
    y2 = q.moe(wdev[0], wdev[1], x, ids2, w2, c["E"], c["S"])
    torch.cuda.synchronize()
    assert torch.equal(ids1, ids2) and torch.equal(w1, w2)
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))
    rid, rw = oracle.router(lg.cpu().numpy(), c["topk"])
    assert np.array_equal(ids1.cpu().numpy(), rid)
    assert (np.abs(w1.cpu().numpy() - rw) <= 2e-6 * rw + 1e-12).all()
