"""Pins of the fp64 oracle to facts outside itself.

Each pin_* function takes a loaded oracle library (ctypes handle) and raises
AssertionError when the oracle disagrees with something the mathematics or a
library routine fixes:

  * torch's scaled_dot_product_attention (float64, CPU) with an explicit
    causal/window mask and K/V heads repeated per query group -- the textbook
    routine the method reduces to when there is no sink;
  * the same routine on an augmented problem in which the sink becomes one
    extra, always-visible key whose logit is the sink and whose value is zero;
  * closed forms (q = 0, window 1, sink at +/-80, a hand-derived example);
  * invariants (probabilities sum to one, packed equals separate, causality,
    head-group isolation, window >= length equals full causal, scale
    homogeneity, sequence permutation).

The same functions run against deliberately broken copies of the oracle in
test_oracle_mutants.py, which shows that each plausible mistake fails at least
one of them.  Pages followed: "TokenSpeed-kernel multi-silicon" (aixai.ru),
section "Числа: Gluon на AMD MI355X" (GQA prefill with sinks and sliding
windows); ai-radar.it, section "AMD MI355X: la prova sul campo".
"""
from __future__ import annotations

import math

import numpy as np
import torch
import torch.nn.functional as F

from oracle import oracle
from sinks_ts_mha_amd import workloads
from _util import oracle_args
from sinks_ts_mha_amd.workloads import bf16_bits


def _run(lib, inp):
    return oracle.prefill(*oracle_args(inp), lib=lib)


def _inputs(seqlens, hq, hkv, window=0, sinks=True, seed=0, scale=0.125, head_dim=64):
    wl = workloads.custom(seqlens, hq, hkv, window=window, sinks=sinks, seed=seed,
                          softmax_scale=scale, head_dim=head_dim)
    return workloads.make_inputs(wl)


def _mask(L, window):
    i = torch.arange(L).view(L, 1)
    j = torch.arange(L).view(1, L)
    m = j <= i
    if window > 0:
        m = m & (i - j < window)
    return m


def _sdpa_reference(inp, augment_sink: bool):
    """Per sequence, per query head: SDPA in float64 with an explicit mask."""
    q = inp["q"].to(torch.float64)
    k = inp["k"].to(torch.float64)
    v = inp["v"].to(torch.float64)
    hq, hkv, D = q.shape[1], k.shape[1], q.shape[2]
    G = hq // hkv
    cu = inp["cu_seqlens"].tolist()
    scale = inp["softmax_scale"]
    out = torch.zeros_like(q)
    for b in range(len(cu) - 1):
        s, e = cu[b], cu[b + 1]
        L = e - s
        if L == 0:
            continue
        qb = q[s:e].transpose(0, 1)                                    # [Hq, L, D]
        kb = k[s:e].repeat_interleave(G, dim=1).transpose(0, 1)        # [Hq, L, D]
        vb = v[s:e].repeat_interleave(G, dim=1).transpose(0, 1)
        mask = _mask(L, inp["window"])
        if augment_sink:
            sig = inp["sinks"].to(torch.float64)
            ones = torch.ones(hq, L, 1, dtype=torch.float64)
            qb = torch.cat([qb, ones], dim=2)
            kb = torch.cat([kb, torch.zeros(hq, L, 1, dtype=torch.float64)], dim=2)
            ksink = torch.zeros(hq, 1, D + 1, dtype=torch.float64)
            ksink[:, 0, D] = sig / scale
            kb = torch.cat([kb, ksink], dim=1)
            vb = torch.cat([vb, torch.zeros(hq, 1, D, dtype=torch.float64)], dim=1)
            mask = torch.cat([mask, torch.ones(L, 1, dtype=torch.bool)], dim=1)
        ob = F.scaled_dot_product_attention(qb.contiguous(), kb.contiguous(), vb.contiguous(),
                                            attn_mask=mask, scale=scale)
        out[s:e] = ob.transpose(0, 1)
    return out.numpy()


def _close(got, ref, tol, what):
    d = float(np.max(np.abs(got - ref))) if got.size else 0.0
    assert d <= tol, f"{what}: max |oracle - reference| = {d:.3e} > {tol:.1e}"


NOSINK_CASES = [([1, 7, 33, 64], 4, 2, 0), ([5, 40], 2, 2, 1), ([17, 50], 4, 1, 5),
                ([64], 8, 4, 2), ([30, 3], 4, 4, 100), ([0, 12, 0, 20], 2, 1, 3)]


def pin_sdpa_no_sink(lib):
    for n, (seqlens, hq, hkv, w) in enumerate(NOSINK_CASES):
        inp = _inputs(seqlens, hq, hkv, window=w, sinks=False, seed=10 + n)
        _close(_run(lib, inp), _sdpa_reference(inp, False), 1e-12,
               f"SDPA no-sink case {seqlens} Hq={hq} Hkv={hkv} W={w}")


SINK_CASES = [([1, 9, 48], 4, 2, 0), ([33], 4, 1, 1), ([20, 41], 8, 2, 6), ([64], 2, 2, 64)]


def pin_sdpa_sink_augmented(lib):
    for n, (seqlens, hq, hkv, w) in enumerate(SINK_CASES):
        inp = _inputs(seqlens, hq, hkv, window=w, sinks=True, seed=20 + n)
        # spread the sinks so that some dominate and some are negligible
        inp["sinks"] = inp["sinks"] * 3.0 + torch.linspace(-2.0, 4.0, hq)
        _close(_run(lib, inp), _sdpa_reference(inp, True), 1e-12,
               f"SDPA augmented-sink case {seqlens} Hq={hq} Hkv={hkv} W={w}")


def _visible_count(i, window):
    return min(i + 1, window) if window > 0 else i + 1


def pin_closed_form_q_zero(lib):
    """q = 0: every visible key has logit 0, so out_i = sum_{j in A_i} v_j / (|A_i| + e^sigma)."""
    for n, (seqlens, hq, hkv, w, with_sink) in enumerate(
            [([1, 9, 40], 4, 2, 0, True), ([25, 6], 4, 2, 3, True), ([30], 8, 2, 1, True),
             ([16, 16], 2, 1, 8, False), ([50], 4, 4, 0, False)]):
        inp = _inputs(seqlens, hq, hkv, window=w, sinks=with_sink, seed=30 + n)
        inp["q"] = torch.zeros_like(inp["q"])
        v = inp["v"].to(torch.float64).numpy()
        G = hq // hkv
        cu = inp["cu_seqlens"].tolist()
        ref = np.zeros(inp["q"].shape, dtype=np.float64)
        for b in range(len(cu) - 1):
            s, e = cu[b], cu[b + 1]
            for i in range(e - s):
                cnt = _visible_count(i, w)
                vsum = v[s + i - cnt + 1: s + i + 1].sum(axis=0)      # [Hkv, D]
                for h in range(hq):
                    extra = math.exp(float(inp["sinks"][h])) if with_sink else 0.0
                    ref[s + i, h] = vsum[h // G] / (cnt + extra)
        _close(_run(lib, inp), ref, 1e-12, f"q=0 closed form {seqlens} W={w} sink={with_sink}")


def pin_closed_form_window_one(lib):
    """W = 1: only the diagonal is visible, out_i = v_i e^{z_ii} / (e^{z_ii} + e^sigma)."""
    inp = _inputs([13, 22], 4, 2, window=1, seed=40)
    q = inp["q"].to(torch.float64).numpy()
    k = inp["k"].to(torch.float64).numpy()
    v = inp["v"].to(torch.float64).numpy()
    sig = inp["sinks"].to(torch.float64).numpy()
    G = 2
    ref = np.zeros(q.shape)
    for t in range(q.shape[0]):
        for h in range(4):
            z = inp["softmax_scale"] * float(np.dot(q[t, h], k[t, h // G]))
            ref[t, h] = v[t, h // G] * (1.0 / (1.0 + math.exp(sig[h] - z)))
    _close(_run(lib, inp), ref, 1e-12, "window-1 closed form")


def pin_hand_example(lib):
    """Hand-derived example, D = 64, one sequence of 3 tokens, 2 query heads, 1 KV head.

    q_i = e0 for every i; k_0 = 8 e0, k_1 = 8 e1, k_2 = 0; v_j = (j + 1) e5; scale 1/8,
    so z_i0 = 1 and z_i1 = z_i2 = 0.  Sinks: 0 for head 0 and ln 2 for head 1.
    Column 5 of the output is then a ratio of small sums of e and integers.
    """
    D = 64
    q = torch.zeros(3, 2, D)
    q[:, :, 0] = 1.0
    k = torch.zeros(3, 1, D)
    k[0, 0, 0] = 8.0
    k[1, 0, 1] = 8.0
    v = torch.zeros(3, 1, D)
    for j in range(3):
        v[j, 0, 5] = j + 1.0
    e = math.e
    base = {"q": q.to(torch.bfloat16), "k": k.to(torch.bfloat16), "v": v.to(torch.bfloat16),
            "sinks": torch.tensor([0.0, math.log(2.0)], dtype=torch.float32),
            "cu_seqlens": torch.tensor([0, 3], dtype=torch.int32), "softmax_scale": 0.125}
    es = [1.0, math.exp(float(torch.tensor(math.log(2.0), dtype=torch.float32)))]  # the fp32 sink, widened
    for w in (0, 2):
        inp = dict(base, window=w)
        out = _run(lib, inp)
        for h in range(2):
            if w == 0:
                expect = [e / (e + es[h]), (e + 2) / (e + 1 + es[h]), (e + 5) / (e + 2 + es[h])]
            else:
                expect = [e / (e + es[h]), (e + 2) / (e + 1 + es[h]), 5.0 / (2 + es[h])]
            got = out[:, h, 5]
            assert np.allclose(got, expect, rtol=1e-14, atol=0), \
                f"hand example W={w} head {h}: {got} vs {expect}"
            others = np.delete(out[:, h, :], 5, axis=1)
            assert np.all(others == 0.0), "hand example: columns other than 5 must be 0"


def pin_sink_extremes(lib):
    inp = _inputs([7, 40], 4, 2, window=0, seed=50)
    big = dict(inp, sinks=torch.full((4,), 80.0))
    out = _run(lib, big)
    assert np.max(np.abs(out)) < 1e-20, "sink +80 must absorb essentially all weight"
    small = dict(inp, sinks=torch.full((4,), -80.0))
    none = dict(inp, sinks=None)
    a, b = _run(lib, small), _run(lib, none)
    _close(a, b, 1e-15 * max(1.0, float(np.max(np.abs(b)))), "sink -80 vs no sink")


def pin_probs_sum_to_one(lib):
    inp = _inputs([5, 37], 4, 2, window=9, seed=60)
    args = oracle_args(inp)
    q, k, v = args[0], args[1], args[2]
    vv = inp["v"].to(torch.float64).numpy()
    out = oracle.prefill(*args, lib=lib)
    for row in (0, 4, 5, 6, 20, 41):
        for h in (0, 3):
            probs, p_sink = oracle.row_probs(*args, row=row, head=h, lib=lib)
            total = float(probs.sum()) + p_sink
            assert abs(total - 1.0) <= 1e-12, f"row {row} head {h}: probabilities sum to {total}"
            assert np.all(probs >= 0.0) and p_sink > 0.0
            s = 0 if row < 5 else 5
            i = row - s
            lo = max(0, i - 9 + 1)
            assert np.all(probs[:lo] == 0.0), "keys outside the window must have zero weight"
            assert np.all(probs[lo:] > 0.0)
            recon = probs @ vv[s:s + i + 1, h // 2]
            assert np.allclose(recon, out[row, h], rtol=1e-12, atol=1e-15)
    _ = q, k, v


def pin_window_covering_equals_full(lib):
    inp = _inputs([3, 50, 21], 4, 2, window=0, seed=70)
    full = _run(lib, inp)
    for w in (50, 51, 1 << 20):
        assert np.array_equal(_run(lib, dict(inp, window=w)), full), f"W={w} must equal full causal"


def pin_packed_equals_separate(lib):
    inp = _inputs([9, 1, 30, 0, 17], 4, 2, window=4, seed=80)
    packed = _run(lib, inp)
    cu = inp["cu_seqlens"].tolist()
    for b in range(len(cu) - 1):
        s, e = cu[b], cu[b + 1]
        if e == s:
            continue
        one = dict(inp, q=inp["q"][s:e], k=inp["k"][s:e], v=inp["v"][s:e],
                   cu_seqlens=torch.tensor([0, e - s], dtype=torch.int32))
        assert np.array_equal(_run(lib, one), packed[s:e]), f"sequence {b} differs when packed"


def pin_permute_sequences(lib):
    inp = _inputs([6, 19, 11], 2, 1, window=0, seed=90)
    out = _run(lib, inp)
    cu = inp["cu_seqlens"].tolist()
    order = [2, 0, 1]
    pieces = [slice(cu[b], cu[b + 1]) for b in order]
    lens = [cu[b + 1] - cu[b] for b in order]
    perm = dict(inp, q=torch.cat([inp["q"][p] for p in pieces]),
                k=torch.cat([inp["k"][p] for p in pieces]),
                v=torch.cat([inp["v"][p] for p in pieces]),
                cu_seqlens=torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32))
    got = _run(lib, perm)
    assert np.array_equal(got, np.concatenate([out[p] for p in pieces]))


def pin_causality(lib):
    """Row i of a sequence depends on no token after i and on no other sequence."""
    inp = _inputs([24, 16], 4, 2, window=0, seed=100)
    base = _run(lib, inp)
    cut = 10
    pert = dict(inp)
    for name in ("q", "k", "v"):
        t = inp[name].clone()
        t[cut + 1:24] = -t[cut + 1:24] * 2.0 + 0.5
        pert[name] = t
    got = _run(lib, pert)
    assert np.array_equal(got[:cut + 1], base[:cut + 1]), "future tokens leaked into the past"
    assert np.array_equal(got[24:], base[24:]), "one sequence leaked into another"
    assert not np.array_equal(got[cut + 1:24], base[cut + 1:24])


def pin_head_groups(lib):
    """Query head h reads KV head floor(h / G): perturbing KV head 1 moves heads 2, 3 only."""
    inp = _inputs([31], 4, 2, window=0, seed=110)
    base = _run(lib, inp)
    pert = dict(inp)
    for name in ("k", "v"):
        t = inp[name].clone()
        t[:, 1] = t[:, 1] * -1.5
        pert[name] = t
    got = _run(lib, pert)
    assert np.array_equal(got[:, :2], base[:, :2]), "heads of group 0 changed"
    assert not np.any(np.all(got[:, 2:] == base[:, 2:], axis=(0, 2))), "heads of group 1 did not change"


def pin_scale_homogeneity(lib):
    """scale multiplies q.k: (2 scale, q) and (scale, 2 q) give identical logits."""
    inp = _inputs([12, 29], 4, 2, window=5, seed=120)
    a = _run(lib, dict(inp, softmax_scale=0.25))
    b = _run(lib, dict(inp, q=(inp["q"].float() * 2.0).to(torch.bfloat16)))
    assert np.array_equal(a, b)
    c = _run(lib, inp)
    assert not np.allclose(a, c), "the scale must change the result"


def pin_rows_equal_prefill(lib):
    """The selected-rows routine gives, bit for bit, the rows of the full routine (which
    the pins above tie to the library routine and the closed forms): ragged packs with
    empty sequences, windows 0, 1, 5 and one covering every sequence, sinks on and off,
    rows in shuffled order with repeats, both head widths."""
    seqlens = [0, 7, 1, 0, 33, 64, 65, 0, 130]
    cases = [(w, sk, 64) for w in (0, 1, 5, 200) for sk in (True, False)] + [(5, True, 128), (0, False, 128)]
    for n, (window, sinks, head_dim) in enumerate(cases):
        inp = _inputs(seqlens, 8, 2, window=window, sinks=sinks, seed=300 + n, head_dim=head_dim,
                      scale=head_dim ** -0.5)
        full = _run(lib, inp)
        T, hq = full.shape[0], full.shape[1]
        g = torch.Generator().manual_seed(400 + n)
        pick = torch.randperm(T * hq, generator=g)
        pick = torch.cat([pick, pick[:17]])          # repeats
        rows = (pick // hq).numpy().astype(np.int64)
        heads = (pick % hq).numpy().astype(np.int32)
        got = oracle.prefill_rows(*oracle_args(inp), rows=rows, heads=heads, lib=lib)
        assert np.array_equal(got, full[rows, heads]), \
            f"rows routine differs from the full routine (W={window} sinks={sinks} D={head_dim})"


ALL_PINS = [pin_rows_equal_prefill, pin_sdpa_no_sink, pin_sdpa_sink_augmented, pin_closed_form_q_zero,
            pin_closed_form_window_one, pin_hand_example, pin_sink_extremes,
            pin_probs_sum_to_one, pin_window_covering_equals_full, pin_packed_equals_separate,
            pin_permute_sequences, pin_causality, pin_head_groups, pin_scale_homogeneity]


# ---------------------------------------------------------------------------
# Pins of the paged-cache form (oracle.cache_attend): new query rows against a
# KV cache, the causal diagonal aligned to the bottom right; decode is q_len 1.

def _cache_inputs(q_lens, k_lens, hq, hkv, page_size, window=0, sinks=True, seed=0, spare=3):
    wl = workloads.CacheWorkload("pin", tuple(q_lens), tuple(k_lens), hq, hkv, page_size,
                                 window=window, sinks=sinks, seed=seed, spare_pages=spare)
    return workloads.make_cache_inputs(wl)


def _cache_run(lib, inp):
    return oracle.cache_attend(
        bf16_bits(inp["q"]), bf16_bits(inp["k_cache"]), bf16_bits(inp["v_cache"]),
        None if inp["sinks"] is None else inp["sinks"].numpy().astype(np.float32),
        inp["cu_seqlens_q"].numpy(), inp["seqlens_k"].numpy(), inp["block_table"].numpy(),
        inp["window"], inp["softmax_scale"], lib=lib)


def _gather(cache, table_row, L, page_size):
    """Contiguous [L, Hkv, D] rows of one sequence, fetched page by page."""
    rows = [cache[int(table_row[j // page_size]), j % page_size] for j in range(L)]
    return torch.stack(rows) if rows else cache[0, :0]


def _cache_sdpa_reference(inp, augment_sink: bool):
    """SDPA in float64 per sequence on gathered K/V, mask aligned to the bottom right."""
    q = inp["q"].to(torch.float64)
    hq, D = q.shape[1], q.shape[2]
    hkv = inp["k_cache"].shape[2]
    G = hq // hkv
    P = inp["page_size"]
    scale, W = inp["softmax_scale"], inp["window"]
    cu = inp["cu_seqlens_q"].tolist()
    out = torch.zeros_like(q)
    for b in range(len(cu) - 1):
        qs, qe = cu[b], cu[b + 1]
        nq, L = qe - qs, int(inp["seqlens_k"][b])
        if nq == 0:
            continue
        k = _gather(inp["k_cache"], inp["block_table"][b], L, P).to(torch.float64)
        v = _gather(inp["v_cache"], inp["block_table"][b], L, P).to(torch.float64)
        pos = torch.arange(nq).view(nq, 1) + (L - nq)
        j = torch.arange(L).view(1, L)
        mask = (j <= pos) & ((pos - j < W) if W > 0 else torch.ones_like(j, dtype=torch.bool))
        qb = q[qs:qe].transpose(0, 1)
        kb = k.repeat_interleave(G, dim=1).transpose(0, 1)
        vb = v.repeat_interleave(G, dim=1).transpose(0, 1)
        if augment_sink:
            sig = inp["sinks"].to(torch.float64)
            qb = torch.cat([qb, torch.ones(hq, nq, 1, dtype=torch.float64)], dim=2)
            kb = torch.cat([kb, torch.zeros(hq, L, 1, dtype=torch.float64)], dim=2)
            ksink = torch.zeros(hq, 1, D + 1, dtype=torch.float64)
            ksink[:, 0, D] = sig / scale
            kb = torch.cat([kb, ksink], dim=1)
            vb = torch.cat([vb, torch.zeros(hq, 1, D, dtype=torch.float64)], dim=1)
            mask = torch.cat([mask, torch.ones(nq, 1, dtype=torch.bool)], dim=1)
        ob = F.scaled_dot_product_attention(qb.contiguous(), kb.contiguous(), vb.contiguous(),
                                            attn_mask=mask, scale=scale)
        # a row that sees no key has no softmax; its output is zero by definition
        ob = torch.where(mask.any(dim=1).view(1, nq, 1), ob, torch.zeros_like(ob))
        out[qs:qe] = ob.transpose(0, 1)
    return out.numpy()


CACHE_CASES = [  # (q_lens, k_lens, Hq, Hkv, page_size, window)
    ([1, 1, 1, 1], [1, 9, 40, 17], 4, 2, 4, 0),
    ([3, 1, 7], [3, 30, 50], 4, 1, 8, 0),
    ([5, 2], [44, 13], 8, 2, 4, 6),
    ([1, 1], [64, 33], 2, 2, 16, 1),
    ([12], [12], 4, 2, 4, 5),
    ([0, 4, 1], [10, 4, 0], 4, 2, 2, 0),
]


def pin_cache_sdpa(lib):
    for n, (ql, kl, hq, hkv, P, w) in enumerate(CACHE_CASES):
        for with_sink in (False, True):
            inp = _cache_inputs(ql, kl, hq, hkv, P, window=w, sinks=with_sink, seed=200 + n)
            if with_sink:
                inp["sinks"] = inp["sinks"] * 3.0 + torch.linspace(-2.0, 4.0, hq)
            _close(_cache_run(lib, inp), _cache_sdpa_reference(inp, with_sink), 1e-12,
                   f"cache SDPA case q_lens={ql} k_lens={kl} page={P} W={w} sink={with_sink}")


def _contiguous_prefill_inputs(inp):
    """The same sequences as plain packed prefill inputs (q_len == k_len for each)."""
    P = inp["page_size"]
    ks, vs = [], []
    for b in range(inp["seqlens_k"].shape[0]):
        L = int(inp["seqlens_k"][b])
        ks.append(_gather(inp["k_cache"], inp["block_table"][b], L, P))
        vs.append(_gather(inp["v_cache"], inp["block_table"][b], L, P))
    return {"q": inp["q"], "k": torch.cat(ks), "v": torch.cat(vs), "sinks": inp["sinks"],
            "cu_seqlens": inp["cu_seqlens_q"], "window": inp["window"],
            "softmax_scale": inp["softmax_scale"]}


def pin_cache_full_chunk_is_prefill(lib):
    """When the new rows are the whole sequence, the cache form is the plain prefill."""
    for n, (lens, P, w) in enumerate([([7, 33, 1], 4, 0), ([20, 48], 16, 9), ([0, 5], 2, 2)]):
        inp = _cache_inputs(lens, lens, 4, 2, P, window=w, seed=220 + n)
        _close(_cache_run(lib, inp), _run(lib, _contiguous_prefill_inputs(inp)), 1e-13,
               f"full chunk vs prefill lens={lens} page={P} W={w}")


def pin_cache_decode_is_last_prefill_row(lib):
    """Decode of position i (q_len 1, k_len i + 1) equals row i of the full prefill."""
    L, P = 37, 8
    for w in (0, 10):
        full = _cache_inputs([L], [L], 4, 2, P, window=w, seed=240 + w)
        ref = _run(lib, _contiguous_prefill_inputs(full))
        for i in (0, 1, 9, 10, 24, L - 1):
            one = dict(full, q=full["q"][i:i + 1],
                       cu_seqlens_q=torch.tensor([0, 1], dtype=torch.int32),
                       seqlens_k=torch.tensor([i + 1], dtype=torch.int32))
            _close(_cache_run(lib, one), ref[i:i + 1], 1e-13, f"decode at position {i}, W={w}")


def pin_cache_page_layout(lib):
    """Where the pages sit in the pool, and what unused slots hold, does not matter."""
    inp = _cache_inputs([2, 1, 4], [19, 26, 9], 4, 2, 4, window=0, seed=260, spare=5)
    base = _cache_run(lib, inp)
    n_pages = inp["k_cache"].shape[0]
    perm = torch.randperm(n_pages, generator=torch.Generator().manual_seed(7))
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(n_pages)
    table = inp["block_table"].clone()
    table[table >= 0] = inv[table[table >= 0].long()].to(torch.int32)
    moved = dict(inp, k_cache=inp["k_cache"][perm], v_cache=inp["v_cache"][perm], block_table=table)
    assert np.array_equal(_cache_run(lib, moved), base), "moving pages changed the result"
    # poison every slot no sequence uses
    used = torch.zeros(n_pages, inp["page_size"], dtype=torch.bool)
    for b in range(3):
        for j in range(int(inp["seqlens_k"][b])):
            used[int(inp["block_table"][b, j // 4]), j % 4] = True
    kc, vc = inp["k_cache"].clone(), inp["v_cache"].clone()
    kc[~used] = float("nan")
    vc[~used] = float("nan")
    poisoned = _cache_run(lib, dict(inp, k_cache=kc, v_cache=vc))
    assert np.array_equal(poisoned, base), "unused cache slots leaked into the result"


def pin_cache_rows_without_keys(lib):
    """A row with no cached key at or before its position has a zero output."""
    inp = _cache_inputs([3, 1, 2], [1, 0, 2], 4, 2, 4, seed=280)
    out = _cache_run(lib, inp)
    assert np.all(out[0:2] == 0.0) and np.any(out[2] != 0.0), "rows before the first key"
    assert np.all(out[3] == 0.0), "empty sequence"
    assert np.all(out[4:6] != 0.0)


ALL_PINS += [pin_cache_sdpa, pin_cache_full_chunk_is_prefill, pin_cache_decode_is_last_prefill_row,
             pin_cache_page_layout, pin_cache_rows_without_keys]
