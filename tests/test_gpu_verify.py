"""GPU parity of the HIP verification path against the float64 oracle.

Small shapes the oracle finishes in seconds, spanning several tiles and a
ragged tail, every GEMM path (vector FMA fp32 / bf16, MFMA with k-split and
row-split work groups, row chunking) and every sampling mode (T = 1,
T != 1 with top-p, greedy), plus edge cases.  All calls go through the C ABI.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from harness import (LOGIT_TOL, LOGIT_TOL_TWO, assert_tokens_match, cap_applies, compare_probs,
                     compare_tokens, two_term_pass, draft_q, greedy_drafts, log_measurement, logits_rel_err,
                     sample_drafts)

pytestmark = pytest.mark.gpu

sv = pytest.importorskip("speculative_decoding_verification_06_amd")
DEV = "cuda"


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def host_to_torch_weights(m, wdtype):
    def t(a):
        if a is None:
            return None
        if wdtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
        return dev(a)
    blocks = [{"w_up": t(b["w_up"]), "w_down": t(b["w_down"]), "gain": t(b["gain"])}
              for b in m["blocks"]]
    return blocks, t(m["lm_head"])


def make_case(key, B, gamma, d, ffn, V, n_blocks, wdtype, T, top_p, sigma=0.5, gains=False):
    m = synth.model_np(key, d, ffn, n_blocks, V, wdtype, random_gain=gains)
    hidden = synth.hidden_np(key, B, gamma, d)
    ell = oracle.forward(hidden, m["blocks"], m["lm_head"], m["eps"])
    noise = synth.noise_np(key, B, gamma, V, sigma)
    q = draft_q(ell, noise)
    if T == 0:
        draft = greedy_drafts(ell, key)
    else:
        draft = sample_drafts(q, T, top_p, key)
    return m, hidden, ell, q, draft


def run_gpu(w, hidden, draft, q, T, top_p, seed):
    n, e, logits, p, qq = sv.verify_debug(w, dev(hidden), dev(draft), dev(q), T, top_p, seed)
    torch.cuda.synchronize()
    cpu = lambda t: None if t is None else t.cpu().numpy()
    return cpu(n), cpu(e), cpu(logits), cpu(p), cpu(qq)


def check(m, hidden, ell, q, draft, T, top_p, seed, w, what, two_term=False):
    n, e, logits, p, qq = run_gpu(w, hidden, draft, q, T, top_p, seed)
    # the plain call (what the benchmark times) decides exactly as the debug call
    n2, e2 = sv.verify(w, dev(hidden), dev(draft), dev(q) if T > 0 else None, T, top_p, seed)
    torch.cuda.synchronize()
    assert np.array_equal(n2.cpu().numpy(), n) and np.array_equal(e2.cpu().numpy(), e), what
    err = logits_rel_err(logits, ell)
    log_measurement({"what": f"{what} logits", "rel_err_max": float(err.max())})
    assert err.max() <= 1e-3, f"{what}: logits rel err {err.max():.2e}"
    # the token comparison below assumes the logits this close
    tol = LOGIT_TOL_TWO if two_term else LOGIT_TOL
    assert err.max() <= tol, f"{what}: logits rel err {err.max():.2e}"
    ref = oracle.spec_verify_from_logits(ell, draft, q, T, top_p, seed, logit_tol=tol)
    assert_tokens_match(n, e, ref, what=what,
                        cap=not two_term and cap_applies(ell.shape[-1], top_p, False))
    if T > 0:
        compare_probs(p, qq, ref, ell, q, T, top_p, range(len(n)), what, tol)
    return err.max()


CASES = [
    # name, B, gamma, d, ffn, V, blocks, wdtype, T, top_p, gains, weights kwargs
    ("tiny-f32", 1, 4, 256, 1024, 512, 1, "f32", 1.0, 1.0, False, {}),
    ("ragged-f32-topp", 3, 5, 200, 300, 1000, 2, "f32", 0.7, 0.9, True, {}),
    ("bf16-mfma-k", 2, 4, 256, 512, 1000, 2, "bf16", 1.0, 1.0, False, {}),
    ("bf16-mfma-k2-greedy", 4, 4, 320, 640, 777, 2, "bf16", 0.0, 1.0, True, {}),
    ("bf16-mfma-rows-topp", 8, 8, 256, 512, 2000, 1, "bf16", 0.7, 0.9, False, {}),
    ("bf16-mfma-chunked", 40, 6, 128, 256, 500, 1, "bf16", 1.3, 0.6, False, {}),
    ("bf16-wide-two-row-groups", 20, 6, 192, 320, 900, 2, "bf16", 1.0, 1.0, True, {}),
    # wide GEMM shapes: one row group of 1 row tile (12 rows), two row groups
    # of 3 and of 4 row tiles (90 and 120 rows)
    ("bf16-wide-one-tile", 4, 2, 160, 224, 650, 1, "bf16", 0.8, 0.9, True, {}),
    ("bf16-wide-90-rows", 10, 8, 128, 256, 600, 1, "bf16", 1.0, 1.0, False, {}),
    ("bf16-wide-120-rows-greedy", 15, 7, 128, 192, 520, 2, "bf16", 0.0, 1.0, True, {}),
    ("bf16-wide-224-greedy", 32, 6, 160, 288, 700, 1, "bf16", 0.0, 1.0, False, {}),
    # one sequence with many drafts (the gamma sweep's longest chains): two
    # row groups of 5 and of 6 row tiles (129 and 161 rows)
    ("bf16-wide-129-rows", 1, 128, 192, 320, 650, 2, "bf16", 0.8, 0.9, True, {}),
    ("bf16-wide-161-rows", 1, 160, 128, 256, 700, 1, "bf16", 1.0, 1.0, False, {}),
    # the exact three-term split kept in wide passes (SPEC_FLAG_EXACT_SPLIT;
    # without it every wide pass takes two terms): two row groups at 224
    # rows greedy, 129 rows sampled with top-p and 90 rows; one row group at
    # 72 rows (the top-p workload's shape) and in the 1024-thread LM head;
    # and 5 rows, a stacked pass, where the flag changes nothing
    ("bf16-wide-224-greedy-exact", 32, 6, 160, 288, 700, 1, "bf16", 0.0, 1.0, False,
     {"exact_split": True}),
    ("bf16-wide-129-rows-exact", 1, 128, 192, 320, 650, 2, "bf16", 0.8, 0.9, True,
     {"exact_split": True}),
    ("bf16-wide-90-rows-exact", 10, 8, 128, 256, 600, 1, "bf16", 1.0, 1.0, False,
     {"exact_split": True}),
    ("bf16-wide-72-rows-exact", 8, 8, 256, 14336, 700, 1, "bf16", 0.7, 0.9, False,
     {"exact_split": True}),
    ("bf16-wide-lm-1024-exact", 3, 5, 128, 192, 70000, 1, "bf16", 0.9, 0.95, False,
     {"exact_split": True}),
    ("bf16-stacked-exact-flag", 1, 4, 128, 256, 600, 1, "bf16", 1.0, 1.0, False,
     {"exact_split": True}),
    # stacked passes of 6 to 8 rows: one eight-row tile of two terms (the
    # large workload's B = 1, gamma = 5 shape), sampled, with top-p and
    # greedy; and 6 rows with the exact split, two five-row tiles of three
    ("bf16-stacked-two-6", 1, 5, 128, 256, 600, 2, "bf16", 1.0, 1.0, True, {}),
    ("bf16-stacked-two-8-topp", 2, 3, 192, 320, 700, 1, "bf16", 0.8, 0.9, False, {}),
    ("bf16-stacked-two-7-greedy", 1, 6, 160, 288, 650, 1, "bf16", 0.0, 1.0, False, {}),
    ("bf16-stacked-6-exact", 1, 5, 128, 256, 600, 1, "bf16", 1.0, 1.0, False,
     {"exact_split": True}),
    # LM heads of more than 4096 tiles at up to 80 rows: the 1024-thread
    # one-row-group shape (18 rows, sampling with top-p; 16 rows, greedy)
    ("bf16-wide-lm-1024", 3, 5, 128, 192, 70000, 1, "bf16", 0.9, 0.95, False, {}),
    ("bf16-wide-lm-1024-greedy", 4, 3, 96, 160, 66000, 1, "bf16", 0.0, 1.0, True, {}),
    # up projections of 14336 columns at up to 80 rows (one K pass per work
    # group when 64-column blocks fill the chip): K of 2 and 8 k-steps
    ("bf16-wide-14336-up", 3, 5, 64, 14336, 500, 1, "bf16", 1.0, 1.0, True, {}),
    ("bf16-wide-14336-up-72", 8, 8, 256, 14336, 700, 1, "bf16", 0.7, 0.9, False, {}),
    ("bf16-fma", 2, 4, 192, 448, 900, 2, "bf16", 1.0, 1.0, True,
     {"keep_rowmajor": True, "mfma_min_rows": 10 ** 6}),
    ("bf16-fma-many-rows", 12, 3, 136, 200, 333, 1, "bf16", 0.8, 1.0, False,
     {"keep_rowmajor": True, "mfma_min_rows": 10 ** 6}),
    ("f32-gamma0", 5, 0, 96, 128, 300, 1, "f32", 1.0, 1.0, False, {}),
    ("f32-no-blocks", 3, 2, 64, 64, 200, 0, "f32", 1.0, 1.0, False, {}),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_verify_parity_small(case):
    name, B, gamma, d, ffn, V, nb, wdtype, T, top_p, gains, wkw = case
    key = (9000 + CASES.index(case),)
    print(f"[case] {name} B={B} gamma={gamma} d={d} ffn={ffn} V={V} blocks={nb} {wdtype} T={T} top_p={top_p}", flush=True)
    m, hidden, ell, q, draft = make_case(key, B, gamma, d, ffn, V, nb, wdtype, T, top_p, gains=gains)
    blocks, lm = host_to_torch_weights(m, wdtype)
    w = sv.Weights(blocks, lm, eps=m["eps"], **wkw)
    M = B * (gamma + 1)
    two = two_term_pass(M, wdtype, wkw.get("exact_split", False), "mfma_min_rows" in wkw)
    for seed in (0, 1, 12345):
        check(m, hidden, ell, q, draft, T, top_p, seed, w, f"{name} seed {seed}", two_term=two)
    if wkw.get("exact_split") and not two_term_pass(M, wdtype):
        # where the default takes three terms the flag leaves the pass as it is
        w3 = sv.Weights(blocks, lm, eps=m["eps"])
        for a, b in zip(run_gpu(w, hidden, draft, q, T, top_p, 7),
                        run_gpu(w3, hidden, draft, q, T, top_p, 7)):
            assert np.array_equal(a, b)
        w3.close()
    w.close()


def test_tiny_workload_steps():
    """The tiny workload as specified: B=1, gamma=4, fp32 weights, 10k verify
    steps, one call per step, fresh hidden states per step, verify seed =
    step.  Every step is checked against the oracle."""
    key = (1,)
    d, ffn, V, gamma, steps = 256, 1024, 512, 4, 10000
    m = synth.model_np(key, d, ffn, 1, V, "f32")
    blocks, lm = host_to_torch_weights(m, "f32")
    w = sv.Weights(blocks, lm, eps=m["eps"])
    ws = w.workspace(1, gamma)
    hidden = np.concatenate([synth.hidden_np((1, 100 + s), 1, gamma, d) for s in range(steps)])
    ell_all = oracle.forward(hidden, m["blocks"], m["lm_head"], m["eps"])
    flagged = draws = mism = knife = ratio_tests = 0
    worst = 0.0
    h_dev = dev(hidden)
    n_all = torch.empty((steps, 1), dtype=torch.int32, device=DEV)
    e_all = torch.empty((steps, 1, gamma + 1), dtype=torch.int32, device=DEV)
    lg_all = torch.empty((steps, 1, gamma + 1, V), dtype=torch.float32, device=DEV)
    qs, drafts = [], []
    for step in range(steps):
        skey = (1, 100 + step)
        ell = ell_all[step:step + 1]
        q = draft_q(ell, synth.noise_np(skey, 1, gamma, V, 0.5))
        qs.append(q)
        drafts.append(sample_drafts(q, 1.0, 1.0, skey))
    q_dev, d_dev = dev(np.concatenate(qs)), dev(np.concatenate(drafts))
    for step in range(steps):
        n, e, logits, _, _ = sv.verify_debug(w, h_dev[step:step + 1], d_dev[step:step + 1],
                                             q_dev[step:step + 1], 1.0, 1.0, step,
                                             want_probs=False, workspace=ws)
        n_all[step].copy_(n)
        e_all[step].copy_(e)
        lg_all[step].copy_(logits)
    torch.cuda.synchronize()
    n_all, e_all, lg_all = n_all.cpu().numpy(), e_all.cpu().numpy(), lg_all.cpu().numpy()
    for step in range(steps):
        ell = ell_all[step:step + 1]
        worst = max(worst, logits_rel_err(lg_all[step], ell).max())
        ref = oracle.spec_verify_from_logits(ell, drafts[step], qs[step], 1.0, 1.0, step,
                                             logit_tol=LOGIT_TOL)
        rep = compare_tokens(n_all[step], e_all[step], ref)
        assert not rep.unexplained, f"tiny step {step}: {rep.record()}"
        flagged += sum(rep.flagged.values())
        knife += rep.knife
        ratio_tests += rep.total["accept"]
        draws += rep.draws
        mism += len(rep.mismatched)
    print(f"tiny: {steps} steps, {draws} draws, {flagged} flagged, {mism} differing rows, "
          f"worst logit rel err {worst:.2e}")
    log_measurement({"what": "tiny 10k steps", "draws": draws, "flagged": flagged,
                     "ratio_knife_edges": knife, "mismatched_rows": mism,
                     "logit_rel_err_max": float(worst)})
    assert worst <= LOGIT_TOL
    assert mism <= 0.001 * draws
    assert knife <= max(1, 0.001 * ratio_tests)
    w.close()


def test_repeat_calls_are_bit_identical():
    key = (77,)
    m, hidden, ell, q, draft = make_case(key, 4, 4, 256, 512, 3000, 2, "bf16", 0.7, 0.9)
    blocks, lm = host_to_torch_weights(m, "bf16")
    w = sv.Weights(blocks, lm, eps=m["eps"])
    outs = [run_gpu(w, hidden, draft, q, 0.7, 0.9, 5) for _ in range(3)]
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert np.array_equal(a, b)
    w.close()


# ---------------------------------------------------------------- rule only (given logits)

RULE_CASES = [
    (4, 4, 512, 1.0, 1.0), (8, 8, 5000, 0.7, 0.9), (3, 6, 1000, 0.0, 1.0),
    (16, 2, 130, 1.3, 0.6), (6, 0, 300, 1.0, 1.0), (5, 3, 64, 1.0, 0.5), (7, 3, 1, 1.0, 1.0),
    (2, 5, 70000, 0.9, 0.95), (1, 4, 32000, 1.0, 1.0), (1, 5, 128256, 1.0, 1.0),
    (2, 3, 128256, 0.7, 0.9), (1, 2, 600000, 1.0, 1.0), (3, 4, 129, 0.0, 1.0),
    # extremes: a nucleus of about one token, near-greedy and near-flat
    # temperatures, top-p with V = 1
    (4, 4, 3000, 1.0, 0.01), (4, 4, 3000, 0.05, 0.9), (3, 3, 3000, 8.0, 0.5),
    (2, 3, 1, 0.7, 0.9),
]


@pytest.mark.parametrize("case", RULE_CASES, ids=[str(c) for c in RULE_CASES])
def test_rule_from_logits_parity(case):
    B, gamma, V, T, top_p = case
    key = (5000 + RULE_CASES.index(case),)
    print(f"[case] rule B={B} gamma={gamma} V={V} T={T} top_p={top_p}", flush=True)
    gen = synth.generator(*key, synth.T_MISC)
    ell = (gen.standard_normal((B, gamma + 1, V), dtype=np.float32) * 2.0)
    q = draft_q(ell.astype(np.float64), synth.noise_np(key, B, gamma, V, 0.7))
    draft = greedy_drafts(ell.astype(np.float64), key) if T == 0 else sample_drafts(q, T, top_p, key)
    for seed in (3, 4):
        n, e = sv.verify_from_logits(dev(ell), dev(draft), dev(q), T, top_p, seed)
        ref = oracle.spec_verify_from_logits(ell, draft, q, T, top_p, seed)
        assert_tokens_match(n.cpu().numpy(), e.cpu().numpy(), ref, what=f"rule {case} seed {seed}",
                            cap=cap_applies(V, top_p, True))


TOPP_PATH_CASES = [
    # name, B, gamma, V, T, top_p, logit grid (0: continuous)
    # a flat 600k-token row: the first digit's crossing bucket overflows the
    # LDS candidate list, so the last pass and the tie scan read the row
    ("candidate-overflow", 1, 2, 600000, 0.8, 0.9, 0.0),
    # logits on a 0.5 grid: thousands of tokens share the cut key, more than
    # one thread orders, so the tie falls back to the ordered range scan
    ("many-ties", 2, 3, 5000, 1.0, 0.6, 0.5),
    ("many-ties-draft-T", 2, 3, 5000, 0.7, 0.75, 0.5),
]


@pytest.mark.parametrize("case", TOPP_PATH_CASES, ids=[c[0] for c in TOPP_PATH_CASES])
def test_rule_topp_paths(case):
    name, B, gamma, V, T, top_p, grid = case
    key = (5600 + TOPP_PATH_CASES.index(case),)
    print(f"[case] topp path {name} B={B} gamma={gamma} V={V} T={T} top_p={top_p}", flush=True)
    gen = synth.generator(*key, synth.T_MISC)
    ell = gen.standard_normal((B, gamma + 1, V), dtype=np.float32) * 2.0
    if grid > 0:
        ell = (np.round(ell / grid) * grid).astype(np.float32)
    q = draft_q(ell.astype(np.float64), synth.noise_np(key, B, gamma, V, 0.7))
    if grid > 0:
        q = (np.round(q * 2.0 ** 12) / 2.0 ** 12).astype(np.float32)   # tied draft probabilities too
        q = (q / q.sum(-1, keepdims=True)).astype(np.float32)
    draft = sample_drafts(q, T, top_p, key)
    for seed in (3, 4):
        n, e = sv.verify_from_logits(dev(ell), dev(draft), dev(q), T, top_p, seed)
        n, e = n.cpu().numpy(), e.cpu().numpy()
        ref = oracle.spec_verify_from_logits(ell, draft, q, T, top_p, seed)
        if grid > 0:
            # exact fp32 inputs and ties broken by ascending id on both sides:
            # the oracle's near-tie band (which covers a whole tie group and
            # would flag most ratio tests here) is no uncertainty, so every
            # row must agree
            assert np.array_equal(n, ref.n_accepted), f"topp {name} seed {seed}: {n} vs {ref.n_accepted}"
            assert np.array_equal(e, ref.emitted), f"topp {name} seed {seed}"
        else:
            assert_tokens_match(n, e, ref, what=f"topp {name} seed {seed}",
                                cap=cap_applies(V, top_p, True))


def test_rule_edge_cases():
    """Bad token ids, a draft outside q's support (q' = 0), and a zero
    residual (p' = q' = one-hot after top-p) that falls back to p'."""
    B, gamma, V = 4, 3, 50
    gen = synth.generator(4242, synth.T_MISC)
    ell = gen.standard_normal((B, gamma + 1, V), dtype=np.float32)
    ell[:, :, 7] += 8.0                      # token 7 dominates every row
    q = draft_q(ell.astype(np.float64), np.zeros((B, gamma, V), dtype=np.float32))
    draft = np.full((B, gamma), 7, dtype=np.int32)
    draft[0, 1] = V                          # row 0: out of range
    draft[1, 2] = -3                         # row 1: negative
    q[2, 0, 11] = 0.0                        # row 2: draft 11 has q = 0
    draft[2, 0] = 11
    draft[3, 0] = 20                         # row 3: outside both nuclei below
    for T, top_p in ((1.0, 1.0), (1.0, 0.3), (0.5, 0.2)):
        n, e = sv.verify_from_logits(dev(ell), dev(draft), dev(q), T, top_p, 9)
        n, e = n.cpu().numpy(), e.cpu().numpy()
        ref = oracle.spec_verify_from_logits(ell, draft, q, T, top_p, 9)
        assert n[0] == -1 and (e[0] == -1).all()
        assert n[1] == -1 and (e[1] == -1).all()
        assert_tokens_match(n, e, ref, what=f"edge T={T} top_p={top_p}")
        if top_p < 1:
            # p' = q' = one-hot on 7, draft 20 has p' = q' = 0: rejected, the
            # residual is zero and the correction falls back to p' -> 7
            assert n[3] == 0 and e[3, 0] == 7


def test_bad_workspace_is_rejected():
    B, gamma, V = 2, 2, 100
    ell = torch.zeros((B, gamma + 1, V), device=DEV)
    draft = torch.zeros((B, gamma), dtype=torch.int32, device=DEV)
    q = torch.full((B, gamma, V), 1.0 / V, device=DEV)
    with pytest.raises(sv.SpecError) as ei:
        sv.verify_from_logits(ell, draft, q, 1.0, 1.0, 0,
                              workspace=torch.empty(16, dtype=torch.uint8, device=DEV))
    assert ei.value.status == sv.SPEC_EWORKSPACE
