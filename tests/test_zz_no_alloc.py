"""The allocation-free entry point (spec_verify_noalloc) against spec_verify.

Both run the same kernels; the allocation-free one keeps its workspace in
the library's static per-GPU scratch.  Calls in a row, the second with a
smaller batch than the first, so each runs on scratch the one before left
behind: each must decide bit for bit as spec_verify with a fresh workspace.
Once its kernels have run, the call must change no device memory use, and a
pass larger than the scratch is refused before anything is launched."""

import numpy as np
import pytest
import torch

import oracle
import synth
from harness import draft_q, sample_drafts

pytestmark = pytest.mark.gpu
sv = pytest.importorskip("speculative_decoding_verification_06_amd")
DEV = "cuda"


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def make_inputs(m, key, B, gamma, V, T, top_p):
    hidden = synth.hidden_np(key, B, gamma, m["blocks"][0]["w_up"].shape[0])
    ell = oracle.forward(hidden, m["blocks"], m["lm_head"], m["eps"])
    q = draft_q(ell, synth.noise_np(key, B, gamma, V, 0.6))
    draft = sample_drafts(q, T, top_p, key) if T > 0 else ell[:, :gamma].argmax(-1).astype(np.int32)
    return dev(hidden), dev(draft), dev(q)


def torch_weights(m):
    t = lambda a: torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    return [{"w_up": t(b["w_up"]), "w_down": t(b["w_down"])} for b in m["blocks"]], t(m["lm_head"])


def test_noalloc_matches_spec_verify_on_two_calls():
    key = (8800,)
    d, ffn, nb, V = 256, 512, 2, 3000
    m = synth.model_np(key, d, ffn, nb, V, "bf16")
    blocks, lm = torch_weights(m)
    w = sv.Weights(blocks, lm, eps=m["eps"])
    calls = [(4, 4, 0.7, 0.9, 11), (1, 2, 1.0, 1.0, 12), (3, 3, 0.0, 1.0, 13)]
    inputs = [make_inputs(m, (8800, i), B, g, V, T, tp) for i, (B, g, T, tp, _) in enumerate(calls)]
    refs = []
    for (B, g, T, tp, seed), (h, dr, q) in zip(calls, inputs):
        n_ref, e_ref = sv.verify(w, h, dr, q if T > 0 else None, T, tp, seed)
        refs.append((n_ref, e_ref))
    torch.cuda.synchronize()
    # Two rounds of three calls in a row (the second call's batch smaller
    # than the first's).  The first launch of a kernel on a device may make the
    # runtime set memory aside for itself (lazy code loading, the per-lane
    # spill area of the queue); the second round must leave device memory
    # use exactly as it finds it.
    for rnd in range(2):
        outs = [(torch.full((B,), -7, dtype=torch.int32, device=DEV),
                 torch.full((B, g + 1), -7, dtype=torch.int32, device=DEV)) for B, g, *_ in calls]
        torch.cuda.synchronize()
        free0 = torch.cuda.mem_get_info()[0]
        for (B, g, T, tp, seed), (h, dr, q), (n, e) in zip(calls, inputs, outs):
            print(f"[case] noalloc round {rnd} B={B} gamma={g} T={T} top_p={tp}", flush=True)
            sv.verify_noalloc(w, h, dr, q if T > 0 else None, T, tp, seed, n, e)
        torch.cuda.synchronize()
        if rnd == 1:
            assert torch.cuda.mem_get_info()[0] == free0
        for (B, g, T, tp, seed), (n, e), (n_ref, e_ref) in zip(calls, outs, refs):
            assert torch.equal(n, n_ref) and torch.equal(e, e_ref), (rnd, B, g, T, tp)
            assert (n.cpu().numpy() >= 0).all()
    w.close()


def test_noalloc_refuses_a_pass_larger_than_the_scratch():
    key = (8801,)
    d, ffn, V = 256, 512, 3000
    m = synth.model_np(key, d, ffn, 1, V, "bf16")
    blocks, lm = torch_weights(m)
    w = sv.Weights(blocks, lm, eps=m["eps"])
    B, gamma = 2000, 7
    assert w.workspace_size(B, gamma) > sv.NOALLOC_SCRATCH_BYTES
    h = torch.zeros((B, gamma + 1, d), device=DEV)
    dr = torch.zeros((B, gamma), dtype=torch.int32, device=DEV)
    q = torch.full((B, gamma, V), 1.0 / V, device=DEV)
    n = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    e = torch.full((B, gamma + 1), -7, dtype=torch.int32, device=DEV)
    with pytest.raises(sv.SpecError) as ei:
        sv.verify_noalloc(w, h, dr, q, 1.0, 1.0, 0, n, e)
    assert ei.value.status == sv.SPEC_ESCRATCH
    torch.cuda.synchronize()
    assert (n == -7).all()          # nothing was launched
    w.close()
