"""GPU parity of the verification pass's decode attention over a KV-cached
prefix (spec_decode_attention) and of the KV commit (spec_kv_commit)
against the float64 oracle (oracle/attention.py).

Tolerance, from the arithmetic: a score is a float32 sum of hd products of
a float32 query, multiplied by scale log2(e) (one rounding, 2^-24 relative)
and split exactly into three bf16 terms, and an exact bf16 key, so in
natural units |delta s| <= (hd + 1) 2^-24 sum_d |q_d k_d| scale; the
hardware exp2 of the score less the row's reference max adds about one ulp
(2^-23 relative) plus 2^-22 for the denormal range; the probabilities enter
P V as two bf16 terms, 2^-16 relative.  The softmax weights then move by at
most 2 |delta s| + the exp error + 2^-16, and the output (a convex
combination of value rows) by that times max |v|.  The test bounds every
output row by
    max|v| (2 hd 2^-24 S1 + 2^-23 max(2 S0, 8) + 2^-22 + 2^-16),
S1 = max_t sum_d |q_d k_d| scale, S0 = max_t |q . k_t| scale, computed
from the oracle's inputs; its exp term also covers a natural-base exp
whose argument is rounded (2^-23 |x| for an argument x)."""

import numpy as np
import pytest
import torch

import oracle
import synth
from harness import log_measurement

pytestmark = pytest.mark.gpu
sv = pytest.importorskip("speculative_decoding_verification_06_amd")
DEV = "cuda"


def bf16_cache(gen, shape):
    return synth.f32_to_bf16_bits(gen.standard_normal(shape, dtype=np.float32))


def to_dev_bf16(bits):
    return torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)


def tolerance(q, K, Vc, L, n_new, scale):
    """Per (b, i, h) bound on |out_gpu - out_ref| (see the module docstring)."""
    B, _, H, hd = q.shape
    G = H // K.shape[1]
    tol = np.zeros((B, n_new, H))
    for b in range(B):
        T = L[b] + n_new
        for h in range(H):
            kk = np.abs(K[b, h // G, :T])
            vmax = np.abs(Vc[b, h // G, :T]).max()
            s1 = (np.abs(q[b, :, h]) @ kk.T).max(axis=-1) * scale          # [n_new]
            s0 = np.abs(q[b, :, h] @ K[b, h // G, :T].T).max(axis=-1) * scale
            tol[b, :, h] = vmax * (2 * hd * 2.0 ** -24 * s1 + 2.0 ** -23 * np.maximum(2 * s0, 8.0)
                                   + 2.0 ** -22 + 2.0 ** -16)
    return tol


CASES = [
    # name, B, n_new, H, Hkv, hd, max_seq, lengths, tree
    ("chain-g4-short", 1, 5, 32, 8, 128, 256, [100], False),
    ("chain-g8-8k", 1, 5, 64, 8, 128, 8192, [8187], False),
    ("tree-15-g8", 2, 15, 64, 8, 128, 3000, [2900, 17], True),
    ("batch-hd64", 6, 7, 16, 4, 64, 704, [0, 1, 63, 64, 65, 697], False),
    ("rows-over-32-tree", 3, 40, 8, 2, 128, 1200, [1000, 5, 300], True),
    ("mha-g1", 2, 3, 4, 4, 64, 96, [93, 40], True),
    ("one-row-cache-end", 2, 1, 8, 8, 128, 72, [71, 70], False),
    ("splits-13", 1, 5, 64, 8, 128, 3328, [3300], False),
    ("splits-256-hd64", 1, 5, 4, 1, 64, 131072, [131000], False),
    ("rt3-chain-hd64", 2, 6, 32, 4, 64, 2048, [1500, 2040], False),
    ("rt4-tree-padded", 3, 9, 48, 8, 128, 1024, [0, 500, 1015], True),
    ("rt1-g2", 4, 5, 4, 2, 128, 512, [10, 64, 128, 300], False),
    ("one-tile-cache", 2, 3, 8, 4, 128, 64, [60, 10], False),
    ("rt5-chain", 2, 10, 64, 8, 128, 640, [600, 3], False),
]
# The launch splits each row's keys S ways (at least four 64-key tiles per
# split) and merges the splits in a second launch when S > 1; S = 1 writes the
# output directly (chain-g4-short, mha-g1, one-row-cache-end, one-tile-cache).
# A work group holds 16-row tiles of rows, one per wave (four waves up to 64
# rows, eight up to 128): one tile in mha-g1, one-row-cache-end, rt1-g2 and
# one-tile-cache, two in chain-g4-short, batch-hd64 and splits-256-hd64,
# three in chain-g8-8k, splits-13 and rt3-chain-hd64, four in rt4-tree-padded
# (padding rows), five in rt5-chain (three waves that only load), eight in
# tree-15-g8 and in rows-over-32-tree (two row groups).  The merge takes four
# dimensions per thread up to 16 splits (2 to 11 here) and one above (32 in
# chain-g8-8k, 256 in splits-256-hd64: more splits than threads per row);
# S = 13 in splits-13 (its groups of eight loads plus a tail).


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_attention_parity(case):
    name, B, n_new, H, Hkv, hd, S, lengths, tree = case
    print(f"[case] attention {name} B={B} n_new={n_new} H={H} Hkv={Hkv} hd={hd} max_seq={S}", flush=True)
    gen = synth.generator(8300 + CASES.index(case), synth.T_MISC)
    q = gen.standard_normal((B, n_new, H, hd), dtype=np.float32)
    K = bf16_cache(gen, (B, Hkv, S, hd))
    Vc = bf16_cache(gen, (B, Hkv, S, hd))
    L = np.array(lengths, dtype=np.int32)
    parent = None
    if tree:
        parent = np.array([[-1] + [int(gen.integers(-1, i)) for i in range(1, n_new)]
                           for _ in range(B)], dtype=np.int32)
    scale = 1.0 / np.sqrt(hd)
    ref = oracle.attention.decode_attention(q, K, Vc, L, parent, scale)
    Vt = np.ascontiguousarray(np.swapaxes(Vc, 2, 3))        # the library's value layout
    out = sv.decode_attention(torch.from_numpy(q).to(DEV), to_dev_bf16(K), to_dev_bf16(Vt),
                              torch.from_numpy(L).to(DEV),
                              None if parent is None else torch.from_numpy(parent).to(DEV), scale)
    out2 = sv.decode_attention(torch.from_numpy(q).to(DEV), to_dev_bf16(K), to_dev_bf16(Vt),
                               torch.from_numpy(L).to(DEV),
                               None if parent is None else torch.from_numpy(parent).to(DEV), scale)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    assert np.array_equal(out.cpu().numpy(), out2.cpu().numpy())       # run-to-run identical
    err = np.abs(got - ref).max(axis=-1)
    tol = tolerance(q.astype(np.float64), oracle.as_f64(K), oracle.as_f64(Vc), L, n_new, scale)
    log_measurement({"what": f"attention {name}", "abs_err_max": float(err.max()),
                     "worst_err_over_tol": float((err / tol).max())})
    print(f"attention {name}: max abs err {err.max():.2e}, worst err/tol {(err / tol).max():.3f}")
    assert (err <= tol).all()


def test_kv_commit_chain_and_tree():
    gen = synth.generator(8390, synth.T_MISC)
    B, Hkv, S, hd, n_new = 3, 2, 64, 128, 6
    K = bf16_cache(gen, (B, Hkv, S, hd))
    Vc = bf16_cache(gen, (B, Hkv, S, hd))
    L = np.array([10, 0, 58], dtype=np.int32)
    n_acc = np.array([3, -1, 5], dtype=np.int32)
    path = np.array([[0, 2, 4, -1, -1], [0, 0, 0, 0, 0], [0, 1, 2, 3, 4]], dtype=np.int32)
    for use_path in (False, True):
        k_ref, v_ref = K.copy(), Vc.copy()
        want = oracle.attention.kv_commit(k_ref, v_ref, L, n_acc, path if use_path else None)
        kd, vd = to_dev_bf16(K), to_dev_bf16(np.ascontiguousarray(np.swapaxes(Vc, 2, 3)))
        ld = torch.from_numpy(L).to(DEV)
        sv.kv_commit(kd, vd, ld, torch.from_numpy(n_acc).to(DEV), n_new,
                     torch.from_numpy(path).to(DEV) if use_path else None)
        torch.cuda.synchronize()
        assert ld.cpu().numpy().tolist() == want.tolist()
        assert np.array_equal(kd.view(torch.int16).cpu().numpy().view(np.uint16), k_ref)
        assert np.array_equal(vd.view(torch.int16).cpu().numpy().view(np.uint16), np.swapaxes(v_ref, 2, 3))
