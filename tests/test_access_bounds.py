"""Host-side bounds of every kernel access of a pass (no GPU, nothing
launched).

spec_diag_access_check evaluates the kernels' address formulas at the
extremes of their index ranges for the launch plans spec_verify would take
and checks them against the buffers spec_workspace_size lays out and the
registered weight layouts.  It covers every row count the GEMM paths serve
(1 .. 448 rows: stacked MFMA up to 8, in eight-row tiles of two terms
from 6 to 8 rows, wide MFMA 9 .. 224 with two activation terms, or three
when the exact split is asked for, chunked plain MFMA beyond; and the
vector-FMA paths), the five workload shapes, and the
shapes the GPU parity tests run.  A planted inconsistency (workspace
buffers one fragment short) must be caught, so the check is not vacuous."""

import itertools

import pytest

import speculative_decoding_verification_06_amd as sv
import synth

F32, BF16 = sv.SPEC_F32, sv.SPEC_BF16


def check(d, ffn, nb, V, wdtype, B, gamma, **kw):
    st, msg, n = sv.access_check(d, ffn, nb, V, wdtype, B, gamma, **kw)
    assert st == sv.SPEC_OK, f"d={d} ffn={ffn} blocks={nb} V={V} B={B} gamma={gamma}: {msg}"
    assert n > 0
    return n


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_workload_shapes(name):
    wl = synth.WORKLOADS[name]
    wd = BF16 if wl.wdtype == "bf16" else F32
    check(wl.d, wl.ffn, wl.n_blocks, wl.V, wd, wl.B, wl.gamma)


@pytest.mark.parametrize("model", ["mid", "large"])
def test_gamma_sweep_shapes(model):
    """The decode-versus-verify sweep: B = 1, gamma = 0 .. 160."""
    wl = synth.WORKLOADS[model]
    for gamma in list(range(0, 9)) + [16, 32, 64, 128, 160]:
        check(wl.d, wl.ffn, wl.n_blocks, wl.V, BF16, 1, gamma)


def test_every_row_count_mfma():
    """Rows 1 .. 448 (B * (gamma + 1)) on shapes with ragged K and N, one and
    two blocks, LM heads of one and of more than 4096 tiles."""
    shapes = [(4096, 14336, 1, 32000), (200, 300, 2, 1000), (136, 200, 1, 70000),
              (8192, 28672, 1, 128256), (96, 160, 1, 66000)]
    for (d, ffn, nb, V) in shapes:
        for M in range(1, 449):
            # every M as B sequences of gamma + 1 rows, two ways
            for B, gamma in {(M, 0), (1, M - 1)}:
                check(d, ffn, nb, V, BF16, B, gamma)


def test_every_row_count_fma():
    for (d, ffn, nb, V), wd, kw in itertools.product(
            [(256, 1024, 1, 512), (200, 300, 2, 1000), (64, 64, 0, 200)],
            [F32, BF16], [{}, {"keep_rowmajor": True, "mfma_min_rows": 10 ** 6}]):
        if wd == F32 and kw:
            continue
        for M in range(1, 449, 7):
            check(d, ffn, nb, V, wd, M, 0, **kw)


def test_parity_test_shapes():
    from test_gpu_verify import CASES
    for name, B, gamma, d, ffn, V, nb, wdtype, T, top_p, gains, wkw in CASES:
        check(d, ffn, nb, V, BF16 if wdtype == "bf16" else F32, B, gamma,
              keep_rowmajor=wkw.get("keep_rowmajor", False), mfma_min_rows=wkw.get("mfma_min_rows", 0),
              exact_split=wkw.get("exact_split", False))


def test_exact_split_row_counts():
    """The row counts where the default takes two terms (6 .. 8 stacked, the
    wide GEMM's 9 .. 224), with the exact three-term split kept instead,
    and a short workspace caught either way."""
    for (d, ffn, nb, V) in [(8192, 28672, 1, 128256), (200, 300, 2, 1000), (160, 288, 1, 700)]:
        for M in range(1, 229):
            check(d, ffn, nb, V, BF16, M, 0, exact_split=True)
    for name in ("topp", "greedy"):
        g = synth.WORKLOADS[name]
        check(g.d, g.ffn, g.n_blocks, g.V, BF16, g.B, g.gamma, exact_split=True)
        for exact in (False, True):
            st, msg, _ = sv.access_check(g.d, g.ffn, g.n_blocks, g.V, BF16, g.B, g.gamma,
                                         shrink_bytes=16, exact_split=exact)
            assert st == sv.SPEC_EINVAL and "outside" in msg


@pytest.mark.parametrize("wl", ["tiny", "mid", "topp", "greedy"])
def test_a_short_workspace_is_caught(wl):
    """Buffers one 16-byte fragment short: some kernel reaches past them."""
    w = synth.WORKLOADS[wl]
    st, msg, _ = sv.access_check(w.d, w.ffn, w.n_blocks, w.V, BF16 if w.wdtype == "bf16" else F32,
                                 w.B, w.gamma, shrink_bytes=16)
    assert st == sv.SPEC_EINVAL and "outside" in msg


def test_tree_test_shapes():
    from test_gpu_tree import TREE_CASES
    for name, B, n, kind, d, ffn, nb, V in TREE_CASES:
        check(d, ffn, nb, V, BF16, B, n)
    wl = synth.WORKLOADS["mid"]
    check(wl.d, wl.ffn, wl.n_blocks, wl.V, BF16, 4, 14)


def test_bad_arguments():
    assert sv.access_check(0, 1, 1, 1, F32, 1, 0)[0] == sv.SPEC_EINVAL
    assert sv.access_check(8, 8, 1, 8, 7, 1, 0)[0] == sv.SPEC_EDTYPE
