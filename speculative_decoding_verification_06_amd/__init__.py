"""Python binding of libspecverify (the C ABI in include/specverify.h).

Argument marshalling only: every step of the verification runs in the HIP
library.  PyTorch supplies device memory and the current stream.  If the
shared library has not been built the import of a binding function raises;
there is no fallback path.
"""

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libspecverify.so")

SPEC_OK, SPEC_EINVAL, SPEC_EDTYPE, SPEC_EWORKSPACE, SPEC_EHIP, SPEC_ENOMEM, SPEC_ESCRATCH = \
    0, -1, -2, -3, -4, -5, -6
NOALLOC_SCRATCH_BYTES = 128 << 20
SPEC_F32, SPEC_BF16 = 0, 1
SPEC_FLAG_KEEP_ROWMAJOR = 1
SPEC_FLAG_EXACT_SPLIT = 2

# Every symbol include/specverify.h declares.
EXPORTS = ["spec_weights_create", "spec_weights_destroy", "spec_workspace_size", "spec_verify",
           "spec_verify_debug", "spec_workspace_size_from_logits", "spec_verify_from_logits",
           "spec_status_string", "spec_default_mfma_min_rows", "spec_profile_enable",
           "spec_profile_read", "spec_stream_read", "spec_verify_noalloc",
           "spec_verify_tree_greedy", "spec_gamma_ctl_create", "spec_gamma_ctl_destroy",
           "spec_gamma_ctl_update", "spec_gamma_ctl_alpha", "spec_gamma_ctl_optimal", "spec_repack",
           "spec_attention_workspace_size", "spec_decode_attention", "spec_kv_commit"]
# Every symbol include/specverify_diag.h declares.
DIAG_EXPORTS = ["spec_diag_access_check"]


class SpecError(RuntimeError):
    def __init__(self, status, what):
        super().__init__(f"{what}: {status_string(status)} ({status})")
        self.status = status


class _Desc(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("ffn", ctypes.c_int32), ("n_blocks", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("wdtype", ctypes.c_int32), ("rms_eps", ctypes.c_float),
                ("w_up", ctypes.POINTER(ctypes.c_void_p)), ("w_down", ctypes.POINTER(ctypes.c_void_p)),
                ("norm_gain", ctypes.POINTER(ctypes.c_void_p)), ("lm_head", ctypes.c_void_p),
                ("flags", ctypes.c_uint32), ("mfma_min_rows", ctypes.c_int32)]


_lib = None


def load():
    """Load libspecverify.so (built by __graft_entry__.build())."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, f32, u64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_uint64, ctypes.c_size_t
    lib.spec_weights_create.argtypes = [ctypes.POINTER(_Desc), vp, ctypes.POINTER(vp)]
    lib.spec_weights_create.restype = i32
    lib.spec_weights_destroy.argtypes = [vp]
    lib.spec_weights_destroy.restype = i32
    lib.spec_workspace_size.argtypes = [vp, i32, i32]
    lib.spec_workspace_size.restype = sz
    common = [vp, i32, i32, vp, vp, vp, f32, f32, u64, vp, vp, vp, sz, vp]
    lib.spec_verify.argtypes = common
    lib.spec_verify.restype = i32
    lib.spec_verify_noalloc.argtypes = [vp, i32, i32, vp, vp, vp, f32, f32, u64, vp, vp, vp]
    lib.spec_verify_noalloc.restype = i32
    lib.spec_verify_tree_greedy.argtypes = [vp, i32, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp]
    lib.spec_verify_tree_greedy.restype = i32
    lib.spec_gamma_ctl_create.argtypes = [i32, i32, i32, i32, ctypes.c_double,
                                          ctypes.POINTER(ctypes.c_double), ctypes.POINTER(vp)]
    lib.spec_gamma_ctl_create.restype = i32
    lib.spec_gamma_ctl_destroy.argtypes = [vp]
    lib.spec_gamma_ctl_destroy.restype = i32
    ip = ctypes.POINTER(ctypes.c_int32)
    lib.spec_gamma_ctl_update.argtypes = [vp, ip, ip, ip]
    lib.spec_gamma_ctl_update.restype = i32
    lib.spec_gamma_ctl_alpha.argtypes = [vp, i32]
    lib.spec_gamma_ctl_alpha.restype = ctypes.c_double
    lib.spec_gamma_ctl_optimal.argtypes = [vp, ctypes.c_double]
    lib.spec_gamma_ctl_optimal.restype = i32
    lib.spec_repack.argtypes = [i32, i32] + [vp] * 8 + [vp]
    lib.spec_repack.restype = i32
    lib.spec_attention_workspace_size.argtypes = [i32] * 6
    lib.spec_attention_workspace_size.restype = sz
    lib.spec_decode_attention.argtypes = [i32] * 6 + [vp] * 5 + [f32, vp, vp, sz, vp]
    lib.spec_decode_attention.restype = i32
    lib.spec_kv_commit.argtypes = [i32] * 5 + [vp] * 6
    lib.spec_kv_commit.restype = i32
    lib.spec_verify_debug.argtypes = common + [vp, vp, vp]
    lib.spec_verify_debug.restype = i32
    lib.spec_workspace_size_from_logits.argtypes = [i32, i32, i32]
    lib.spec_workspace_size_from_logits.restype = sz
    lib.spec_verify_from_logits.argtypes = [i32, i32, i32, vp, vp, vp, f32, f32, u64, vp, vp, vp, sz, vp]
    lib.spec_verify_from_logits.restype = i32
    lib.spec_status_string.argtypes = [i32]
    lib.spec_status_string.restype = ctypes.c_char_p
    lib.spec_default_mfma_min_rows.argtypes = []
    lib.spec_default_mfma_min_rows.restype = i32
    lib.spec_profile_enable.argtypes = [vp, i32]
    lib.spec_profile_enable.restype = i32
    lib.spec_profile_read.argtypes = [vp, ctypes.POINTER(ctypes.c_double),
                                      ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64)]
    lib.spec_profile_read.restype = i32
    lib.spec_stream_read.argtypes = [vp, sz, vp, vp]
    lib.spec_stream_read.restype = i32
    lib.spec_diag_access_check.argtypes = [i32] * 6 + [ctypes.c_uint32] + [i32] * 3 + [
        ctypes.c_char_p, sz, ctypes.POINTER(ctypes.c_int64)]
    lib.spec_diag_access_check.restype = i32
    _lib = lib
    return lib


def status_string(status):
    return load().spec_status_string(int(status)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status, what):
    if status != SPEC_OK:
        raise SpecError(status, what)


def _dev(t, dtype, name):
    if not (t.is_cuda and t.dtype == dtype and t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous {dtype} device tensor")
    return t


class Weights:
    """Target weights registered with the library (it keeps its own copy).

    blocks: list of dicts with "w_up" [d][ffn], "w_down" [ffn][d] and an
    optional "gain" [d]; lm_head [d][V].  All tensors on the device, all
    torch.float32 or all torch.bfloat16.
    """

    def __init__(self, blocks, lm_head, eps=1e-6, keep_rowmajor=False, mfma_min_rows=0,
                 exact_split=False, stream=None):
        lib = load()
        dtype = lm_head.dtype
        if dtype not in (torch.float32, torch.bfloat16):
            raise ValueError("weights must be float32 or bfloat16")
        d, V = lm_head.shape
        ffn = blocks[0]["w_up"].shape[1] if blocks else 1
        for blk in blocks:
            _dev(blk["w_up"], dtype, "w_up")
            _dev(blk["w_down"], dtype, "w_down")
            if tuple(blk["w_up"].shape) != (d, ffn) or tuple(blk["w_down"].shape) != (ffn, d):
                raise ValueError("block shapes must be [d][ffn] and [ffn][d]")
        _dev(lm_head, dtype, "lm_head")
        n = len(blocks)
        gains = [blk.get("gain") for blk in blocks]
        if any(g is not None for g in gains) and any(g is None for g in gains):
            raise ValueError("give a gain for every block or for none")
        arr = ctypes.c_void_p * max(n, 1)
        self._up = arr(*[b["w_up"].data_ptr() for b in blocks])
        self._down = arr(*[b["w_down"].data_ptr() for b in blocks])
        self._gain = arr(*[_dev(g, dtype, "gain").data_ptr() for g in gains]) if n and gains[0] is not None else None
        desc = _Desc(int(d), int(ffn), n, int(V), SPEC_BF16 if dtype == torch.bfloat16 else SPEC_F32,
                     float(eps), ctypes.cast(self._up, ctypes.POINTER(ctypes.c_void_p)),
                     ctypes.cast(self._down, ctypes.POINTER(ctypes.c_void_p)),
                     ctypes.cast(self._gain, ctypes.POINTER(ctypes.c_void_p)) if self._gain is not None else None,
                     ctypes.c_void_p(lm_head.data_ptr()),
                     _flags(keep_rowmajor, exact_split), int(mfma_min_rows))
        handle = ctypes.c_void_p()
        _check(lib.spec_weights_create(ctypes.byref(desc), _stream(stream), ctypes.byref(handle)),
               "spec_weights_create")
        self.handle = handle
        self.d, self.ffn, self.n_blocks, self.V, self.dtype = int(d), int(ffn), n, int(V), dtype

    def close(self):
        if getattr(self, "handle", None):
            load().spec_weights_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def profile(self, on=True):
        """Bracket every GEMM launch with HIP events on its stream."""
        _check(load().spec_profile_enable(self.handle, 1 if on else 0), "spec_profile_enable")

    def profile_read(self):
        """(summed GEMM ms, GEMM launches, algorithmic weight bytes) since the last read."""
        ms, n, b = ctypes.c_double(), ctypes.c_int64(), ctypes.c_int64()
        _check(load().spec_profile_read(self.handle, ctypes.byref(ms), ctypes.byref(n),
                                        ctypes.byref(b)), "spec_profile_read")
        return ms.value, n.value, b.value

    def workspace_size(self, B, gamma):
        return int(load().spec_workspace_size(self.handle, int(B), int(gamma)))

    def workspace(self, B, gamma):
        n = self.workspace_size(B, gamma)
        if n == 0:
            raise SpecError(SPEC_EINVAL, "spec_workspace_size")
        return torch.empty(n, dtype=torch.uint8, device="cuda")


def _outputs(B, gamma, n_accepted, emitted):
    if n_accepted is None:
        n_accepted = torch.empty(B, dtype=torch.int32, device="cuda")
    if emitted is None:
        emitted = torch.empty((B, gamma + 1), dtype=torch.int32, device="cuda")
    return n_accepted, emitted


def verify(w, hidden, draft_tokens, q, temperature, top_p, seed, workspace=None,
           n_accepted=None, emitted=None, stream=None):
    """spec_verify; returns (n_accepted [B], emitted [B][gamma+1]) int32."""
    B, G1, d = hidden.shape
    gamma = G1 - 1
    _dev(hidden, torch.float32, "hidden")
    _dev(draft_tokens, torch.int32, "draft_tokens")
    if q is not None:
        _dev(q, torch.float32, "q")
    n_accepted, emitted = _outputs(B, gamma, n_accepted, emitted)
    if workspace is None:
        workspace = w.workspace(B, gamma)
    _check(load().spec_verify(w.handle, B, gamma, _ptr(hidden), _ptr(draft_tokens), _ptr(q),
                              float(temperature), float(top_p), int(seed), _ptr(n_accepted),
                              _ptr(emitted), _ptr(workspace), workspace.numel(), _stream(stream)),
           "spec_verify")
    return n_accepted, emitted


def verify_noalloc(w, hidden, draft_tokens, q, temperature, top_p, seed, n_accepted, emitted,
                   stream=None):
    """spec_verify_noalloc: the pass in the library's static scratch, into
    caller-allocated outputs n_accepted [B] and emitted [B][gamma+1]."""
    B, G1, d = hidden.shape
    gamma = G1 - 1
    _dev(hidden, torch.float32, "hidden")
    _dev(draft_tokens, torch.int32, "draft_tokens")
    if q is not None:
        _dev(q, torch.float32, "q")
    _dev(n_accepted, torch.int32, "n_accepted")
    _dev(emitted, torch.int32, "emitted")
    if tuple(n_accepted.shape) != (B,) or tuple(emitted.shape) != (B, G1):
        raise ValueError("outputs must be n_accepted [B] and emitted [B][gamma+1]")
    _check(load().spec_verify_noalloc(w.handle, B, gamma, _ptr(hidden), _ptr(draft_tokens), _ptr(q),
                                      float(temperature), float(top_p), int(seed), _ptr(n_accepted),
                                      _ptr(emitted), _stream(stream)),
           "spec_verify_noalloc")
    return n_accepted, emitted


def verify_debug(w, hidden, draft_tokens, q, temperature, top_p, seed, want_probs=True,
                 workspace=None, stream=None):
    """spec_verify_debug; returns (n_accepted, emitted, logits, p', q')."""
    B, G1, d = hidden.shape
    gamma = G1 - 1
    _dev(hidden, torch.float32, "hidden")
    _dev(draft_tokens, torch.int32, "draft_tokens")
    n_accepted, emitted = _outputs(B, gamma, None, None)
    logits = torch.empty((B, G1, w.V), dtype=torch.float32, device="cuda")
    tempered = want_probs and temperature > 0
    p_out = torch.empty((B, G1, w.V), dtype=torch.float32, device="cuda") if tempered else None
    q_out = torch.empty((B, gamma, w.V), dtype=torch.float32, device="cuda") if tempered else None
    if workspace is None:
        workspace = w.workspace(B, gamma)
    _check(load().spec_verify_debug(w.handle, B, gamma, _ptr(hidden), _ptr(draft_tokens), _ptr(q),
                                    float(temperature), float(top_p), int(seed), _ptr(n_accepted),
                                    _ptr(emitted), _ptr(workspace), workspace.numel(),
                                    _stream(stream), _ptr(logits), _ptr(p_out), _ptr(q_out)),
           "spec_verify_debug")
    return n_accepted, emitted, logits, p_out, q_out


def verify_tree_greedy(w, hidden, parent, tokens, want_logits=False, workspace=None, stream=None):
    """spec_verify_tree_greedy; hidden [B][n+1][d] (row 0 the root), parent
    and tokens [B][n] int32.  Returns (n_accepted [B], emitted [B][n+1],
    path [B][n], logits [B][n+1][V] or None)."""
    B, G1, d = hidden.shape
    n = G1 - 1
    _dev(hidden, torch.float32, "hidden")
    _dev(parent, torch.int32, "parent")
    _dev(tokens, torch.int32, "tokens")
    n_acc = torch.empty(B, dtype=torch.int32, device="cuda")
    emitted = torch.empty((B, G1), dtype=torch.int32, device="cuda")
    path = torch.empty((B, max(n, 1)), dtype=torch.int32, device="cuda")[:, :n]
    logits = torch.empty((B, G1, w.V), dtype=torch.float32, device="cuda") if want_logits else None
    if workspace is None:
        workspace = w.workspace(B, n)
    _check(load().spec_verify_tree_greedy(w.handle, B, n, _ptr(hidden), _ptr(parent), _ptr(tokens),
                                          _ptr(n_acc), _ptr(emitted), _ptr(path), _ptr(workspace),
                                          workspace.numel(), _stream(stream), _ptr(logits)),
           "spec_verify_tree_greedy")
    return n_acc, emitted, path, logits


class GammaController:
    """spec_gamma_ctl_*: per-sequence speculation-depth choice (host only).
    target_ms: verification time per pass for gamma = 0 .. gamma_max."""

    def __init__(self, n_seq, gamma_min, gamma_max, gamma_init, draft_ms_per_token, target_ms):
        lib = load()
        arr = (ctypes.c_double * len(target_ms))(*[float(x) for x in target_ms])
        if len(target_ms) <= gamma_max:
            raise ValueError("target_ms needs gamma_max + 1 entries")
        h = ctypes.c_void_p()
        _check(lib.spec_gamma_ctl_create(int(n_seq), int(gamma_min), int(gamma_max), int(gamma_init),
                                         float(draft_ms_per_token), arr, ctypes.byref(h)),
               "spec_gamma_ctl_create")
        self.handle, self.n_seq = h, int(n_seq)

    def update(self, n_accepted, gamma_used):
        n = (ctypes.c_int32 * self.n_seq)(*[int(x) for x in n_accepted])
        g = (ctypes.c_int32 * self.n_seq)(*[int(x) for x in gamma_used])
        out = (ctypes.c_int32 * self.n_seq)()
        _check(load().spec_gamma_ctl_update(self.handle, n, g, out), "spec_gamma_ctl_update")
        return list(out)

    def alpha(self, seq):
        return load().spec_gamma_ctl_alpha(self.handle, int(seq))

    def optimal(self, alpha):
        return load().spec_gamma_ctl_optimal(self.handle, float(alpha))

    def close(self):
        if getattr(self, "handle", None):
            load().spec_gamma_ctl_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def repack(n_accepted, emitted, committed, stream=None):
    """spec_repack on device tensors (committed is advanced in place).
    Returns (tokens, offsets, order, bin_offsets, stats) device tensors."""
    B, G1 = emitted.shape
    for t, name in ((n_accepted, "n_accepted"), (emitted, "emitted"), (committed, "committed")):
        _dev(t, torch.int32, name)
    z = lambda n: torch.empty(n, dtype=torch.int32, device="cuda")
    tokens, offsets, order, bins, stats = z(B * G1), z(B + 1), z(B), z(G1 + 2), z(2)
    _check(load().spec_repack(B, G1 - 1, _ptr(n_accepted), _ptr(emitted), _ptr(committed),
                              _ptr(tokens), _ptr(offsets), _ptr(order), _ptr(bins), _ptr(stats),
                              _stream(stream)), "spec_repack")
    return tokens, offsets, order, bins, stats


def _bf16_bits(t, name):
    if not (t.is_cuda and t.dtype == torch.bfloat16 and t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous bfloat16 device tensor")
    return t


def attention_workspace_size(B, n_new, H, Hkv, head_dim, max_seq):
    return int(load().spec_attention_workspace_size(B, n_new, H, Hkv, head_dim, max_seq))


def decode_attention(q, k_cache, v_cache, cache_len, parent=None, scale=None, out=None,
                     workspace=None, stream=None):
    """spec_decode_attention; q [B][n_new][H][hd] fp32, k_cache
    [B][Hkv][max_seq][hd] and v_cache [B][Hkv][hd][max_seq] bf16, cache_len
    [B] int32, parent [B][n_new] int32 or None (chain).  Returns out
    [B][n_new][H][hd] fp32."""
    B, n_new, H, hd = q.shape
    Hkv, max_seq = k_cache.shape[1], k_cache.shape[2]
    if tuple(v_cache.shape) != (B, Hkv, hd, max_seq):
        raise ValueError("v_cache must be [B][Hkv][hd][max_seq]")
    _dev(q, torch.float32, "q")
    _bf16_bits(k_cache, "k_cache")
    _bf16_bits(v_cache, "v_cache")
    _dev(cache_len, torch.int32, "cache_len")
    if parent is not None:
        _dev(parent, torch.int32, "parent")
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        n = attention_workspace_size(B, n_new, H, Hkv, hd, max_seq)
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")
    scale = 1.0 / hd ** 0.5 if scale is None else float(scale)
    _check(load().spec_decode_attention(B, n_new, H, Hkv, hd, max_seq, _ptr(q), _ptr(k_cache),
                                        _ptr(v_cache), _ptr(cache_len), _ptr(parent), scale,
                                        _ptr(out), _ptr(workspace), workspace.numel(),
                                        _stream(stream)), "spec_decode_attention")
    return out


def kv_commit(k_cache, v_cache, cache_len, n_accepted, n_new, path=None, stream=None):
    """spec_kv_commit (cache_len advanced in place, the caches gathered for a
    tree); k_cache [B][Hkv][max_seq][hd], v_cache [B][Hkv][hd][max_seq]."""
    B, Hkv, max_seq, hd = k_cache.shape
    _dev(cache_len, torch.int32, "cache_len")
    _dev(n_accepted, torch.int32, "n_accepted")
    if path is not None:
        _dev(path, torch.int32, "path")
    _check(load().spec_kv_commit(B, n_new, Hkv, hd, max_seq, _ptr(_bf16_bits(k_cache, "k_cache")),
                                 _ptr(_bf16_bits(v_cache, "v_cache")), _ptr(cache_len),
                                 _ptr(n_accepted), _ptr(path), _stream(stream)), "spec_kv_commit")


def workspace_size_from_logits(B, gamma, V):
    return int(load().spec_workspace_size_from_logits(int(B), int(gamma), int(V)))


def verify_from_logits(logits, draft_tokens, q, temperature, top_p, seed, workspace=None,
                       n_accepted=None, emitted=None, stream=None):
    """spec_verify_from_logits; logits [B][gamma+1][V] fp32 on the device."""
    B, G1, V = logits.shape
    gamma = G1 - 1
    _dev(logits, torch.float32, "logits")
    _dev(draft_tokens, torch.int32, "draft_tokens")
    if q is not None:
        _dev(q, torch.float32, "q")
    n_accepted, emitted = _outputs(B, gamma, n_accepted, emitted)
    if workspace is None:
        n = workspace_size_from_logits(B, gamma, V)
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")
    _check(load().spec_verify_from_logits(B, gamma, V, _ptr(logits), _ptr(draft_tokens), _ptr(q),
                                          float(temperature), float(top_p), int(seed),
                                          _ptr(n_accepted), _ptr(emitted), _ptr(workspace),
                                          workspace.numel(), _stream(stream)),
           "spec_verify_from_logits")
    return n_accepted, emitted


def stream_read(src, sink, nbytes=None, stream=None):
    """spec_stream_read over the first nbytes of the device tensor src."""
    nbytes = src.numel() * src.element_size() if nbytes is None else int(nbytes)
    _check(load().spec_stream_read(_ptr(src), nbytes, _ptr(sink), _stream(stream)),
           "spec_stream_read")


def _flags(keep_rowmajor, exact_split):
    return (SPEC_FLAG_KEEP_ROWMAJOR if keep_rowmajor else 0) | (SPEC_FLAG_EXACT_SPLIT if exact_split else 0)


def access_check(d, ffn, n_blocks, vocab, wdtype, B, gamma, mfma_min_rows=0, keep_rowmajor=False,
                 shrink_bytes=0, exact_split=False):
    """spec_diag_access_check: (status, message, ranges checked); host only."""
    buf = ctypes.create_string_buffer(512)
    n = ctypes.c_int64()
    st = load().spec_diag_access_check(int(d), int(ffn), int(n_blocks), int(vocab), int(wdtype),
                                       int(mfma_min_rows), _flags(keep_rowmajor, exact_split), int(B),
                                       int(gamma), int(shrink_bytes), buf, 512, ctypes.byref(n))
    return st, buf.value.decode(), n.value


def default_mfma_min_rows():
    return int(load().spec_default_mfma_min_rows())
