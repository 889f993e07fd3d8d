"""ctypes binding of libspecverify.so (C ABI in include/spec_verify.h).

Argument marshalling only: every function forwards device pointers
(``tensor.data_ptr()``), sizes and the HIP stream handle to the C ABI of the
same name, and raises ``SpecVerifyError`` on a negative status. All the work
runs in the library's HIP kernels; there is no CPU fallback, and loading fails
loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

import torch

# SPEC_VERIFY_LIB selects another build of the same sources (for instance the
# host-sanitizer build of the test suite).
LIB_PATH = os.environ.get("SPEC_VERIFY_LIB") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libspecverify.so")

SPEC_F32 = 0
SPEC_BF16 = 1
SPEC_OK = 0
SPEC_EINVAL = -1
SPEC_EHIP = -2
SPEC_ENOMEM = -3
SPEC_ESTATE = -4
SPEC_ESCRATCH = -5
SPEC_VERIFY_NOALLOC_SCRATCH_BYTES = 16 << 20

EXPORTED = (
    "spec_verify_init", "spec_verify_set_stream", "spec_verify", "spec_verify_offset_ptr",
    "spec_accept_logprobs",
    "spec_verify_copy_lse", "spec_verify_philox_words", "spec_verify_enable_timing",
    "spec_verify_read_timing", "spec_verify_get_geometry", "spec_verify_destroy",
    "spec_verify_strerror", "spec_verify_outcomes", "spec_outcome_fanout",
    "spec_bandit_init", "spec_bandit_set_stream", "spec_bandit_step", "spec_bandit_get_state",
    "spec_bandit_set_state", "spec_bandit_destroy",
    "spec_lowrank_head_init", "spec_lowrank_head_set_stream", "spec_lowrank_head",
    "spec_lowrank_head_copy_activation", "spec_lowrank_head_destroy",
    "spec_tree_prune", "spec_tree_verify_init", "spec_tree_verify_set_stream",
    "spec_tree_verify_greedy", "spec_tree_verify_sample", "spec_tree_verify_destroy",
    "spec_tree_verify_gave_up", "spec_tree_verify_set_spin_limit",
    "spec_verify_noalloc", "spec_hbm_read_probe",
)

SPEC_TREE_MAX_NODES = 256

SPEC_OUTCOME_MAX_F = 64
SPEC_FANOUT_MAX_LENGTHS = 256
SPEC_BANDIT_UCB1 = 0
SPEC_BANDIT_THOMPSON = 1
SPEC_BANDIT_MAX_ARMS = 64


class SpecVerifyError(RuntimeError):
    def __init__(self, func: str, code: int):
        self.code = code
        super().__init__(f"{func} failed: {code} ({_strerror(code)})")


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (raises if it is missing: there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(path)
    P, i32, u64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64
    sig = {
        "spec_verify_init": ([i32, i32, i32, i32, P, ctypes.POINTER(P)], i32),
        "spec_verify_set_stream": ([P, P], i32),
        "spec_verify": ([P, P, P, P, P, u64, u64, P, P], i32),
        "spec_verify_offset_ptr": ([P, P, P, P, P, u64, P, P, P], i32),
        "spec_verify_noalloc": ([i32, i32, i32, i32, P, P, P, P, P, u64, u64, P, P], i32),
        "spec_hbm_read_probe": ([P, u64, P, i32, P], i32),
        "spec_accept_logprobs": ([P, P, u64, u64, P], i32),
        "spec_verify_copy_lse": ([P, P], i32),
        "spec_verify_philox_words": ([P, u64, u64, P], i32),
        "spec_verify_enable_timing": ([P, i32], i32),
        "spec_verify_read_timing": ([P, P, i32], i32),
        "spec_verify_get_geometry": ([P, P], i32),
        "spec_verify_destroy": ([P], i32),
        "spec_verify_strerror": ([i32], ctypes.c_char_p),
        "spec_verify_outcomes": ([P, P, P, P, i32, P, P, P, P], i32),
        "spec_outcome_fanout": ([i32, i32, i32, P, P, i32, P, P, P], i32),
        "spec_bandit_init": ([i32, i32, i32, i32, i32, P, ctypes.POINTER(P)], i32),
        "spec_bandit_set_stream": ([P, P], i32),
        "spec_bandit_step": ([P, P, P, u64, u64, P], i32),
        "spec_bandit_get_state": ([P, P, P], i32),
        "spec_bandit_set_state": ([P, P, P], i32),
        "spec_bandit_destroy": ([P], i32),
        "spec_lowrank_head_init": ([i32, i32, i32, i32, P, ctypes.POINTER(P)], i32),
        "spec_lowrank_head_set_stream": ([P, P], i32),
        "spec_lowrank_head": ([P, P, P, P, P, P, P], i32),
        "spec_lowrank_head_copy_activation": ([P, P], i32),
        "spec_lowrank_head_destroy": ([P], i32),
        "spec_tree_prune": ([i32, i32, P, P, ctypes.c_double, i32, P, P, P, P, P], i32),
        "spec_tree_verify_init": ([i32, i32, i32, i32, P, ctypes.POINTER(P)], i32),
        "spec_tree_verify_set_stream": ([P, P], i32),
        "spec_tree_verify_greedy": ([P, P, P, P, P, P, P, P], i32),
        "spec_tree_verify_sample": ([P, P, P, P, P, P, P, u64, u64, P, P, P], i32),
        "spec_tree_verify_destroy": ([P], i32),
        "spec_tree_verify_gave_up": ([P, ctypes.POINTER(u64)], i32),
        "spec_tree_verify_set_spin_limit": ([P, i32], i32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _strerror(code: int) -> str:
    try:
        return load_library().spec_verify_strerror(code).decode()
    except Exception:  # pragma: no cover - library missing
        return "unknown"


def _check(func: str, rc: int) -> int:
    if rc < 0:
        raise SpecVerifyError(func, rc)
    return rc


def _ptr(t: torch.Tensor | None):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the verification library must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream_handle(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def dtype_code(dtype: torch.dtype) -> int:
    if dtype == torch.bfloat16:
        return SPEC_BF16
    if dtype == torch.float32:
        return SPEC_F32
    raise TypeError(f"logits must be bfloat16 or float32, got {dtype}")


class Context:
    """Owns a spec_verify_ctx*; destroyed with spec_verify_destroy."""

    def __init__(self, handle: ctypes.c_void_p, batch: int, gamma: int, vocab: int, dtype: int):
        self.handle = handle
        self.batch, self.gamma, self.vocab, self.dtype = batch, gamma, vocab, dtype

    def __del__(self):
        if getattr(self, "handle", None):
            try:
                load_library().spec_verify_destroy(self.handle)
            except Exception:
                pass
            self.handle = None


def spec_verify_init(batch: int, gamma: int, vocab: int, dtype, stream=None) -> Context:
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)
    h = ctypes.c_void_p()
    _check("spec_verify_init", load_library().spec_verify_init(
        batch, gamma, vocab, code, _stream_handle(stream), ctypes.byref(h)))
    return Context(h, batch, gamma, vocab, code)


def spec_verify_set_stream(ctx: Context, stream=None) -> None:
    _check("spec_verify_set_stream",
           load_library().spec_verify_set_stream(ctx.handle, _stream_handle(stream)))


def _expect(t, shape, dtype, name):
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")


def spec_verify(ctx: Context, logits_draft, logits_target, draft_tokens, temperature,
                seed: int, offset: int, out_accept_len, out_tokens) -> None:
    B, G, V = ctx.batch, ctx.gamma, ctx.vocab
    ldt = torch.bfloat16 if ctx.dtype == SPEC_BF16 else torch.float32
    if G > 0:
        _expect(logits_draft, (B, G, V), ldt, "logits_draft")
        _expect(draft_tokens, (B, G), torch.int32, "draft_tokens")
    _expect(logits_target, (B, G + 1, V), ldt, "logits_target")
    _expect(temperature, (B,), torch.float32, "temperature")
    _expect(out_accept_len, (B,), torch.int32, "out_accept_len")
    _expect(out_tokens, (B, G + 1), torch.int32, "out_tokens")
    _check("spec_verify", load_library().spec_verify(
        ctx.handle, _ptr(logits_draft) if G > 0 else None, _ptr(logits_target),
        _ptr(draft_tokens) if G > 0 else None, _ptr(temperature), seed, offset,
        _ptr(out_accept_len), _ptr(out_tokens)))


def spec_verify_offset_ptr(ctx: Context, logits_draft, logits_target, draft_tokens, temperature,
                           seed: int, offset_dev, out_accept_len, out_tokens) -> None:
    """spec_verify with the Philox offset read on the device from offset_dev, a
    one-element int64 (or uint64) device tensor holding the offset's bits."""
    B, G, V = ctx.batch, ctx.gamma, ctx.vocab
    ldt = torch.bfloat16 if ctx.dtype == SPEC_BF16 else torch.float32
    if G > 0:
        _expect(logits_draft, (B, G, V), ldt, "logits_draft")
        _expect(draft_tokens, (B, G), torch.int32, "draft_tokens")
    _expect(logits_target, (B, G + 1, V), ldt, "logits_target")
    _expect(temperature, (B,), torch.float32, "temperature")
    _expect(out_accept_len, (B,), torch.int32, "out_accept_len")
    _expect(out_tokens, (B, G + 1), torch.int32, "out_tokens")
    if offset_dev is None or offset_dev.numel() != 1 or offset_dev.element_size() != 8 \
            or offset_dev.device.type != "cuda":
        raise ValueError("offset_dev must be a one-element 64-bit device tensor")
    _check("spec_verify_offset_ptr", load_library().spec_verify_offset_ptr(
        ctx.handle, _ptr(logits_draft) if G > 0 else None, _ptr(logits_target),
        _ptr(draft_tokens) if G > 0 else None, _ptr(temperature), seed, _ptr(offset_dev),
        _ptr(out_accept_len), _ptr(out_tokens)))


def spec_verify_noalloc(logits_draft, logits_target, draft_tokens, temperature, seed: int,
                        offset: int, out_accept_len, out_tokens, stream=None) -> int:
    """spec_verify without a context, working in the library's fixed device
    scratch array (no allocation). Shapes come from logits_target [B, G+1, V].
    Returns the C status (SPEC_OK, or SPEC_ESCRATCH when the shape's workspace
    exceeds the array); raises on other errors."""
    B, G1, V = logits_target.shape
    G = G1 - 1
    ldt = logits_target.dtype
    if G > 0:
        _expect(logits_draft, (B, G, V), ldt, "logits_draft")
        _expect(draft_tokens, (B, G), torch.int32, "draft_tokens")
    _expect(temperature, (B,), torch.float32, "temperature")
    _expect(out_accept_len, (B,), torch.int32, "out_accept_len")
    _expect(out_tokens, (B, G + 1), torch.int32, "out_tokens")
    rc = load_library().spec_verify_noalloc(
        B, G, V, dtype_code(ldt), _stream_handle(stream),
        _ptr(logits_draft) if G > 0 else None, _ptr(logits_target),
        _ptr(draft_tokens) if G > 0 else None, _ptr(temperature), seed, offset,
        _ptr(out_accept_len), _ptr(out_tokens))
    if rc not in (SPEC_OK, SPEC_ESCRATCH):
        _check("spec_verify_noalloc", rc)
    return rc


def spec_hbm_read_probe(buf, sink, blocks: int, stream=None) -> None:
    """Read-only HBM probe over the bytes of device tensor buf (measurement
    utility); sink is an int32/uint32 device tensor of at least `blocks` words."""
    if buf.device.type != "cuda" or sink.device.type != "cuda" or sink.numel() < blocks:
        raise ValueError("buf and sink must be device tensors, sink of at least `blocks` words")
    nbytes = buf.numel() * buf.element_size()
    _check("spec_hbm_read_probe", load_library().spec_hbm_read_probe(
        _ptr(buf), nbytes, _ptr(sink), int(blocks), _stream_handle(stream)))


def spec_accept_logprobs(ctx: Context, logprobs, seed: int, offset: int, out_accept_len) -> None:
    B, G = ctx.batch, ctx.gamma
    _expect(logprobs, (B, G, 2), torch.float32, "logprobs")
    _expect(out_accept_len, (B,), torch.int32, "out_accept_len")
    _check("spec_accept_logprobs", load_library().spec_accept_logprobs(
        ctx.handle, _ptr(logprobs), seed, offset, _ptr(out_accept_len)))


def spec_verify_outcomes(ctx: Context, logits_draft, logits_target, draft_tokens, top_f: int,
                         out_tokens, out_probs, out_pk, out_mass=None) -> None:
    """Law of the last verification's outcome (call after spec_verify with the
    same inputs): out_tokens [B, G+1, F] int32, out_probs [B, G+1, F] float32,
    out_pk [B, G+1] float32, out_mass [B, G+1] float32 or None."""
    B, G, V = ctx.batch, ctx.gamma, ctx.vocab
    ldt = torch.bfloat16 if ctx.dtype == SPEC_BF16 else torch.float32
    if G > 0:
        _expect(logits_draft, (B, G, V), ldt, "logits_draft")
        _expect(draft_tokens, (B, G), torch.int32, "draft_tokens")
    _expect(logits_target, (B, G + 1, V), ldt, "logits_target")
    _expect(out_tokens, (B, G + 1, top_f), torch.int32, "out_tokens")
    _expect(out_probs, (B, G + 1, top_f), torch.float32, "out_probs")
    _expect(out_pk, (B, G + 1), torch.float32, "out_pk")
    _expect(out_mass, (B, G + 1), torch.float32, "out_mass")
    _check("spec_verify_outcomes", load_library().spec_verify_outcomes(
        ctx.handle, _ptr(logits_draft) if G > 0 else None, _ptr(logits_target),
        _ptr(draft_tokens) if G > 0 else None, top_f, _ptr(out_tokens), _ptr(out_probs),
        _ptr(out_pk), _ptr(out_mass)))


def spec_outcome_fanout(pk, probs, budget: int, out_n, out_hit=None, stream=None) -> None:
    """Speculation-cache entries per length for `budget` entries per sequence:
    pk [B, L] float32 and probs [B, L, F] float32 (spec_verify_outcomes'
    out_pk and out_probs); out_n [B, L] int32, out_hit [B] float64 or None."""
    B, L = pk.shape
    F = probs.shape[2]
    _expect(pk, (B, L), torch.float32, "pk")
    _expect(probs, (B, L, F), torch.float32, "probs")
    _expect(out_n, (B, L), torch.int32, "out_n")
    _expect(out_hit, (B,), torch.float64, "out_hit")
    _check("spec_outcome_fanout", load_library().spec_outcome_fanout(
        B, L, F, _ptr(pk), _ptr(probs), int(budget), _ptr(out_n), _ptr(out_hit),
        _stream_handle(stream)))


def spec_verify_copy_lse(ctx: Context, out_lse) -> None:
    _expect(out_lse, (ctx.batch, 2 * ctx.gamma + 1), torch.float64, "out_lse")
    _check("spec_verify_copy_lse", load_library().spec_verify_copy_lse(ctx.handle, _ptr(out_lse)))


def spec_verify_philox_words(ctx: Context, seed: int, offset: int, out_words) -> None:
    _expect(out_words, (ctx.batch, ctx.gamma + 1, 4), torch.int32, "out_words")
    _check("spec_verify_philox_words",
           load_library().spec_verify_philox_words(ctx.handle, seed, offset, _ptr(out_words)))


def spec_verify_enable_timing(ctx: Context, max_calls: int) -> None:
    _check("spec_verify_enable_timing", load_library().spec_verify_enable_timing(ctx.handle, max_calls))


def spec_verify_read_timing(ctx: Context, max_calls: int):
    """Per-call kernel durations in ms: list of (row_norm, accept, residual)."""
    buf = (ctypes.c_float * (3 * max(max_calls, 1)))()
    n = _check("spec_verify_read_timing",
               load_library().spec_verify_read_timing(ctx.handle, buf, max_calls))
    return [(buf[3 * i], buf[3 * i + 1], buf[3 * i + 2]) for i in range(n)]


def spec_verify_get_geometry(ctx: Context) -> dict:
    out = (ctypes.c_int * 3)()
    _check("spec_verify_get_geometry", load_library().spec_verify_get_geometry(ctx.handle, out))
    return dict(row_splits=out[0], residual_splits=out[1], block=out[2])


def spec_verify_destroy(ctx: Context) -> None:
    if ctx.handle:
        rc = load_library().spec_verify_destroy(ctx.handle)
        ctx.handle = None
        _check("spec_verify_destroy", rc)


def spec_verify_strerror(code: int) -> str:
    return _strerror(code)


class BanditContext:
    """Owns a spec_bandit_ctx*; destroyed with spec_bandit_destroy."""

    def __init__(self, handle: ctypes.c_void_p, groups: int, arms: int, batch: int, gamma: int,
                 policy: int):
        self.handle = handle
        self.groups, self.arms, self.batch, self.gamma, self.policy = groups, arms, batch, gamma, policy

    def __del__(self):
        if getattr(self, "handle", None):
            try:
                load_library().spec_bandit_destroy(self.handle)
            except Exception:
                pass
            self.handle = None


def spec_bandit_init(groups: int, arms: int, batch: int, gamma: int, policy: int,
                     stream=None) -> BanditContext:
    h = ctypes.c_void_p()
    _check("spec_bandit_init", load_library().spec_bandit_init(
        groups, arms, batch, gamma, policy, _stream_handle(stream), ctypes.byref(h)))
    return BanditContext(h, groups, arms, batch, gamma, policy)


def spec_bandit_set_stream(ctx: BanditContext, stream=None) -> None:
    _check("spec_bandit_set_stream",
           load_library().spec_bandit_set_stream(ctx.handle, _stream_handle(stream)))


def spec_bandit_step(ctx: BanditContext, accept_len, arm_played, seed: int, offset: int,
                     out_arm) -> None:
    """accept_len [B] / arm_played [G] int32 device tensors (both None for the
    first choice); out_arm [G] int32 device tensor (may be arm_played)."""
    if accept_len is not None:
        _expect(accept_len, (ctx.batch,), torch.int32, "accept_len")
        _expect(arm_played, (ctx.groups,), torch.int32, "arm_played")
    _expect(out_arm, (ctx.groups,), torch.int32, "out_arm")
    _check("spec_bandit_step", load_library().spec_bandit_step(
        ctx.handle, _ptr(accept_len), _ptr(arm_played) if accept_len is not None else None,
        seed, offset, _ptr(out_arm)))


def spec_bandit_get_state(ctx: BanditContext):
    """(counts [G, K] uint32, sums [G, K] float64) as host numpy arrays."""
    import numpy as np
    counts = np.zeros((ctx.groups, ctx.arms), np.uint32)
    sums = np.zeros((ctx.groups, ctx.arms), np.float64)
    _check("spec_bandit_get_state", load_library().spec_bandit_get_state(
        ctx.handle, counts.ctypes.data, sums.ctypes.data))
    return counts, sums


def spec_bandit_set_state(ctx: BanditContext, counts=None, sums=None) -> None:
    """Restore a saved state (host arrays [G, K]); no arguments resets to zero."""
    import numpy as np
    if counts is None and sums is None:
        _check("spec_bandit_set_state", load_library().spec_bandit_set_state(ctx.handle, None, None))
        return
    c = np.ascontiguousarray(counts, np.uint32).reshape(ctx.groups, ctx.arms)
    s = np.ascontiguousarray(sums, np.float64).reshape(ctx.groups, ctx.arms)
    _check("spec_bandit_set_state", load_library().spec_bandit_set_state(
        ctx.handle, c.ctypes.data, s.ctypes.data))


def spec_bandit_destroy(ctx: BanditContext) -> None:
    if ctx.handle:
        rc = load_library().spec_bandit_destroy(ctx.handle)
        ctx.handle = None
        _check("spec_bandit_destroy", rc)


class HeadContext:
    """Owns a spec_head_ctx*; destroyed with spec_lowrank_head_destroy."""

    def __init__(self, handle: ctypes.c_void_p, rows: int, hidden: int, rank: int, vocab: int):
        self.handle = handle
        self.rows, self.hidden, self.rank, self.vocab = rows, hidden, rank, vocab

    def __del__(self):
        if getattr(self, "handle", None):
            try:
                load_library().spec_lowrank_head_destroy(self.handle)
            except Exception:
                pass
            self.handle = None


def _bf16_like(t, shape, name):
    """bf16 tensors may be passed as torch.bfloat16 or as their int16 bits."""
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype not in (torch.bfloat16, torch.int16):
        raise TypeError(f"{name}: dtype {t.dtype}, expected bfloat16 (or int16 bits)")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")


def spec_lowrank_head_init(rows: int, hidden: int, rank: int, vocab: int, stream=None) -> HeadContext:
    h = ctypes.c_void_p()
    _check("spec_lowrank_head_init", load_library().spec_lowrank_head_init(
        rows, hidden, rank, vocab, _stream_handle(stream), ctypes.byref(h)))
    return HeadContext(h, rows, hidden, rank, vocab)


def spec_lowrank_head_set_stream(ctx: HeadContext, stream=None) -> None:
    _check("spec_lowrank_head_set_stream",
           load_library().spec_lowrank_head_set_stream(ctx.handle, _stream_handle(stream)))


def spec_lowrank_head(ctx: HeadContext, hidden, w_down, w_up, temperature, out_logits, out_lse) -> None:
    """hidden [N, d], w_down [r, d], w_up [V, r], out_logits [N, V] bf16;
    temperature [N] float32; out_lse [N] float64."""
    N, d, r, V = ctx.rows, ctx.hidden, ctx.rank, ctx.vocab
    _bf16_like(hidden, (N, d), "hidden")
    _bf16_like(w_down, (r, d), "w_down")
    _bf16_like(w_up, (V, r), "w_up")
    _bf16_like(out_logits, (N, V), "out_logits")
    _expect(temperature, (N,), torch.float32, "temperature")
    _expect(out_lse, (N,), torch.float64, "out_lse")
    _check("spec_lowrank_head", load_library().spec_lowrank_head(
        ctx.handle, _ptr(hidden), _ptr(w_down), _ptr(w_up), _ptr(temperature),
        _ptr(out_logits), _ptr(out_lse)))


def spec_lowrank_head_copy_activation(ctx: HeadContext, out_u) -> None:
    _bf16_like(out_u, (ctx.rows, ctx.rank), "out_u")
    _check("spec_lowrank_head_copy_activation",
           load_library().spec_lowrank_head_copy_activation(ctx.handle, _ptr(out_u)))


def spec_lowrank_head_destroy(ctx: HeadContext) -> None:
    if ctx.handle:
        rc = load_library().spec_lowrank_head_destroy(ctx.handle)
        ctx.handle = None
        _check("spec_lowrank_head_destroy", rc)


def spec_tree_prune(parent, logq, tau: float, budget: int, out_cum, out_new_index, out_new_parent,
                    out_count, stream=None) -> None:
    """parent [B, M] int32, logq [B, M] float32; outputs out_cum [B, M] float64,
    out_new_index / out_new_parent [B, M] int32, out_count [B] int32."""
    B, M = parent.shape
    _expect(parent, (B, M), torch.int32, "parent")
    _expect(logq, (B, M), torch.float32, "logq")
    _expect(out_cum, (B, M), torch.float64, "out_cum")
    _expect(out_new_index, (B, M), torch.int32, "out_new_index")
    _expect(out_new_parent, (B, M), torch.int32, "out_new_parent")
    _expect(out_count, (B,), torch.int32, "out_count")
    _check("spec_tree_prune", load_library().spec_tree_prune(
        B, M, _ptr(parent), _ptr(logq), float(tau), int(budget), _ptr(out_cum),
        _ptr(out_new_index), _ptr(out_new_parent), _ptr(out_count), _stream_handle(stream)))


class TreeContext:
    """Owns a spec_tree_ctx*; destroyed with spec_tree_verify_destroy."""

    def __init__(self, handle: ctypes.c_void_p, batch: int, max_nodes: int, vocab: int, dtype: int):
        self.handle = handle
        self.batch, self.max_nodes, self.vocab, self.dtype = batch, max_nodes, vocab, dtype

    def __del__(self):
        if getattr(self, "handle", None):
            try:
                load_library().spec_tree_verify_destroy(self.handle)
            except Exception:
                pass
            self.handle = None


def spec_tree_verify_init(batch: int, max_nodes: int, vocab: int, dtype, stream=None) -> TreeContext:
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)
    h = ctypes.c_void_p()
    _check("spec_tree_verify_init", load_library().spec_tree_verify_init(
        batch, max_nodes, vocab, code, _stream_handle(stream), ctypes.byref(h)))
    return TreeContext(h, batch, max_nodes, vocab, code)


def spec_tree_verify_set_stream(ctx: TreeContext, stream=None) -> None:
    _check("spec_tree_verify_set_stream",
           load_library().spec_tree_verify_set_stream(ctx.handle, _stream_handle(stream)))


def spec_tree_verify_greedy(ctx: TreeContext, parent, token, n_nodes, target, out_length,
                            out_path, out_extra) -> None:
    B, M, V = ctx.batch, ctx.max_nodes, ctx.vocab
    ldt = torch.bfloat16 if ctx.dtype == SPEC_BF16 else torch.float32
    _expect(parent, (B, M), torch.int32, "parent")
    _expect(token, (B, M), torch.int32, "token")
    _expect(n_nodes, (B,), torch.int32, "n_nodes")
    _expect(target, (B, M, V), ldt, "target")
    _expect(out_length, (B,), torch.int32, "out_length")
    _expect(out_path, (B, M), torch.int32, "out_path")
    _expect(out_extra, (B,), torch.int32, "out_extra")
    _check("spec_tree_verify_greedy", load_library().spec_tree_verify_greedy(
        ctx.handle, _ptr(parent), _ptr(token), _ptr(n_nodes), _ptr(target), _ptr(out_length),
        _ptr(out_path), _ptr(out_extra)))


def spec_tree_verify_sample(ctx: TreeContext, parent, token, n_nodes, draft, target, temperature,
                            seed: int, offset: int, out_length, out_path, out_extra) -> None:
    B, M, V = ctx.batch, ctx.max_nodes, ctx.vocab
    ldt = torch.bfloat16 if ctx.dtype == SPEC_BF16 else torch.float32
    _expect(parent, (B, M), torch.int32, "parent")
    _expect(token, (B, M), torch.int32, "token")
    _expect(n_nodes, (B,), torch.int32, "n_nodes")
    _expect(draft, (B, M, V), ldt, "draft")
    _expect(target, (B, M, V), ldt, "target")
    _expect(temperature, (B,), torch.float32, "temperature")
    _expect(out_length, (B,), torch.int32, "out_length")
    _expect(out_path, (B, M), torch.int32, "out_path")
    _expect(out_extra, (B,), torch.int32, "out_extra")
    _check("spec_tree_verify_sample", load_library().spec_tree_verify_sample(
        ctx.handle, _ptr(parent), _ptr(token), _ptr(n_nodes), _ptr(draft), _ptr(target),
        _ptr(temperature), seed, offset, _ptr(out_length), _ptr(out_path), _ptr(out_extra)))


def spec_tree_verify_gave_up(ctx: TreeContext) -> int:
    """Trees reported with length -2 by the sampled calls on ctx so far (syncs its stream)."""
    n = ctypes.c_uint64(0)
    _check("spec_tree_verify_gave_up",
           load_library().spec_tree_verify_gave_up(ctx.handle, ctypes.byref(n)))
    return n.value


def spec_tree_verify_set_spin_limit(ctx: TreeContext, polls: int) -> None:
    """Test hook: polls before a part gives up waiting for a partner."""
    _check("spec_tree_verify_set_spin_limit",
           load_library().spec_tree_verify_set_spin_limit(ctx.handle, int(polls)))


def spec_tree_verify_destroy(ctx: TreeContext) -> None:
    if ctx.handle:
        rc = load_library().spec_tree_verify_destroy(ctx.handle)
        ctx.handle = None
        _check("spec_tree_verify_destroy", rc)
