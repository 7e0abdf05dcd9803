"""Python binding of libdraft_attn.so (MI355X draft-head decode attention).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/draft_attn.h. PyTorch supplies
device memory and the current stream. There is no fallback: if the library is
missing, importing the binding raises.
"""

from __future__ import annotations

import ctypes
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdraft_attn.so")

FULL, WINDOW, FOLD = 0, 1, 2
ROPE_NEOX, ROPE_NONE = 0, 1
OK, EINVAL, ENOSPC, EHIP, ENOTSUP = 0, -1, -2, -3, -4
MAX_ROWS = 32
ABI_VERSION = 4
PLAN_ITEM_INTS = 7
_MODES = {"full": FULL, "window": WINDOW, "fold": FOLD}
_ROPES = {"neox": ROPE_NEOX, "none": ROPE_NONE}
FOLD_B, FOLD_JOINT, FOLD_VIRTUAL = 0, 1, 2
_FOLD_VARIANTS = {"B": FOLD_B, "A": FOLD_JOINT, "B'": FOLD_VIRTUAL}
LAUNCH_AUTO, LAUNCH_TWO_PASS, LAUNCH_SINGLE = 0, 1, 2
_LAUNCHES = {"auto": LAUNCH_AUTO, "two_pass": LAUNCH_TWO_PASS, "single": LAUNCH_SINGLE}
OUT_F32, OUT_BF16 = 0, 1
_OUT_DTYPES = {"f32": OUT_F32, "bf16": OUT_BF16}
MAX_GROUP_ITEMS = 64
NOALLOC_SCRATCH_BYTES = 16 << 20
STATUS_BAD_BLOCK, STATUS_LENGTHS, STATUS_APPEND_BAD_BLOCK = 1, 2, 4


class Params(ctypes.Structure):
    """Mirror of draft_attn_params (field order and types must match the header)."""
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("num_seqs", ctypes.c_int32),
        ("num_draft_tokens", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("mode", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("n_sink", ctypes.c_int32),
        ("n0", ctypes.c_int32),
        ("rope", ctypes.c_int32),
        ("alpha", ctypes.c_float),
        ("beta", ctypes.c_float),
        ("kappa", ctypes.c_float),
        ("softmax_scale", ctypes.c_float),
        ("rope_theta", ctypes.c_double),
        ("debug_visit", ctypes.c_void_p),
        ("debug_visit_stride", ctypes.c_int64),
        ("prof_events", ctypes.c_void_p * 2),
        ("split_keys", ctypes.c_int32),
        ("fold_variant", ctypes.c_int32),
        ("launch", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
        ("status_flags", ctypes.c_void_p),
    ]


class AppendParams(ctypes.Structure):
    """Mirror of draft_attn_append_params."""
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("num_seqs", ctypes.c_int32),
        ("num_new", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("rope", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("rope_theta", ctypes.c_double),
        ("status_flags", ctypes.c_void_p),
    ]


class DraftAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {strerror(status)} (status {status})")
        self.status = status


def _load():
    # torch and this library must share one HIP runtime (both bind the soname
    # libamdhip64.so.7): load torch's copy first when torch is installed.
    try:
        import torch  # noqa: F401
    except ImportError:  # pragma: no cover
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                          "or python draft_attention_amd/build.py")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(Params)
    vp, i32p = ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32)
    lib.draft_attn_params_init.argtypes = [P]
    lib.draft_attn_params_init.restype = None
    lib.draft_attn_workspace_size.argtypes = [P, i32p, ctypes.POINTER(ctypes.c_size_t)]
    lib.draft_attn_workspace_size.restype = ctypes.c_int
    lib.draft_attn_decode.argtypes = [P, vp, vp, vp, vp, vp, vp, i32p, vp, vp, vp, ctypes.c_size_t, vp]
    lib.draft_attn_decode.restype = ctypes.c_int
    lib.draft_attn_decode_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, i32p, vp, vp, vp]
    lib.draft_attn_decode_noalloc.restype = ctypes.c_int
    lib.draft_attn_launch_floor.argtypes = [P, i32p, ctypes.c_int32, vp]
    lib.draft_attn_launch_floor.restype = ctypes.c_int
    lib.draft_attn_decode_draft.argtypes = [P, vp, vp, vp, vp, vp, vp, i32p, vp, vp, vp, vp, vp, ctypes.c_size_t,
                                            vp]
    lib.draft_attn_decode_draft.restype = ctypes.c_int
    lib.draft_attn_plan.argtypes = [P, i32p, i32p, ctypes.c_int64, ctypes.POINTER(ctypes.c_int64), i32p, i32p]
    lib.draft_attn_plan.restype = ctypes.c_int
    lib.draft_attn_merge_draft.argtypes = [P, vp, vp, vp, vp, i32p, vp, vp, vp]
    lib.draft_attn_merge_draft.restype = ctypes.c_int
    lib.draft_attn_ring_size.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, i32p, i32p]
    lib.draft_attn_ring_size.restype = ctypes.c_int
    lib.draft_attn_ring_table.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, i32p,
                                          ctypes.c_int32, i32p, ctypes.c_int32, i32p, ctypes.c_int32]
    lib.draft_attn_ring_table.restype = ctypes.c_int
    AP = ctypes.POINTER(AppendParams)
    lib.draft_attn_append_params_init.argtypes = [AP]
    lib.draft_attn_append_params_init.restype = None
    lib.draft_attn_append.argtypes = [AP, vp, vp, vp, vp, i32p, vp, vp, vp, vp]
    lib.draft_attn_append.restype = ctypes.c_int
    lib.draft_attn_strerror.argtypes = [ctypes.c_int]
    lib.draft_attn_strerror.restype = ctypes.c_char_p
    lib.draft_attn_version.argtypes = []
    lib.draft_attn_version.restype = ctypes.c_int
    if lib.draft_attn_version() != ABI_VERSION:
        raise ImportError("libdraft_attn.so ABI version mismatch")
    if ctypes.sizeof(Params) != 136 or ctypes.sizeof(AppendParams) != 56:
        raise ImportError("params mirror has the wrong size")
    return lib


lib = _load()


def strerror(status: int) -> str:
    return lib.draft_attn_strerror(int(status)).decode()


def make_params(*, num_seqs, num_draft_tokens, num_q_heads, num_kv_heads, head_dim, num_blocks,
                max_blocks_per_seq, mode="full", window=0, n_sink=0, alpha=1.0, beta=0.0, kappa=0.0,
                n0=1, softmax_scale=None, rope="neox", rope_theta=1e4, split_keys=0,
                debug_visit=0, debug_visit_stride=0, prof_events=None, fold_variant="B", launch="auto",
                out_dtype="f32", status_flags=0) -> Params:
    p = Params()
    lib.draft_attn_params_init(ctypes.byref(p))
    p.num_seqs = int(num_seqs)
    p.num_draft_tokens = int(num_draft_tokens)
    p.num_q_heads = int(num_q_heads)
    p.num_kv_heads = int(num_kv_heads)
    p.head_dim = int(head_dim)
    p.num_blocks = int(num_blocks)
    p.max_blocks_per_seq = int(max_blocks_per_seq)
    p.mode = _MODES[mode] if isinstance(mode, str) else int(mode)
    p.window = int(window)
    p.n_sink = int(n_sink)
    p.alpha = float(alpha)
    p.beta = float(beta)
    p.kappa = float(kappa)
    p.n0 = int(n0)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(head_dim) if head_dim > 0 else 0.0
    p.softmax_scale = float(softmax_scale)
    p.rope = _ROPES[rope] if isinstance(rope, str) else int(rope)
    p.rope_theta = float(rope_theta)
    p.split_keys = int(split_keys)
    p.fold_variant = _FOLD_VARIANTS[fold_variant] if isinstance(fold_variant, str) else int(fold_variant)
    p.launch = _LAUNCHES[launch] if isinstance(launch, str) else int(launch)
    p.out_dtype = _out_code(out_dtype)
    p.debug_visit = int(debug_visit) or None
    p.debug_visit_stride = int(debug_visit_stride)
    p.status_flags = int(status_flags) or None
    if prof_events is not None:
        p.prof_events[0] = int(prof_events[0])
        p.prof_events[1] = int(prof_events[1])
    return p


def _out_code(out_dtype) -> int:
    """out_dtype given as "f32" / "bf16", a torch dtype, or the header's code."""
    if isinstance(out_dtype, str):
        return _OUT_DTYPES[out_dtype]
    if isinstance(out_dtype, int):
        return out_dtype
    import torch
    return {torch.float32: OUT_F32, torch.bfloat16: OUT_BF16}[out_dtype]


def _out_torch_dtype(code: int):
    import torch
    return torch.bfloat16 if code == OUT_BF16 else torch.float32


def _host_i32(values):
    arr = (ctypes.c_int32 * max(len(values), 1))(*[int(x) for x in values])
    return arr


def _expect(t, name, dtype, shape, device):
    """Argument check of the binding: the C ABI sees only pointers, so shapes, dtypes,
    device and contiguity are checked here. shape entries of None match any size."""
    if device.type != "cuda":
        raise ValueError(f"{name}: tensors must be on a GPU (cuda) device, got {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if t.dim() != len(shape) or any(want is not None and got != want for got, want in zip(t.shape, shape)):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple('*' if x is None else x for x in shape)}")
    if t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def _check_cache(k_cache, v_cache, k_side, Hkv, d, device):
    import torch
    NB = k_cache.shape[0]
    _expect(k_cache, "k_cache", torch.bfloat16, (NB, Hkv, d // 8, 16, 8), device)
    _expect(v_cache, "v_cache", torch.bfloat16, (NB, Hkv, d, 16), device)
    if k_side is not None:
        _expect(k_side, "k_side", torch.bfloat16, (NB, Hkv, d // 8, 16, 8), device)


def workspace_size(params: Params, ctx_lens) -> int:
    n = ctypes.c_size_t(0)
    st = lib.draft_attn_workspace_size(ctypes.byref(params), _host_i32(ctx_lens), ctypes.byref(n))
    if st != OK:
        raise DraftAttnError(st, "draft_attn_workspace_size")
    return int(n.value)


def plan(params: Params, ctx_lens):
    """Work items {seq, kv_head, range_begin, range_end, partition, first_step,
    step_stride} (the item reads the range's 32-key steps first_step,
    first_step + step_stride, ...) and the chunk size."""
    host = _host_i32(ctx_lens)
    total = ctypes.c_int64(0)
    chunk = ctypes.c_int32(0)
    st = lib.draft_attn_plan(ctypes.byref(params), host, None, 0, ctypes.byref(total), ctypes.byref(chunk), None)
    if st != OK:
        raise DraftAttnError(st, "draft_attn_plan")
    buf = (ctypes.c_int32 * (PLAN_ITEM_INTS * max(total.value, 1)))()
    st = lib.draft_attn_plan(ctypes.byref(params), host, buf, total.value, ctypes.byref(total),
                             ctypes.byref(chunk), None)
    if st != OK:
        raise DraftAttnError(st, "draft_attn_plan")
    items = [tuple(buf[PLAN_ITEM_INTS * i:PLAN_ITEM_INTS * (i + 1)]) for i in range(total.value)]
    return items, int(chunk.value)


def launch_of(params: Params, ctx_lens) -> str:
    """Launch shape a call with these params and lengths uses: "two_pass" or "single"."""
    total, chunk, launch = ctypes.c_int64(0), ctypes.c_int32(0), ctypes.c_int32(0)
    st = lib.draft_attn_plan(ctypes.byref(params), _host_i32(ctx_lens), None, 0, ctypes.byref(total),
                             ctypes.byref(chunk), ctypes.byref(launch))
    if st != OK:
        raise DraftAttnError(st, "draft_attn_plan")
    return "single" if launch.value == LAUNCH_SINGLE else "two_pass"


def prepare_launch_floor(params: Params, ctx_lens, kernels: int, stream=None):
    """A callable that enqueues draft_attn_launch_floor: the launch shape of the decode
    call with these params and lengths, with empty kernels (kernels = 1: the streaming
    pass's grid only; 2: and the merge pass's)."""
    import torch
    host = _host_i32(ctx_lens)
    s = torch.cuda.current_stream().cuda_stream if stream is None else int(stream)
    fn = lib.draft_attn_launch_floor
    ref = ctypes.byref(params)

    def call():
        st = fn(ref, host, int(kernels), s)
        if st != OK:
            raise DraftAttnError(st, "draft_attn_launch_floor")
    call._keep = (params, host)
    return call


class PreparedDecode:
    """One decode call with its arguments marshalled once; calling it enqueues the
    call again on the stream given at preparation (or on `stream`)."""

    def __init__(self, params, args, out, lse, keep, fused=False):
        self.params, self.args, self.out, self.lse, self._keep = params, args, out, lse, keep
        self._fn = lib.draft_attn_decode_draft if fused else lib.draft_attn_decode

    def __call__(self, stream=None, prof_events=None):
        p = self.params
        if prof_events is not None:
            p.prof_events[0], p.prof_events[1] = int(prof_events[0]), int(prof_events[1])
        else:
            p.prof_events[0] = p.prof_events[1] = None
        args = self.args if stream is None else self.args[:-1] + (int(stream),)
        st = self._fn(ctypes.byref(p), *args)
        if st != OK:
            raise DraftAttnError(st, self._fn.__name__)
        return self.out, self.lse


def prepare(q, k_cache, v_cache, block_table, ctx_len, *, mode="full", window=0, n_sink=0, alpha=1.0,
            beta=0.0, kappa=0.0, n0=1, softmax_scale=None, rope="neox", rope_theta=1e4, k_side=None,
            ctx_lens=None, out=None, lse=None, workspace=None, stream=None, split_keys=0,
            debug_visit=None, fold_variant="B", launch="auto", out_dtype="f32", k_draft=None,
            v_draft=None, status=None, num_blocks=None) -> PreparedDecode:
    """Marshal the arguments of decode() once (same meaning as there)."""
    import torch

    B, T, Hq, d = q.shape
    Hkv = k_cache.shape[1]
    dev = q.device
    _expect(q, "q", torch.bfloat16, (B, T, Hq, d), dev)
    _check_cache(k_cache, v_cache, k_side, Hkv, d, dev)
    _expect(block_table, "block_table", torch.int32, (B, None), dev)
    _expect(ctx_len, "ctx_len", torch.int32, (B,), dev)
    if ctx_lens is None:
        ctx_lens = [int(x) for x in ctx_len.cpu().tolist()]
    if len(ctx_lens) != B:
        raise ValueError(f"ctx_lens: {len(ctx_lens)} lengths for {B} sequences")
    visit_ptr, visit_stride = 0, 0
    if debug_visit is not None:
        _expect(debug_visit, "debug_visit", torch.uint8, (B, None), dev)
        visit_ptr, visit_stride = debug_visit.data_ptr(), debug_visit.shape[1]
    status_ptr = 0
    if status is not None:
        _expect(status, "status", torch.int32, (1,), dev)
        status_ptr = status.data_ptr()
    nb = k_cache.shape[0] if num_blocks is None else int(num_blocks)
    if nb > k_cache.shape[0]:
        raise ValueError(f"num_blocks {nb} exceeds the pools' {k_cache.shape[0]} blocks")
    p = make_params(num_seqs=B, num_draft_tokens=T, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d,
                    num_blocks=nb, max_blocks_per_seq=block_table.shape[1], mode=mode,
                    window=window, n_sink=n_sink, alpha=alpha, beta=beta, kappa=kappa, n0=n0,
                    softmax_scale=softmax_scale, rope=rope, rope_theta=rope_theta,
                    split_keys=split_keys, debug_visit=visit_ptr, debug_visit_stride=visit_stride,
                    fold_variant=fold_variant, launch=launch, out_dtype=out_dtype, status_flags=status_ptr)
    if out is None:
        out = torch.empty((B, T, Hq, d), dtype=_out_torch_dtype(p.out_dtype), device=dev)
    _expect(out, "out", _out_torch_dtype(p.out_dtype), (B, T, Hq, d), dev)
    if lse is None:
        lse = torch.empty((B, T, Hq), dtype=torch.float32, device=dev)
    _expect(lse, "lse", torch.float32, (B, T, Hq), dev)
    need = workspace_size(p, ctx_lens)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    s = torch.cuda.current_stream(dev).cuda_stream if stream is None else int(stream)
    ptr = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    host = _host_i32(ctx_lens)
    fused = k_draft is not None or v_draft is not None
    if fused:
        _expect(k_draft, "k_draft", torch.bfloat16, (B, T, Hkv, d), dev)
        _expect(v_draft, "v_draft", torch.bfloat16, (B, T, Hkv, d), dev)
        args = (ptr(q), ptr(k_cache), ptr(v_cache), ptr(k_side), ptr(block_table), ptr(ctx_len), host,
                ptr(k_draft), ptr(v_draft), ptr(out), ptr(lse), ptr(workspace),
                workspace.numel() * workspace.element_size(), s)
    else:
        args = (ptr(q), ptr(k_cache), ptr(v_cache), ptr(k_side), ptr(block_table), ptr(ctx_len), host, ptr(out),
                ptr(lse), ptr(workspace), workspace.numel() * workspace.element_size(), s)
    keep = (q, k_cache, v_cache, k_side, block_table, ctx_len, workspace, debug_visit, host, k_draft, v_draft,
            status)
    return PreparedDecode(p, args, out, lse, keep, fused=fused)


def decode(q, k_cache, v_cache, block_table, ctx_len, *, mode="full", window=0, n_sink=0, alpha=1.0,
           beta=0.0, kappa=0.0, n0=1, softmax_scale=None, rope="neox", rope_theta=1e4, k_side=None,
           ctx_lens=None, out=None, lse=None, workspace=None, stream=None, split_keys=0,
           debug_visit=None, prof_events=None, fold_variant="B", launch="auto", out_dtype="f32",
           k_draft=None, v_draft=None, status=None, num_blocks=None):
    """Enqueue draft_attn_decode on the current (or given) stream; returns (out, lse).

    With k_draft / v_draft (bf16 [B,T,Hkv,d], the step's draft keys and values),
    enqueues draft_attn_decode_draft instead: the same result merged with each
    draft token's causal attention over draft keys 0..t.

    q bf16 [B,T,Hq,d]; k_cache / k_side bf16 [NB,Hkv,d/8,16,8]; v_cache bf16 [NB,Hkv,d,16];
    block_table int32 [B,MB]; ctx_len int32 [B] on the device; ctx_lens: the same
    lengths as a host list (read from ctx_len when omitted, which synchronises).
    out / lse / workspace are allocated with torch when not given. launch: "auto",
    "two_pass" or "single"; out_dtype: "f32" or "bf16" (the dtype of out). status: an
    optional int32 [1] device tensor into which the kernels OR STATUS_* bits (a table
    entry outside the pool, lengths that disagree); the caller clears it. num_blocks:
    blocks of the pools the table may name (default: all of them).
    """
    call = prepare(q, k_cache, v_cache, block_table, ctx_len, mode=mode, window=window, n_sink=n_sink, alpha=alpha,
                   beta=beta, kappa=kappa, n0=n0, softmax_scale=softmax_scale, rope=rope, rope_theta=rope_theta,
                   k_side=k_side, ctx_lens=ctx_lens, out=out, lse=lse, workspace=workspace, stream=stream,
                   split_keys=split_keys, debug_visit=debug_visit, fold_variant=fold_variant, launch=launch,
                   out_dtype=out_dtype, k_draft=k_draft, v_draft=v_draft, status=status, num_blocks=num_blocks)
    return call(prof_events=prof_events)


def decode_noalloc(q, k_cache, v_cache, block_table, ctx_len, *, out, lse, ctx_lens, mode="full", window=0,
                   n_sink=0, alpha=1.0, beta=0.0, kappa=0.0, n0=1, softmax_scale=None, rope="neox", rope_theta=1e4,
                   k_side=None, stream=None, split_keys=0, fold_variant="B", launch="auto", out_dtype="f32",
                   status=None):
    """Enqueue draft_attn_decode_noalloc: decode() without a workspace (the library's
    per-GPU scratch holds the partial records) and without allocating anything here
    either: out, lse and the host lengths ctx_lens must be given. Calls that overlap
    in time on one GPU race on that scratch."""
    import torch

    B, T, Hq, d = q.shape
    Hkv = k_cache.shape[1]
    dev = q.device
    _expect(q, "q", torch.bfloat16, (B, T, Hq, d), dev)
    _check_cache(k_cache, v_cache, k_side, Hkv, d, dev)
    _expect(block_table, "block_table", torch.int32, (B, None), dev)
    _expect(ctx_len, "ctx_len", torch.int32, (B,), dev)
    if len(ctx_lens) != B:
        raise ValueError(f"ctx_lens: {len(ctx_lens)} lengths for {B} sequences")
    status_ptr = 0
    if status is not None:
        _expect(status, "status", torch.int32, (1,), dev)
        status_ptr = status.data_ptr()
    p = make_params(num_seqs=B, num_draft_tokens=T, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d,
                    num_blocks=k_cache.shape[0], max_blocks_per_seq=block_table.shape[1], mode=mode,
                    window=window, n_sink=n_sink, alpha=alpha, beta=beta, kappa=kappa, n0=n0,
                    softmax_scale=softmax_scale, rope=rope, rope_theta=rope_theta, split_keys=split_keys,
                    fold_variant=fold_variant, launch=launch, out_dtype=out_dtype, status_flags=status_ptr)
    _expect(out, "out", _out_torch_dtype(p.out_dtype), (B, T, Hq, d), dev)
    _expect(lse, "lse", torch.float32, (B, T, Hq), dev)
    s = torch.cuda.current_stream(dev).cuda_stream if stream is None else int(stream)
    st = lib.draft_attn_decode_noalloc(ctypes.byref(p), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                       None if k_side is None else k_side.data_ptr(), block_table.data_ptr(),
                                       ctx_len.data_ptr(), _host_i32(ctx_lens), out.data_ptr(), lse.data_ptr(), s)
    if st != OK:
        raise DraftAttnError(st, "draft_attn_decode_noalloc")
    return out, lse


def _check_append(k_new, v_new, block_table, pos, k_cache, v_cache, k_side):
    import torch
    B, n_new, Hkv, d = k_new.shape
    dev = k_new.device
    _expect(k_new, "k_new", torch.bfloat16, (B, n_new, Hkv, d), dev)
    _expect(v_new, "v_new", torch.bfloat16, (B, n_new, Hkv, d), dev)
    _expect(block_table, "block_table", torch.int32, (B, None), dev)
    _expect(pos, "pos", torch.int32, (B,), dev)
    _check_cache(k_cache, v_cache, k_side, Hkv, d, dev)


def _check_merge(q, k_draft, v_draft, ctx_len, out, lse, num_kv_heads):
    import torch
    B, T, Hq, d = q.shape
    dev = q.device
    _expect(q, "q", torch.bfloat16, (B, T, Hq, d), dev)
    _expect(k_draft, "k_draft", torch.bfloat16, (B, T, num_kv_heads, d), dev)
    _expect(v_draft, "v_draft", torch.bfloat16, (B, T, num_kv_heads, d), dev)
    _expect(ctx_len, "ctx_len", torch.int32, (B,), dev)
    _expect(out, "out", torch.float32, (B, T, Hq, d), dev)
    _expect(lse, "lse", torch.float32, (B, T, Hq), dev)


def make_append_params(*, num_seqs, num_new, num_kv_heads, head_dim, num_blocks, max_blocks_per_seq,
                       rope="neox", rope_theta=1e4, status_flags=0) -> AppendParams:
    p = AppendParams()
    lib.draft_attn_append_params_init(ctypes.byref(p))
    p.num_seqs, p.num_new, p.num_kv_heads, p.head_dim = int(num_seqs), int(num_new), int(num_kv_heads), int(head_dim)
    p.num_blocks, p.max_blocks_per_seq = int(num_blocks), int(max_blocks_per_seq)
    p.rope = _ROPES[rope] if isinstance(rope, str) else int(rope)
    p.rope_theta = float(rope_theta)
    p.status_flags = int(status_flags) or None
    return p


def append(k_new, v_new, block_table, pos, k_cache, v_cache, k_side=None, *, rope="neox", rope_theta=1e4,
           pos_host=None, stream=None, num_blocks=None, status=None):
    """Enqueue draft_attn_append: write k_new / v_new ([B, n_new, Hkv, d] bf16) at positions
    pos[b] + i (pos: int32 [B] on the device; pos_host: the same values as a list).
    num_blocks: blocks of the pools the table may name (default: all of them); status: an
    optional int32 [1] device tensor that receives STATUS_APPEND_BAD_BLOCK."""
    import torch

    B, n_new, Hkv, d = k_new.shape
    _check_append(k_new, v_new, block_table, pos, k_cache, v_cache, k_side)
    if pos_host is None:
        pos_host = [int(x) for x in pos.cpu().tolist()]
    status_ptr = 0
    if status is not None:
        _expect(status, "status", torch.int32, (1,), k_new.device)
        status_ptr = status.data_ptr()
    nb = k_cache.shape[0] if num_blocks is None else int(num_blocks)
    if nb > k_cache.shape[0]:
        raise ValueError(f"num_blocks {nb} exceeds the pools' {k_cache.shape[0]} blocks")
    p = make_append_params(num_seqs=B, num_new=n_new, num_kv_heads=Hkv, head_dim=d, num_blocks=nb,
                           max_blocks_per_seq=block_table.shape[1], rope=rope, rope_theta=rope_theta,
                           status_flags=status_ptr)
    s = torch.cuda.current_stream(k_new.device).cuda_stream if stream is None else int(stream)
    st = lib.draft_attn_append(ctypes.byref(p), k_new.data_ptr(), v_new.data_ptr(), block_table.data_ptr(),
                               pos.data_ptr(), _host_i32(pos_host), k_cache.data_ptr(), v_cache.data_ptr(),
                               None if k_side is None else k_side.data_ptr(), s)
    if st != OK:
        raise DraftAttnError(st, "draft_attn_append")


class PreparedCall:
    """A library call with its arguments marshalled once; calling it enqueues the call again
    (on the stream given at preparation, or on `stream`)."""

    def __init__(self, fn, name, params, args, keep, result=None):
        self._fn, self._name, self.params, self.args, self._keep, self._result = fn, name, params, args, keep, result

    def __call__(self, stream=None):
        args = self.args if stream is None else self.args[:-1] + (int(stream),)
        st = self._fn(ctypes.byref(self.params), *args)
        if st != OK:
            raise DraftAttnError(st, self._name)
        return self._result


def prepare_append(k_new, v_new, block_table, pos, k_cache, v_cache, k_side=None, *, rope="neox", rope_theta=1e4,
                   pos_host=None, stream=None) -> PreparedCall:
    """Marshal the arguments of append() once (same meaning as there)."""
    import torch

    B, n_new, Hkv, d = k_new.shape
    _check_append(k_new, v_new, block_table, pos, k_cache, v_cache, k_side)
    if pos_host is None:
        pos_host = [int(x) for x in pos.cpu().tolist()]
    p = make_append_params(num_seqs=B, num_new=n_new, num_kv_heads=Hkv, head_dim=d, num_blocks=k_cache.shape[0],
                           max_blocks_per_seq=block_table.shape[1], rope=rope, rope_theta=rope_theta)
    s = torch.cuda.current_stream(k_new.device).cuda_stream if stream is None else int(stream)
    host = _host_i32(pos_host)
    args = (k_new.data_ptr(), v_new.data_ptr(), block_table.data_ptr(), pos.data_ptr(), host, k_cache.data_ptr(),
            v_cache.data_ptr(), None if k_side is None else k_side.data_ptr(), s)
    keep = (k_new, v_new, block_table, pos, k_cache, v_cache, k_side, host)
    return PreparedCall(lib.draft_attn_append, "draft_attn_append", p, args, keep)


def prepare_merge_draft(q, k_draft, v_draft, ctx_len, out, lse, *, num_blocks, max_blocks_per_seq, num_kv_heads,
                        mode="full", window=0, n_sink=0, alpha=1.0, beta=0.0, kappa=0.0, n0=1, softmax_scale=None,
                        rope="neox", rope_theta=1e4, ctx_lens=None, stream=None) -> PreparedCall:
    """Marshal the arguments of merge_draft() once (same meaning as there)."""
    import torch

    B, T, Hq, d = q.shape
    _check_merge(q, k_draft, v_draft, ctx_len, out, lse, num_kv_heads)
    if ctx_lens is None:
        ctx_lens = [int(x) for x in ctx_len.cpu().tolist()]
    p = make_params(num_seqs=B, num_draft_tokens=T, num_q_heads=Hq, num_kv_heads=num_kv_heads, head_dim=d,
                    num_blocks=num_blocks, max_blocks_per_seq=max_blocks_per_seq, mode=mode, window=window,
                    n_sink=n_sink, alpha=alpha, beta=beta, kappa=kappa, n0=n0, softmax_scale=softmax_scale,
                    rope=rope, rope_theta=rope_theta)
    s = torch.cuda.current_stream(q.device).cuda_stream if stream is None else int(stream)
    host = _host_i32(ctx_lens)
    args = (q.data_ptr(), k_draft.data_ptr(), v_draft.data_ptr(), ctx_len.data_ptr(), host, out.data_ptr(),
            lse.data_ptr(), s)
    keep = (q, k_draft, v_draft, ctx_len, out, lse, host)
    return PreparedCall(lib.draft_attn_merge_draft, "draft_attn_merge_draft", p, args, keep, (out, lse))


def merge_draft(q, k_draft, v_draft, ctx_len, out, lse, *, num_blocks, max_blocks_per_seq, num_kv_heads,
                mode="full", window=0, n_sink=0, alpha=1.0, beta=0.0, kappa=0.0, n0=1, softmax_scale=None,
                rope="neox", rope_theta=1e4, ctx_lens=None, stream=None):
    """Enqueue draft_attn_merge_draft: fold the draft tokens' causal self-attention into
    (out, lse) from decode() of the same step, in place. k_draft, v_draft: [B, T, Hkv, d] bf16."""
    import torch

    B, T, Hq, d = q.shape
    _check_merge(q, k_draft, v_draft, ctx_len, out, lse, num_kv_heads)
    if ctx_lens is None:
        ctx_lens = [int(x) for x in ctx_len.cpu().tolist()]
    p = make_params(num_seqs=B, num_draft_tokens=T, num_q_heads=Hq, num_kv_heads=num_kv_heads, head_dim=d,
                    num_blocks=num_blocks, max_blocks_per_seq=max_blocks_per_seq, mode=mode, window=window,
                    n_sink=n_sink, alpha=alpha, beta=beta, kappa=kappa, n0=n0, softmax_scale=softmax_scale,
                    rope=rope, rope_theta=rope_theta)
    s = torch.cuda.current_stream(q.device).cuda_stream if stream is None else int(stream)
    st = lib.draft_attn_merge_draft(ctypes.byref(p), q.data_ptr(), k_draft.data_ptr(), v_draft.data_ptr(),
                                    ctx_len.data_ptr(), _host_i32(ctx_lens), out.data_ptr(), lse.data_ptr(), s)
    if st != OK:
        raise DraftAttnError(st, "draft_attn_merge_draft")
    return out, lse


def ring_size(window, n_sink, max_new):
    """(sink_blocks, ring_len) of the compact window-mode ring for these sizes."""
    sb, rl = ctypes.c_int32(0), ctypes.c_int32(0)
    st = lib.draft_attn_ring_size(int(window), int(n_sink), int(max_new), ctypes.byref(sb), ctypes.byref(rl))
    if st != OK:
        raise DraftAttnError(st, "draft_attn_ring_size")
    return int(sb.value), int(rl.value)


def ring_table(length, max_new, window, n_sink, sink_phys, ring_phys, max_blocks_per_seq):
    """Block-table row (list of ints) of a ring-buffer sequence; see draft_attn_ring_table."""
    row = (ctypes.c_int32 * int(max_blocks_per_seq))()
    sp = (ctypes.c_int32 * max(len(sink_phys), 1))(*sink_phys)
    rp = (ctypes.c_int32 * max(len(ring_phys), 1))(*ring_phys)
    st = lib.draft_attn_ring_table(int(length), int(max_new), int(window), int(n_sink), sp, len(sink_phys), rp,
                                   len(ring_phys), row, int(max_blocks_per_seq))
    if st != OK:
        raise DraftAttnError(st, "draft_attn_ring_table")
    return list(row)
