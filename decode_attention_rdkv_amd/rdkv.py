"""Python binding of librdkv: argument marshalling only.

Every function here checks tensor placement, dtype and shape, passes raw
device pointers and the current HIP stream to the C ABI declared in
include/rdkv.h, and raises RdkvError on a non-OK status.  All computation
happens in the library's HIP kernels; torch only provides device memory and
the stream.  If the library is missing, load() raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "librdkv.so")
HEAD_DIM = 128

c_i32, c_i64, c_u64, c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p


class Dims(ctypes.Structure):
    _fields_ = [("n_tokens", c_i64), ("n_seq", c_i32), ("n_layers", c_i32), ("n_q_heads", c_i32),
                ("n_kv_heads", c_i32), ("head_dim", c_i32), ("reserved", c_i32)]


class Layout(ctypes.Structure):
    _fields_ = [("dims", Dims), ("budget_v", c_i64), ("budget_k", c_i64), ("n_seg", c_i64), ("nk_max", c_i64),
                ("cache_bytes", c_u64), ("slots_offset", c_u64), ("slot_bytes", c_u64), ("slot_off_v", c_u64),
                ("slot_off_krec", c_u64), ("slot_off_pos", c_u64), ("decode_workspace_bytes", c_u64),
                ("zone_c_capacity", c_i32), ("rec_max", c_i32), ("max_chunks", c_i32), ("chunk_tok2", c_i32),
                ("n_generations", c_i32), ("token_slots", c_i32), ("gen_budget_v", c_i64), ("gen_budget_k", c_i64),
                ("gen_offset", c_u64), ("gen_bytes", c_u64), ("zc_stats_bytes", c_u64),
                ("rollover_workspace_bytes", c_u64)]

    @property
    def group(self) -> int:
        return self.dims.n_q_heads // self.dims.n_kv_heads


class PagedLayout(ctypes.Structure):
    _fields_ = [("dims", Dims), ("budget_v_max", c_i64), ("budget_k_max", c_i64), ("n_seg", c_i64),
                ("n_pages", c_i64), ("max_pages", c_i64), ("nk_max", c_i64), ("table_offset", c_u64),
                ("pool_offset", c_u64), ("cache_bytes", c_u64), ("decode_workspace_bytes", c_u64),
                ("zone_c_capacity", c_i32), ("rec_max", c_i32), ("max_chunks", c_i32), ("token_slots", c_i32),
                ("chunk_tok2", c_i32), ("reserved", c_i32)]

    @property
    def group(self) -> int:
        return self.dims.n_q_heads // self.dims.n_kv_heads


class LaunchShape(ctypes.Structure):
    _fields_ = [("token_slots", c_i32), ("rec_max", c_i32), ("max_chunks", c_i32), ("reserved", c_i32),
                ("decode_workspace_bytes", c_u64)]


STATUS = ["RDKV_OK", "RDKV_ERR_NULL", "RDKV_ERR_SHAPE", "RDKV_ERR_UNSUPPORTED", "RDKV_ERR_BUDGET",
          "RDKV_ERR_ALIGN", "RDKV_ERR_WORKSPACE", "RDKV_ERR_CAPACITY", "RDKV_ERR_HIP", "RDKV_ERR_OVERFLOW"]
RDKV_ERR_OVERFLOW = 9

# exported symbol -> (restype, argtypes)
SIGNATURES = {
    "rdkv_version": (c_i32, []),
    "rdkv_status_string": (ctypes.c_char_p, [c_i32]),
    "rdkv_layout_init": (c_i32, [ctypes.POINTER(Dims), c_i64, c_i64, c_i32, ctypes.POINTER(Layout)]),
    "rdkv_layout_init_rollover": (c_i32, [ctypes.POINTER(Dims), c_i64, c_i64, c_i32, c_i32, c_i64, c_i64,
                                          ctypes.POINTER(Layout)]),
    "rdkv_score_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(Dims)]),
    "rdkv_score": (c_i32, [ctypes.POINTER(Dims), c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, ctypes.c_size_t, c_vp]),
    "rdkv_score_lse": (c_i32, [ctypes.POINTER(Dims), c_vp, c_vp, c_vp, c_vp]),
    "rdkv_score_from_lse": (c_i32, [ctypes.POINTER(Dims), c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                    ctypes.c_size_t, c_vp]),
    "rdkv_allocate_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(Dims), c_i32]),
    "rdkv_allocate": (c_i32, [ctypes.POINTER(Dims), c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp,
                              c_vp, ctypes.c_size_t, c_vp]),
    "rdkv_allocate_shared": (c_i32, [ctypes.POINTER(Dims), c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i32, c_vp, c_vp,
                                     c_vp, c_vp, c_vp, ctypes.c_size_t, c_vp]),
    "rdkv_cache_init": (c_i32, [ctypes.POINTER(Layout), c_vp, ctypes.c_size_t, c_vp]),
    "rdkv_pack": (c_i32, [ctypes.POINTER(Layout), c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, ctypes.c_size_t, c_vp]),
    "rdkv_pack_status": (c_i32, [ctypes.POINTER(Layout), c_vp, ctypes.c_size_t, c_vp, c_vp]),
    "rdkv_decode": (c_i32, [ctypes.POINTER(Layout), c_vp, ctypes.c_size_t, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp,
                            ctypes.c_size_t, c_vp]),
    "rdkv_decode_shape": (c_i32, [ctypes.POINTER(Layout), c_vp, ctypes.c_size_t, c_vp, ctypes.c_size_t, c_vp,
                                  ctypes.POINTER(LaunchShape)]),
    "rdkv_decode_shaped": (c_i32, [ctypes.POINTER(Layout), ctypes.POINTER(LaunchShape), c_vp, ctypes.c_size_t, c_i32,
                                   c_vp, c_vp, c_vp, c_vp, c_vp, ctypes.c_size_t, c_vp]),
    "rdkv_decode_accumulate": (c_i32, [ctypes.POINTER(Layout), c_vp, ctypes.c_size_t, c_i32, c_vp, c_vp, c_vp, c_vp,
                                       c_vp, c_vp, ctypes.c_size_t, c_vp]),
    "rdkv_rollover_score": (c_i32, [ctypes.POINTER(Layout), c_vp, ctypes.c_size_t, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "rdkv_rollover": (c_i32, [ctypes.POINTER(Layout), c_vp, ctypes.c_size_t, c_i32, c_vp, c_vp, ctypes.c_size_t,
                              c_vp]),
    "rdkv_decode_static": (c_i32, [ctypes.POINTER(Layout), c_vp, ctypes.c_size_t, c_i32, c_vp, c_vp, c_vp, c_vp,
                                   c_vp]),
    "rdkv_decode_partials": (c_i32, [ctypes.POINTER(Layout), c_vp, ctypes.c_size_t, c_i32, c_vp, c_vp, c_vp, c_vp,
                                     ctypes.c_size_t, c_vp]),
    "rdkv_decode_merge": (c_i32, [ctypes.POINTER(Layout), c_vp, ctypes.c_size_t, c_i32, c_vp, c_vp, ctypes.c_size_t,
                                  c_vp]),
    "rdkv_paged_layout_init": (c_i32, [ctypes.POINTER(Dims), c_i64, c_i64, c_i32, c_i64,
                                       ctypes.POINTER(PagedLayout)]),
    "rdkv_paged_cache_init": (c_i32, [ctypes.POINTER(PagedLayout), c_vp, ctypes.c_size_t, c_vp]),
    "rdkv_paged_staging_bytes": (ctypes.c_size_t, [ctypes.POINTER(PagedLayout), c_i64, c_i64, c_i64]),
    "rdkv_paged_stage": (c_i32, [ctypes.POINTER(PagedLayout), c_i64, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp,
                                 ctypes.c_size_t, c_vp, c_vp]),
    "rdkv_paged_commit": (c_i32, [ctypes.POINTER(PagedLayout), c_i32, c_i64, c_i64, c_i64, c_vp, ctypes.c_size_t,
                                  c_vp, c_vp, ctypes.c_size_t, c_vp]),
    "rdkv_paged_release": (c_i32, [ctypes.POINTER(PagedLayout), c_i32, c_vp, ctypes.c_size_t, c_vp]),
    "rdkv_paged_decode": (c_i32, [ctypes.POINTER(PagedLayout), c_vp, ctypes.c_size_t, ctypes.POINTER(c_i32), c_vp,
                                  c_vp, c_vp, c_vp, c_vp, ctypes.c_size_t, c_vp]),
    "rdkv_paged_decode_shape": (c_i32, [ctypes.POINTER(PagedLayout), c_vp, ctypes.c_size_t, c_vp, ctypes.c_size_t,
                                        c_vp, ctypes.POINTER(LaunchShape)]),
    "rdkv_paged_decode_shaped": (c_i32, [ctypes.POINTER(PagedLayout), ctypes.POINTER(LaunchShape), c_vp,
                                         ctypes.c_size_t, ctypes.POINTER(c_i32), c_vp, c_vp, c_vp, c_vp, c_vp,
                                         ctypes.c_size_t, c_vp]),
    "rdkv_unpack": (c_i32, [ctypes.POINTER(Layout), c_vp, ctypes.c_size_t, c_i64, c_vp, c_vp, c_vp]),
}


class RdkvError(RuntimeError):
    def __init__(self, status: int, where: str):
        name = STATUS[status] if 0 <= status < len(STATUS) else str(status)
        super().__init__(f"{where}: {name}")
        self.status = status
        self.name = name


_lib: Optional[ctypes.CDLL] = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load librdkv.so (built in-tree); raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m decode_attention_rdkv_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int, where: str):
    if status != 0:
        raise RdkvError(status, where)


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t: Optional[torch.Tensor], dtype, shape=None, name="tensor") -> int:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t.data_ptr()


def make_dims(n_seq, n_layers, n_q_heads, n_kv_heads, n_tokens, head_dim=HEAD_DIM) -> Dims:
    return Dims(n_tokens=n_tokens, n_seq=n_seq, n_layers=n_layers, n_q_heads=n_q_heads, n_kv_heads=n_kv_heads,
                head_dim=head_dim, reserved=0)


def version() -> int:
    return load().rdkv_version()


def layout(dims: Dims, budget_v: int, budget_k: int, zone_c_capacity: int) -> Layout:
    out = Layout()
    _check(load().rdkv_layout_init(ctypes.byref(dims), budget_v, budget_k, zone_c_capacity, ctypes.byref(out)),
           "rdkv_layout_init")
    return out


def layout_rollover(dims: Dims, budget_v: int, budget_k: int, zone_c_capacity: int, n_generations: int,
                    gen_budget_v: int, gen_budget_k: int) -> Layout:
    """Layout whose zone C rolls over into up to n_generations generation blobs."""
    out = Layout()
    _check(load().rdkv_layout_init_rollover(ctypes.byref(dims), budget_v, budget_k, zone_c_capacity, n_generations,
                                            gen_budget_v, gen_budget_k, ctypes.byref(out)),
           "rdkv_layout_init_rollover")
    return out


def score_workspace_bytes(dims: Dims) -> int:
    return int(load().rdkv_score_workspace_bytes(ctypes.byref(dims)))


def score(dims: Dims, Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, workspace: Optional[torch.Tensor] = None):
    """Stage-1 weights; returns (w_tok, var_tok, w_chan) fp32 tensors."""
    lib = load()
    S, L, Hq, Hk, N = dims.n_seq, dims.n_layers, dims.n_q_heads, dims.n_kv_heads, dims.n_tokens
    dev = Q.device
    w_tok = torch.empty((S, L, Hk, N), dtype=torch.float32, device=dev)
    var_tok = torch.empty((S, L, Hk, N), dtype=torch.float32, device=dev)
    w_chan = torch.empty((S, L, Hk, HEAD_DIM), dtype=torch.float32, device=dev)
    ws_bytes = lib.rdkv_score_workspace_bytes(ctypes.byref(dims))
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    _check(lib.rdkv_score(ctypes.byref(dims), _ptr(Q, torch.float16, (S, L, Hq, N, HEAD_DIM), "Q"),
                          _ptr(K, torch.float16, (S, L, Hk, N, HEAD_DIM), "K"),
                          _ptr(V, torch.float16, (S, L, Hk, N, HEAD_DIM), "V"),
                          w_tok.data_ptr(), var_tok.data_ptr(), w_chan.data_ptr(),
                          _ptr(workspace, torch.uint8, None, "workspace"), workspace.numel(), _stream()),
           "rdkv_score")
    return w_tok, var_tok, w_chan


def score_lse(dims: Dims, Q: torch.Tensor, K: torch.Tensor, out: Optional[torch.Tensor] = None):
    """Row log-sum-exp (natural log) of the causal scaled scores: fp32 [S][L][Hq][N]."""
    lib = load()
    S, L, Hq, Hk, N = dims.n_seq, dims.n_layers, dims.n_q_heads, dims.n_kv_heads, dims.n_tokens
    if out is None:
        out = torch.empty((S, L, Hq, N), dtype=torch.float32, device=Q.device)
    _check(lib.rdkv_score_lse(ctypes.byref(dims), _ptr(Q, torch.float16, (S, L, Hq, N, HEAD_DIM), "Q"),
                              _ptr(K, torch.float16, (S, L, Hk, N, HEAD_DIM), "K"),
                              _ptr(out, torch.float32, (S, L, Hq, N), "lse"), _stream()),
           "rdkv_score_lse")
    return out


def score_from_lse(dims: Dims, Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, lse: torch.Tensor,
                   workspace: Optional[torch.Tensor] = None):
    """Stage-1 weights from a given natural-log row LSE; returns (w_tok, var_tok, w_chan)."""
    lib = load()
    S, L, Hq, Hk, N = dims.n_seq, dims.n_layers, dims.n_q_heads, dims.n_kv_heads, dims.n_tokens
    dev = Q.device
    w_tok = torch.empty((S, L, Hk, N), dtype=torch.float32, device=dev)
    var_tok = torch.empty((S, L, Hk, N), dtype=torch.float32, device=dev)
    w_chan = torch.empty((S, L, Hk, HEAD_DIM), dtype=torch.float32, device=dev)
    ws_bytes = lib.rdkv_score_workspace_bytes(ctypes.byref(dims))
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    _check(lib.rdkv_score_from_lse(ctypes.byref(dims), _ptr(Q, torch.float16, (S, L, Hq, N, HEAD_DIM), "Q"),
                                   _ptr(K, torch.float16, (S, L, Hk, N, HEAD_DIM), "K"),
                                   _ptr(V, torch.float16, (S, L, Hk, N, HEAD_DIM), "V"),
                                   _ptr(lse, torch.float32, (S, L, Hq, N), "lse"),
                                   w_tok.data_ptr(), var_tok.data_ptr(), w_chan.data_ptr(),
                                   _ptr(workspace, torch.uint8, None, "workspace"), workspace.numel(), _stream()),
           "rdkv_score_from_lse")
    return w_tok, var_tok, w_chan


def allocate_workspace_bytes(dims: Dims, group: int = 1) -> int:
    return int(load().rdkv_allocate_workspace_bytes(ctypes.byref(dims), group))


def allocate(dims: Dims, w_tok, var_tok, w_chan, K, budget_v: int, budget_k: int,
             workspace: Optional[torch.Tensor] = None):
    """Bit allocation; returns (bits_tok u8, bits_chan u8, var_chan f32, lambda f64 [...,2])."""
    return allocate_shared(dims, w_tok, var_tok, w_chan, K, budget_v, budget_k, 1, workspace=workspace)


def allocate_shared(dims: Dims, w_tok, var_tok, w_chan, K, budget_v: int, budget_k: int, group: int,
                    workspace: Optional[torch.Tensor] = None):
    """Bit allocation with one budget per group of `group` consecutive segments
    (rdkv_allocate for group 1)."""
    lib = load()
    S, L, Hk, N = dims.n_seq, dims.n_layers, dims.n_kv_heads, dims.n_tokens
    dev = K.device
    bits_tok = torch.empty((S, L, Hk, N), dtype=torch.uint8, device=dev)
    bits_chan = torch.empty((S, L, Hk, HEAD_DIM), dtype=torch.uint8, device=dev)
    var_chan = torch.empty((S, L, Hk, HEAD_DIM), dtype=torch.float32, device=dev)
    lam = torch.empty((S, L, Hk, 2), dtype=torch.float64, device=dev)
    if workspace is None:
        workspace = torch.empty(max(allocate_workspace_bytes(dims, group), 16), dtype=torch.uint8, device=dev)
    args = (ctypes.byref(dims), _ptr(w_tok, torch.float32, (S, L, Hk, N), "w_tok"),
            _ptr(var_tok, torch.float32, (S, L, Hk, N), "var_tok"),
            _ptr(w_chan, torch.float32, (S, L, Hk, HEAD_DIM), "w_chan"),
            _ptr(K, torch.float16, (S, L, Hk, N, HEAD_DIM), "K"), budget_v, budget_k)
    outs = (bits_tok.data_ptr(), bits_chan.data_ptr(), var_chan.data_ptr(), lam.data_ptr(), workspace.data_ptr(),
            workspace.numel() * workspace.element_size(), _stream())
    if group == 1:
        _check(lib.rdkv_allocate(*args, *outs), "rdkv_allocate")
    else:
        _check(lib.rdkv_allocate_shared(*args, group, *outs), "rdkv_allocate_shared")
    return bits_tok, bits_chan, var_chan, lam


def cache_init(lay: Layout, cache: Optional[torch.Tensor] = None, device="cuda") -> torch.Tensor:
    """A zeroed cache blob with header and empty descriptors (uint8 tensor)."""
    if cache is None:
        cache = torch.empty(lay.cache_bytes, dtype=torch.uint8, device=device)
    _check(load().rdkv_cache_init(ctypes.byref(lay), _ptr(cache, torch.uint8, None, "cache"), cache.numel(),
                                  _stream()), "rdkv_cache_init")
    return cache


def pack(lay: Layout, cache: torch.Tensor, K, V, bits_tok, bits_chan, layer_begin: int = 0, check: bool = True):
    """Quantize and pack layers [layer_begin, layer_begin + K.shape[1]) into the cache.

    With `check` (the default), waits for the stream and raises
    RdkvError(RDKV_ERR_OVERFLOW) if any segment of the cache was packed empty
    because its allocation exceeded the layout's budgets (rdkv_pack_status).
    """
    d = lay.dims
    S, Lin, Hk, N = d.n_seq, K.shape[1], d.n_kv_heads, d.n_tokens
    _check(load().rdkv_pack(ctypes.byref(lay), layer_begin, Lin,
                            _ptr(K, torch.float16, (S, Lin, Hk, N, HEAD_DIM), "K"),
                            _ptr(V, torch.float16, (S, Lin, Hk, N, HEAD_DIM), "V"),
                            _ptr(bits_tok, torch.uint8, (S, Lin, Hk, N), "bits_tok"),
                            _ptr(bits_chan, torch.uint8, (S, Lin, Hk, HEAD_DIM), "bits_chan"),
                            _ptr(cache, torch.uint8, None, "cache"), cache.numel(), _stream()),
           "rdkv_pack")
    if check:
        n = pack_status(lay, cache).item()
        if n:
            raise RdkvError(RDKV_ERR_OVERFLOW, f"rdkv_pack: {n} segment(s) exceed the layout's budgets and were "
                                               f"packed empty")


def pack_status(lay: Layout, cache: torch.Tensor) -> torch.Tensor:
    """Device int32[1]: segments packed empty because their allocation did not fit."""
    out = torch.empty(4, dtype=torch.int32, device=cache.device)
    _check(load().rdkv_pack_status(ctypes.byref(lay), _ptr(cache, torch.uint8, None, "cache"), cache.numel(),
                                   out.data_ptr(), _stream()), "rdkv_pack_status")
    return out[:1]


def decode_workspace(lay: Layout, device="cuda") -> torch.Tensor:
    return torch.empty(max(int(lay.decode_workspace_bytes), 16), dtype=torch.uint8, device=device)


def decode_shape(lay: Layout, cache: torch.Tensor, workspace: Optional[torch.Tensor] = None) -> "LaunchShape":
    """The decode launch shape of the prefill blob's segments (synchronous: reads the device)."""
    if workspace is None:
        workspace = torch.empty(16, dtype=torch.uint8, device=cache.device)
    out = LaunchShape()
    _check(load().rdkv_decode_shape(ctypes.byref(lay), _ptr(cache, torch.uint8, None, "cache"), cache.numel(),
                                    _ptr(workspace, torch.uint8, None, "workspace"), workspace.numel(), _stream(),
                                    ctypes.byref(out)),
           "rdkv_decode_shape")
    return out


def decode(lay: Layout, cache: torch.Tensor, c_len: int, q, k_new=None, v_new=None,
           workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
           shape: Optional["LaunchShape"] = None) -> torch.Tensor:
    """One decode step (rdkv_decode_shaped with `shape`); returns out fp32 [S][L][Hq][128]."""
    d = lay.dims
    S, L, Hq, Hk = d.n_seq, d.n_layers, d.n_q_heads, d.n_kv_heads
    if workspace is None:
        workspace = decode_workspace(lay, q.device)
    if out is None:
        out = torch.empty((S, L, Hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    args = (_ptr(cache, torch.uint8, None, "cache"), cache.numel(), c_len,
            _ptr(q, torch.float16, (S, L, Hq, HEAD_DIM), "q"),
            _ptr(k_new, torch.float16, (S, L, Hk, HEAD_DIM), "k_new"),
            _ptr(v_new, torch.float16, (S, L, Hk, HEAD_DIM), "v_new"),
            _ptr(out, torch.float32, (S, L, Hq, HEAD_DIM), "out"),
            _ptr(workspace, torch.uint8, None, "workspace"), workspace.numel(), _stream())
    if shape is None:
        _check(load().rdkv_decode(ctypes.byref(lay), *args), "rdkv_decode")
    else:
        _check(load().rdkv_decode_shaped(ctypes.byref(lay), ctypes.byref(shape), *args), "rdkv_decode_shaped")
    return out


def zone_c_stats(lay: Layout, device="cuda") -> torch.Tensor:
    """Zeroed decode-time statistics of zone C: fp32 [S][L][Hkv][G][cap + 128]."""
    d = lay.dims
    return torch.zeros((d.n_seq, d.n_layers, d.n_kv_heads, lay.group, lay.zone_c_capacity + HEAD_DIM),
                       dtype=torch.float32, device=device)


def decode_accumulate(lay: Layout, cache: torch.Tensor, c_len: int, q, k_new, v_new, stats: torch.Tensor,
                      workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """rdkv_decode_accumulate: one decode step that also adds each zone-C row's
    attention mass and the query channel squares to `stats`."""
    d = lay.dims
    S, L, Hq, Hk = d.n_seq, d.n_layers, d.n_q_heads, d.n_kv_heads
    if workspace is None:
        workspace = decode_workspace(lay, q.device)
    if out is None:
        out = torch.empty((S, L, Hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    _check(load().rdkv_decode_accumulate(
        ctypes.byref(lay), _ptr(cache, torch.uint8, None, "cache"), cache.numel(), c_len,
        _ptr(q, torch.float16, (S, L, Hq, HEAD_DIM), "q"), _ptr(k_new, torch.float16, (S, L, Hk, HEAD_DIM), "k_new"),
        _ptr(v_new, torch.float16, (S, L, Hk, HEAD_DIM), "v_new"), _ptr(out, torch.float32, (S, L, Hq, HEAD_DIM), "out"),
        _ptr(stats, torch.float32, (S, L, Hk, lay.group, lay.zone_c_capacity + HEAD_DIM), "stats"),
        _ptr(workspace, torch.uint8, None, "workspace"), workspace.numel(), _stream()), "rdkv_decode_accumulate")
    return out


def rollover_score(lay: Layout, cache: torch.Tensor, stats: torch.Tensor):
    """Stage-1 weights of the zone-C tokens: (w_tok [S][L][Hkv][cap], var_tok, w_chan [S][L][Hkv][128])."""
    d = lay.dims
    S, L, Hk, cap = d.n_seq, d.n_layers, d.n_kv_heads, lay.zone_c_capacity
    w_tok = torch.empty((S, L, Hk, cap), dtype=torch.float32, device=cache.device)
    var_tok = torch.empty_like(w_tok)
    w_chan = torch.empty((S, L, Hk, HEAD_DIM), dtype=torch.float32, device=cache.device)
    _check(load().rdkv_rollover_score(ctypes.byref(lay), _ptr(cache, torch.uint8, None, "cache"), cache.numel(),
                                      _ptr(stats, torch.float32, None, "stats"), w_tok.data_ptr(), var_tok.data_ptr(),
                                      w_chan.data_ptr(), _stream()), "rdkv_rollover_score")
    return w_tok, var_tok, w_chan


def rollover(lay: Layout, cache: torch.Tensor, generation: int, stats: torch.Tensor,
             workspace: Optional[torch.Tensor] = None):
    """rdkv_rollover: pack the full zone C into generation blob `generation`, clear zone C and `stats`."""
    if workspace is None:
        workspace = torch.empty(max(int(lay.rollover_workspace_bytes), 16), dtype=torch.uint8, device=cache.device)
    _check(load().rdkv_rollover(ctypes.byref(lay), _ptr(cache, torch.uint8, None, "cache"), cache.numel(), generation,
                                _ptr(stats, torch.float32, None, "stats"),
                                _ptr(workspace, torch.uint8, None, "workspace"), workspace.numel(), _stream()),
           "rdkv_rollover")


STATIC_SCRATCH_BYTES = 64 << 20


def decode_static(lay: Layout, cache: torch.Tensor, c_len: int, q, k_new=None, v_new=None,
                  out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """rdkv_decode_static: one decode step with the library's own device
    scratch instead of a workspace (the C call allocates nothing; pass `out`
    to keep this wrapper from allocating it)."""
    d = lay.dims
    S, L, Hq, Hk = d.n_seq, d.n_layers, d.n_q_heads, d.n_kv_heads
    if out is None:
        out = torch.empty((S, L, Hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    _check(load().rdkv_decode_static(ctypes.byref(lay), _ptr(cache, torch.uint8, None, "cache"), cache.numel(), c_len,
                                     _ptr(q, torch.float16, (S, L, Hq, HEAD_DIM), "q"),
                                     _ptr(k_new, torch.float16, (S, L, Hk, HEAD_DIM), "k_new"),
                                     _ptr(v_new, torch.float16, (S, L, Hk, HEAD_DIM), "v_new"),
                                     _ptr(out, torch.float32, (S, L, Hq, HEAD_DIM), "out"), _stream()),
           "rdkv_decode_static")
    return out


def decode_partials(lay: Layout, cache: torch.Tensor, c_len: int, q, k_new=None, v_new=None,
                    workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """First split-K phase (append + per-chunk partials); returns the workspace."""
    d = lay.dims
    S, L, Hq, Hk = d.n_seq, d.n_layers, d.n_q_heads, d.n_kv_heads
    if workspace is None:
        workspace = decode_workspace(lay, q.device)
    _check(load().rdkv_decode_partials(ctypes.byref(lay), _ptr(cache, torch.uint8, None, "cache"), cache.numel(),
                                       c_len, _ptr(q, torch.float16, (S, L, Hq, HEAD_DIM), "q"),
                                       _ptr(k_new, torch.float16, (S, L, Hk, HEAD_DIM), "k_new"),
                                       _ptr(v_new, torch.float16, (S, L, Hk, HEAD_DIM), "v_new"),
                                       _ptr(workspace, torch.uint8, None, "workspace"), workspace.numel(), _stream()),
           "rdkv_decode_partials")
    return workspace


def decode_merge(lay: Layout, cache: torch.Tensor, zone_c_rows: int, workspace: torch.Tensor,
                 out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Second split-K phase: merge the partials into out fp32 [S][L][Hq][128]."""
    d = lay.dims
    if out is None:
        out = torch.empty((d.n_seq, d.n_layers, d.n_q_heads, HEAD_DIM), dtype=torch.float32, device=cache.device)
    _check(load().rdkv_decode_merge(ctypes.byref(lay), _ptr(cache, torch.uint8, None, "cache"), cache.numel(),
                                    zone_c_rows, _ptr(out, torch.float32, None, "out"),
                                    _ptr(workspace, torch.uint8, None, "workspace"), workspace.numel(), _stream()),
           "rdkv_decode_merge")
    return out


def unpack(lay: Layout, cache: torch.Tensor, seg: int):
    """Dequantized kept rows of one segment: (k_hat, v_hat) fp32 [nk_max][128]."""
    nk = max(int(lay.nk_max), 1)
    k_hat = torch.zeros((nk, HEAD_DIM), dtype=torch.float32, device=cache.device)
    v_hat = torch.zeros((nk, HEAD_DIM), dtype=torch.float32, device=cache.device)
    _check(load().rdkv_unpack(ctypes.byref(lay), _ptr(cache, torch.uint8, None, "cache"), cache.numel(), seg,
                              k_hat.data_ptr(), v_hat.data_ptr(), _stream()), "rdkv_unpack")
    return k_hat, v_hat


# ---------------------------------------------------------------- paged cache

PAGE_BYTES = 32768


def paged_layout(dims_max: Dims, budget_v_max: int, budget_k_max: int, zone_c_capacity: int,
                 n_pages: int) -> PagedLayout:
    out = PagedLayout()
    _check(load().rdkv_paged_layout_init(ctypes.byref(dims_max), budget_v_max, budget_k_max, zone_c_capacity,
                                         n_pages, ctypes.byref(out)), "rdkv_paged_layout_init")
    return out


def paged_cache_init(pl: PagedLayout, cache: Optional[torch.Tensor] = None, device="cuda") -> torch.Tensor:
    if cache is None:
        cache = torch.empty(pl.cache_bytes, dtype=torch.uint8, device=device)
    _check(load().rdkv_paged_cache_init(ctypes.byref(pl), _ptr(cache, torch.uint8, None, "cache"), cache.numel(),
                                        _stream()), "rdkv_paged_cache_init")
    return cache


def paged_staging_bytes(pl: PagedLayout, n_tokens: int, budget_v: int, budget_k: int) -> int:
    return int(load().rdkv_paged_staging_bytes(ctypes.byref(pl), n_tokens, budget_v, budget_k))


def paged_stage(pl: PagedLayout, n_tokens: int, budget_v: int, budget_k: int, K, V, bits_tok, bits_chan,
                staging: Optional[torch.Tensor] = None):
    """Pack one sequence into a staging buffer; returns (staging, pages_needed
    device int32 [L*Hkv])."""
    d = pl.dims
    L, Hk = d.n_layers, d.n_kv_heads
    if staging is None:
        staging = torch.empty(max(paged_staging_bytes(pl, n_tokens, budget_v, budget_k), 16), dtype=torch.uint8,
                              device=K.device)
    need = torch.empty(max(L * Hk, 4), dtype=torch.int32, device=K.device)
    _check(load().rdkv_paged_stage(ctypes.byref(pl), n_tokens, budget_v, budget_k,
                                   _ptr(K, torch.float16, (L, Hk, n_tokens, HEAD_DIM), "K"),
                                   _ptr(V, torch.float16, (L, Hk, n_tokens, HEAD_DIM), "V"),
                                   _ptr(bits_tok, torch.uint8, (L, Hk, n_tokens), "bits_tok"),
                                   _ptr(bits_chan, torch.uint8, (L, Hk, HEAD_DIM), "bits_chan"),
                                   _ptr(staging, torch.uint8, None, "staging"), staging.numel(), need.data_ptr(),
                                   _stream()), "rdkv_paged_stage")
    return staging, need[:L * Hk]


def paged_commit(pl: PagedLayout, cache: torch.Tensor, seq: int, n_tokens: int, budget_v: int, budget_k: int,
                 staging: torch.Tensor, pages: torch.Tensor):
    """Commit a staged sequence into slot `seq` on the given pages (device int32 [L*Hkv][max_pages])."""
    d = pl.dims
    _check(load().rdkv_paged_commit(ctypes.byref(pl), seq, n_tokens, budget_v, budget_k,
                                    _ptr(staging, torch.uint8, None, "staging"), staging.numel(),
                                    _ptr(pages, torch.int32, (d.n_layers * d.n_kv_heads, pl.max_pages), "pages"),
                                    _ptr(cache, torch.uint8, None, "cache"), cache.numel(), _stream()),
           "rdkv_paged_commit")


def paged_release(pl: PagedLayout, cache: torch.Tensor, seq: int):
    _check(load().rdkv_paged_release(ctypes.byref(pl), seq, _ptr(cache, torch.uint8, None, "cache"), cache.numel(),
                                     _stream()), "rdkv_paged_release")


def paged_decode_workspace(pl: PagedLayout, device="cuda") -> torch.Tensor:
    return torch.empty(max(int(pl.decode_workspace_bytes), 16), dtype=torch.uint8, device=device)


def paged_decode_shape(pl: PagedLayout, cache: torch.Tensor, workspace: Optional[torch.Tensor] = None) -> LaunchShape:
    """The decode launch shape of the slots in use (synchronous: reads the device)."""
    if workspace is None:
        workspace = torch.empty(16, dtype=torch.uint8, device=cache.device)
    out = LaunchShape()
    _check(load().rdkv_paged_decode_shape(ctypes.byref(pl), _ptr(cache, torch.uint8, None, "cache"), cache.numel(),
                                          _ptr(workspace, torch.uint8, None, "workspace"), workspace.numel(),
                                          _stream(), ctypes.byref(out)),
           "rdkv_paged_decode_shape")
    return out


def paged_decode(pl: PagedLayout, cache: torch.Tensor, c_len, q, k_new=None, v_new=None,
                 workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                 shape: Optional[LaunchShape] = None) -> torch.Tensor:
    """One decode step over every sequence slot; c_len: host sequence of the
    slots' zone-C rows before the step.  With `shape` (paged_decode_shape),
    rdkv_paged_decode_shaped.  Returns out fp32 [S][L][Hq][128]."""
    d = pl.dims
    S, L, Hq, Hk = d.n_seq, d.n_layers, d.n_q_heads, d.n_kv_heads
    cl = (c_i32 * S)(*[int(x) for x in c_len])
    if workspace is None:
        workspace = paged_decode_workspace(pl, q.device)
    if out is None:
        out = torch.empty((S, L, Hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    args = (_ptr(cache, torch.uint8, None, "cache"), cache.numel(), cl,
            _ptr(q, torch.float16, (S, L, Hq, HEAD_DIM), "q"),
            _ptr(k_new, torch.float16, (S, L, Hk, HEAD_DIM), "k_new"),
            _ptr(v_new, torch.float16, (S, L, Hk, HEAD_DIM), "v_new"),
            _ptr(out, torch.float32, (S, L, Hq, HEAD_DIM), "out"),
            _ptr(workspace, torch.uint8, None, "workspace"), workspace.numel(), _stream())
    if shape is None:
        _check(load().rdkv_paged_decode(ctypes.byref(pl), *args), "rdkv_paged_decode")
    else:
        _check(load().rdkv_paged_decode_shaped(ctypes.byref(pl), ctypes.byref(shape), *args),
               "rdkv_paged_decode_shaped")
    return out


# ---------------------------------------------------------------- descriptor readout

DESC_BYTES = 256
HEADER_BYTES = 256


def descriptors(lay: Layout, cache: torch.Tensor):
    """Per-segment counts read back from the blob (host numpy dict of arrays).

    n_tok [n_seg][4] (kept tokens at 2/4/8/16 bits), n_chan [n_seg][4] (channels
    at 16/8/4/2 bits), rec [n_seg] (record bytes of a 2/4/8-bit token), flags.
    """
    import numpy as np
    raw = cache[HEADER_BYTES:HEADER_BYTES + DESC_BYTES * lay.n_seg].cpu().numpy().reshape(lay.n_seg, DESC_BYTES)
    i32 = raw[:, :48].copy().view(np.int32)
    return dict(n_tok=i32[:, 0:4].copy(), n_kept=i32[:, 4].copy(), n_chan=i32[:, 5:9].copy(),
                rec=i32[:, 9].copy(), flags=i32[:, 11].copy())


def decode_bytes(lay: Layout, desc: dict, n_c: int) -> dict:
    """Bytes of one decode step, from the descriptors.

    Algorithmic bytes (what the method has to move): V codes or fp16 rows of
    every kept token, one (scale, zero) word per 2/4/8-bit V row, K codes and
    fp16 channels (sum over kept channels of their bits, per kept token), one
    (scale, zero) word per present integer K part per kept token, zone-C rows,
    the queries and the fp32 outputs; `total` is their sum.  `k_padding` is
    what the stored K records add on top (each part rounded up to a word):
    read by the kernel, but not counted as algorithmic.
    """
    import numpy as np
    n_tok = desc["n_tok"].astype(np.int64)
    n_kept = desc["n_kept"].astype(np.int64)
    n_chan = desc["n_chan"].astype(np.int64)                      # channels at 16, 8, 4, 2 bits
    v = int((n_tok * np.array([32, 64, 128, 256])).sum())
    v_meta = int(4 * n_tok[:, :3].sum())
    k_bits = int((n_kept * (n_chan * np.array([16, 8, 4, 2])).sum(axis=1)).sum())
    k = (k_bits + 7) // 8
    k_meta = int(4 * (n_kept * (n_chan[:, 1:] > 0).sum(axis=1)).sum())
    k_read = int((n_kept * desc["rec"]).sum() - 4 * n_tok[:, 3].sum())
    zc = int(lay.n_seg * n_c * 2 * HEAD_DIM * 2)
    d = lay.dims
    qo = d.n_seq * d.n_layers * d.n_q_heads * HEAD_DIM * (2 + 4)
    return dict(v=v, v_meta=v_meta, k=k, k_meta=k_meta, zone_c=zc, q_out=qo,
                total=v + v_meta + k + k_meta + zc + qo, k_padding=k_read - (k + k_meta + v_meta))
