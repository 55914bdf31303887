"""Python binding of libsikv.so: self-indexing compressed-key decode attention on gfx950.

Thin ctypes layer with the same names as the C ABI (include/sikv.h).  It only
marshals arguments: torch supplies device memory and the current stream, and
every step of the computation runs in the library's HIP kernels.  There is no
CPU fallback: if the library is missing or fails to load, importing this
package raises.

Method: "Self-Indexing KVCache: Predicting Sparse Attention from Compressed
Keys" (web summary, technical part, §2.1 items 1-4).
"""

from __future__ import annotations

import ctypes
import math
import os

import torch  # first: the library then binds to the HIP runtime torch has loaded

from . import _abi

HEAD_DIM = 128
N_SINK = 64
# SIKV_LIBRARY: another build of the same library to load instead (a host-side
# sanitised one, say); by default the in-tree libsikv.so.
LIB_PATH = os.environ.get("SIKV_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libsikv.so")

OP_ENCODE, OP_SCORE_TOPK, OP_SPARSE_ATTN, OP_DECODE_STEP, OP_KMEANS = 0, 1, 2, 3, 4
FLAG_EXACT_SELECT = _abi.FLAG_EXACT_SELECT


class SikvError(RuntimeError):
    """A libsikv call returned a non-zero status."""

    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__(f"{call}: {status_str(status)} (status {status})")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python bit_self_indexed_amd/build.py` "
            "(the HIP library is required, there is no fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    _abi.declare(lib)
    if lib.sikv_abi_version() != _abi.ABI_VERSION:
        raise ImportError("libsikv.so ABI version mismatch; rebuild it")
    if lib.sikv_desc_size() != ctypes.sizeof(_abi.CacheDesc):
        raise ImportError("libsikv.so cache descriptor layout mismatch; rebuild it")
    return lib


lib = _load()


def status_str(status: int) -> str:
    return lib.sikv_status_str(int(status)).decode()


def _check(status: int, call: str) -> None:
    if status != 0:
        raise SikvError(status, call)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _bits(t: torch.Tensor) -> torch.Tensor:
    """bf16 tensors are passed as their bit patterns; uint16/int16 pass through."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16)
    if t.dtype in (torch.int16, torch.uint16):
        return t
    raise TypeError(f"expected bfloat16 (or its uint16 bits), got {t.dtype}")


def _strides_rows(t: torch.Tensor, name: str):
    """Strides (b, h, t) in elements of a [B, H, T, 128] tensor with unit channel stride."""
    if t.dim() != 4 or t.shape[-1] != HEAD_DIM or t.stride(-1) != 1:
        raise ValueError(f"{name} must be [B, H, T, 128] with contiguous channels")
    return t.stride(0), t.stride(1), t.stride(2)


class Timer:
    """A caller-owned kernel timer (sikv_timer): calls on a cache whose ``timer``
    is set, and comparator calls given ``timer=``, bracket each kernel they
    launch with HIP events on their stream.  ``read()`` synchronises on them."""

    def __init__(self):
        h = ctypes.c_void_p()
        _check(lib.sikv_timer_create(ctypes.byref(h)), "sikv_timer_create")
        self.handle = h

    def reset(self) -> None:
        _check(lib.sikv_timer_reset(self.handle), "sikv_timer_reset")

    def read(self) -> dict:
        """{kernel name: (launches, total ms)} since the last reset."""
        res = {}
        for i in range(lib.sikv_timer_count()):
            n = ctypes.c_int64()
            ms = ctypes.c_double()
            _check(lib.sikv_timer_read(self.handle, i, ctypes.byref(n), ctypes.byref(ms)),
                   "sikv_timer_read")
            res[lib.sikv_timer_name(i).decode()] = (int(n.value), float(ms.value))
        return res

    def close(self) -> None:
        if self.handle:
            _check(lib.sikv_timer_destroy(self.handle), "sikv_timer_destroy")
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _timer(t) -> ctypes.c_void_p | None:
    return None if t is None else t.handle


class Workspace:
    """Caller-owned device scratch, grown on demand (256-byte aligned)."""

    def __init__(self, device):
        self.device = torch.device(device)
        self.buf = None

    def get(self, nbytes: int):
        if nbytes == 0:
            return None, 0
        if self.buf is None or self.buf.numel() < nbytes + 256:
            self.buf = torch.empty(nbytes + 256, dtype=torch.uint8, device=self.device)
        base = self.buf.data_ptr()
        off = (-base) % 256
        return ctypes.c_void_p(base + off), self.buf.numel() - off


class Cache:
    """The compressed key cache of one layer plus a reference to its value cache.

    codes uint8 [B,Hkv,cap,16], alpha fp32 [B,Hkv,cap], mu fp32 [B,Hkv,128],
    k_sink bf16 [B,Hkv,64,128] are owned here; ``v`` (bf16 [B,Hkv,>=cap,128],
    unit channel stride) is only referenced.  codebook=True adds data-derived
    centres, fp32 [B,Hkv,32,16,4], written at prefill and used by every call.
    quant_v=True keeps the values 2-bit instead: vrec uint8 [B,Hkv,cap,64], one
    record per token (value codes, bytes 0..31; fp16 scale/zero words of the 4
    channel groups, 32..47; a copy of the key code, 48..63), and v_sink bf16
    [B,Hkv,64,128], written by sikv_encode_v / sikv_encode or the fused append
    step; ``v`` is then not read.  ``vq`` and ``vsz`` are views of the record
    fields (codes [B,Hkv,cap,32] uint8, words [B,Hkv,cap,4] int32).
    """

    def __init__(self, batch: int, n_kv_heads: int, capacity: int, device="cuda",
                 v: torch.Tensor | None = None, codebook: bool = False, quant_v: bool = False):
        dev = torch.device(device)
        self.batch, self.n_kv_heads, self.capacity = batch, n_kv_heads, capacity
        self.n_tokens = 0
        self.codes = torch.zeros((batch, n_kv_heads, capacity, 16), dtype=torch.uint8, device=dev)
        self.alpha = torch.zeros((batch, n_kv_heads, capacity), dtype=torch.float32, device=dev)
        self.mu = torch.zeros((batch, n_kv_heads, HEAD_DIM), dtype=torch.float32, device=dev)
        self.k_sink = torch.zeros((batch, n_kv_heads, N_SINK, HEAD_DIM), dtype=torch.bfloat16,
                                  device=dev)
        self.codebook = (torch.zeros((batch, n_kv_heads, 32, 16, 4), dtype=torch.float32,
                                     device=dev) if codebook else None)
        self.vrec = self.v_sink = None
        if quant_v:
            self.vrec = torch.zeros((batch, n_kv_heads, capacity, 64), dtype=torch.uint8,
                                    device=dev)
            self.v_sink = torch.zeros((batch, n_kv_heads, N_SINK, HEAD_DIM), dtype=torch.bfloat16,
                                      device=dev)
        self.v = v
        self.seq_lens = None  # ragged batch: int32 [B] on the device (see view())
        self.page_table = None  # paged pool (see paged())
        self.page_size = self.pages_per_seq = self.n_pages = 0
        self.timer = None  # a Timer: every call on this cache times its kernels
        self.ws = Workspace(dev)

    @classmethod
    def paged(cls, batch: int, n_kv_heads: int, page_size: int, n_pages: int,
              page_table: torch.Tensor, device="cuda", v: torch.Tensor | None = None,
              codebook: bool = False, quant_v: bool = False) -> "Cache":
        """A cache whose per-token arrays live in a pool of n_pages pages of page_size
        tokens (all KV heads per page): codes [n_pages,Hkv,P,16], alpha [n_pages,Hkv,P],
        vrec [n_pages,Hkv,P,64]; page_table int32 [batch, pages_per_seq] on the device
        maps each sequence's logical pages to pool pages; ``v`` (bf16 values) is a pool
        [n_pages,Hkv,P,128] addressed the same way.  Means, sinks and codebooks stay per
        sequence."""
        dev = torch.device(device)
        pps = int(page_table.shape[1])
        c = cls(batch, n_kv_heads, 1, device=dev, v=v, codebook=codebook, quant_v=False)
        c.capacity = pps * page_size
        P = page_size
        c.codes = torch.zeros((n_pages, n_kv_heads, P, 16), dtype=torch.uint8, device=dev)
        c.alpha = torch.zeros((n_pages, n_kv_heads, P), dtype=torch.float32, device=dev)
        if quant_v:
            c.vrec = torch.zeros((n_pages, n_kv_heads, P, 64), dtype=torch.uint8, device=dev)
            c.v_sink = torch.zeros((batch, n_kv_heads, N_SINK, HEAD_DIM), dtype=torch.bfloat16,
                                   device=dev)
        c.page_table = page_table
        c.page_size, c.pages_per_seq, c.n_pages = P, pps, n_pages
        return c

    @property
    def device(self):
        return self.codes.device

    def desc(self) -> _abi.CacheDesc:
        d = _abi.CacheDesc()
        d.batch, d.n_kv_heads, d.head_dim = self.batch, self.n_kv_heads, HEAD_DIM
        d.capacity, d.n_tokens, d.n_sink = self.capacity, self.n_tokens, N_SINK
        d.codes = self.codes.data_ptr()
        d.alpha = self.alpha.data_ptr()
        d.mu = self.mu.data_ptr()
        d.k_sink = self.k_sink.data_ptr()
        if self.v is not None:
            sb, sh, st = _strides_rows(self.v, "v")
            d.v = self.v.data_ptr()
            d.v_stride_b, d.v_stride_h, d.v_stride_t = sb, sh, st
        d.codebook = self.codebook.data_ptr() if self.codebook is not None else None
        d.vrec, d.v_sink = _ptr(self.vrec), _ptr(self.v_sink)
        d.seq_lens = _ptr(self.seq_lens)
        if self.page_table is not None:
            d.page_table = self.page_table.data_ptr()
            d.page_size, d.pages_per_seq, d.n_pages = (self.page_size, self.pages_per_seq,
                                                       self.n_pages)
        d.flags = 0
        d.timer = _timer(self.timer)
        return d

    @property
    def vq(self):
        return None if self.vrec is None else self.vrec[..., :32]

    @property
    def vsz(self):
        return None if self.vrec is None else self.vrec[..., 32:48].view(torch.int32)

    def view(self, b: int) -> "Cache":
        """Sequence b as a batch-1 cache sharing this cache's memory (for ragged
        prefill: encode each sequence with its own length, then set seq_lens)."""
        c = Cache.__new__(Cache)
        c.batch, c.n_kv_heads, c.capacity = 1, self.n_kv_heads, self.capacity
        c.n_tokens = self.n_tokens
        paged = self.page_table is not None
        pooled = ("codes", "alpha", "vrec", "v") if paged else ()
        for name in ("codes", "alpha", "mu", "k_sink", "codebook", "vrec", "v_sink", "v"):
            t = getattr(self, name)
            setattr(c, name, None if t is None else (t if name in pooled else t[b:b + 1]))
        c.seq_lens = None
        c.page_table = self.page_table[b:b + 1] if paged else None
        c.page_size, c.pages_per_seq, c.n_pages = self.page_size, self.pages_per_seq, self.n_pages
        c.timer = self.timer
        c.ws = self.ws
        return c


def workspace_bytes(op: int, cache: Cache, n_q_heads: int = 1, top_k: int = 1) -> int:
    d = cache.desc()
    return int(lib.sikv_workspace_bytes(op, ctypes.byref(d), n_q_heads, top_k))


def sikv_encode(cache: Cache, k: torch.Tensor, t_begin: int = 0, t_end: int | None = None,
                recompute_mu: bool = True) -> None:
    """Compress keys of tokens [t_begin, t_end) (k holds exactly those rows).
    recompute_mu=True: prefill of the whole cache (t_begin 0, sets n_tokens);
    False: append with the frozen mean (raises n_tokens to t_end)."""
    kb = _bits(k)
    if t_end is None:
        t_end = t_begin + kb.shape[2]
    sb, sh, st = _strides_rows(kb, "k")
    if recompute_mu:
        cache.n_tokens = t_end
    d = cache.desc()
    need = int(lib.sikv_workspace_bytes(OP_ENCODE, ctypes.byref(d), 1, 1)) if recompute_mu else 0
    ws, wsn = cache.ws.get(need)
    _check(lib.sikv_encode(ctypes.byref(d), kb.data_ptr(), sb, sh, st, t_begin, t_end,
                           1 if recompute_mu else 0, ws, wsn, _stream(cache.device)),
           "sikv_encode")
    if not recompute_mu:
        cache.n_tokens = max(cache.n_tokens, t_end)


def sikv_encode_v(cache: Cache, v: torch.Tensor, t_begin: int = 0) -> None:
    """2-bit value codes of tokens [t_begin, t_begin + v.shape[2]) (v holds
    exactly those rows); rows below 64 are also kept whole in cache.v_sink."""
    vb = _bits(v)
    sb, sh, st = _strides_rows(vb, "v")
    d = cache.desc()
    _check(lib.sikv_encode_v(ctypes.byref(d), vb.data_ptr(), sb, sh, st, t_begin,
                             t_begin + vb.shape[2], _stream(cache.device)), "sikv_encode_v")


def sikv_score_topk(cache: Cache, q: torch.Tensor, top_k: int, idx: torch.Tensor | None = None,
                    scores: torch.Tensor | None = None, exact_select: bool = False) -> torch.Tensor:
    """exact_select: skip the sampled threshold and take the exact whole-head
    selection path (SIKV_FLAG_EXACT_SELECT for this call only; same result)."""
    qb = _bits(q).contiguous()
    n_q = qb.shape[1]
    d = cache.desc()
    if exact_select:
        d.flags |= FLAG_EXACT_SELECT
    if idx is None:
        idx = torch.empty((cache.batch, cache.n_kv_heads, top_k), dtype=torch.int32,
                          device=cache.device)
    need = int(lib.sikv_workspace_bytes(OP_SCORE_TOPK, ctypes.byref(d), n_q, top_k))
    ws, wsn = cache.ws.get(need)
    _check(lib.sikv_score_topk(ctypes.byref(d), qb.data_ptr(), n_q, top_k, idx.data_ptr(),
                               _ptr(scores), ws, wsn, _stream(cache.device)), "sikv_score_topk")
    return idx


def sikv_sparse_attn(cache: Cache, q: torch.Tensor, idx: torch.Tensor,
                     sm_scale: float | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    qb = _bits(q).contiguous()
    n_q = qb.shape[1]
    top_k = idx.shape[-1]
    sm = 1.0 / math.sqrt(HEAD_DIM) if sm_scale is None else float(sm_scale)
    if out is None:
        out = torch.empty((cache.batch, n_q, HEAD_DIM), dtype=torch.float32, device=cache.device)
    d = cache.desc()
    need = int(lib.sikv_workspace_bytes(OP_SPARSE_ATTN, ctypes.byref(d), n_q, top_k))
    ws, wsn = cache.ws.get(need)
    idx = idx.contiguous()
    _check(lib.sikv_sparse_attn(ctypes.byref(d), qb.data_ptr(), n_q, idx.data_ptr(), top_k,
                                ctypes.c_float(sm), out.data_ptr(), ws, wsn, _stream(cache.device)),
           "sikv_sparse_attn")
    return out


def sikv_decode_step(cache: Cache, q: torch.Tensor, top_k: int, sm_scale: float | None = None,
                     idx_out: torch.Tensor | None = None, out: torch.Tensor | None = None,
                     exact_select: bool = False):
    qb = _bits(q).contiguous()
    n_q = qb.shape[1]
    sm = 1.0 / math.sqrt(HEAD_DIM) if sm_scale is None else float(sm_scale)
    if out is None:
        out = torch.empty((cache.batch, n_q, HEAD_DIM), dtype=torch.float32, device=cache.device)
    d = cache.desc()
    if exact_select:
        d.flags |= FLAG_EXACT_SELECT
    need = int(lib.sikv_workspace_bytes(OP_DECODE_STEP, ctypes.byref(d), n_q, top_k))
    ws, wsn = cache.ws.get(need)
    _check(lib.sikv_decode_step(ctypes.byref(d), qb.data_ptr(), n_q, top_k, ctypes.c_float(sm),
                                _ptr(idx_out), out.data_ptr(), ws, wsn, _stream(cache.device)),
           "sikv_decode_step")
    return out


def _append_decode_step(cache: Cache, k_new, q, top_k, sm_scale, idx_out, out, v_new,
                        static: bool):
    kb = _bits(k_new)
    if kb.dim() != 4 or kb.shape[2] != 1:
        raise ValueError("k_new must be [B, Hkv, 1, 128]")
    ksb, ksh, _ = _strides_rows(kb, "k_new")
    vnb, vsb, vsh = None, 0, 0
    if v_new is not None:
        vnb = _bits(v_new)
        if vnb.dim() != 4 or vnb.shape[2] != 1:
            raise ValueError("v_new must be [B, Hkv, 1, 128]")
        vsb, vsh, _ = _strides_rows(vnb, "v_new")
    qb = _bits(q).contiguous()
    n_q = qb.shape[1]
    sm = 1.0 / math.sqrt(HEAD_DIM) if sm_scale is None else float(sm_scale)
    if out is None:
        out = torch.empty((cache.batch, n_q, HEAD_DIM), dtype=torch.float32, device=cache.device)
    cache.n_tokens += 1
    if cache.seq_lens is not None:
        cache.seq_lens += 1   # every sequence appends one token (stream-ordered on the device)
    try:
        d = cache.desc()
        args = (ctypes.byref(d), kb.data_ptr(), ksb, ksh, _ptr(vnb), vsb, vsh, qb.data_ptr(), n_q,
                top_k, ctypes.c_float(sm), _ptr(idx_out), out.data_ptr())
        if static:
            _check(lib.sikv_append_decode_step_static(*args, _stream(cache.device)),
                   "sikv_append_decode_step_static")
        else:
            need = int(lib.sikv_workspace_bytes(OP_DECODE_STEP, ctypes.byref(d), n_q, top_k))
            ws, wsn = cache.ws.get(need)
            _check(lib.sikv_append_decode_step(*args, ws, wsn, _stream(cache.device)),
                   "sikv_append_decode_step")
    except Exception:
        cache.n_tokens -= 1
        if cache.seq_lens is not None:
            cache.seq_lens -= 1
        raise
    return out


def sikv_append_decode_step(cache: Cache, k_new: torch.Tensor, q: torch.Tensor, top_k: int,
                            sm_scale: float | None = None, idx_out: torch.Tensor | None = None,
                            out: torch.Tensor | None = None, v_new: torch.Tensor | None = None):
    """sikv_encode of token cache.n_tokens (k_new: [B, Hkv, 1, 128]) then
    sikv_decode_step over n_tokens + 1 tokens, in one call (raises n_tokens).
    v_new ([B, Hkv, 1, 128], quantised-value caches only) is encoded too."""
    return _append_decode_step(cache, k_new, q, top_k, sm_scale, idx_out, out, v_new, False)


def sikv_append_decode_step_static(cache: Cache, k_new: torch.Tensor, q: torch.Tensor,
                                   top_k: int, sm_scale: float | None = None,
                                   idx_out: torch.Tensor | None = None,
                                   out: torch.Tensor | None = None,
                                   v_new: torch.Tensor | None = None):
    """sikv_append_decode_step with the library's static device scratch instead of
    a workspace: allocates nothing on the device (``out`` and ``idx_out`` given),
    for callers that cannot allocate; the call serialises with every other call of
    it on the same GPU (they share the scratch)."""
    return _append_decode_step(cache, k_new, q, top_k, sm_scale, idx_out, out, v_new, True)


def sikv_dense_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                    sm_scale: float | None = None, out: torch.Tensor | None = None,
                    ws: Workspace | None = None, timer: Timer | None = None) -> torch.Tensor:
    """Dense bf16 decode attention over every token (the comparator)."""
    qb, kb, vb = _bits(q).contiguous(), _bits(k), _bits(v)
    B, n_q = qb.shape[0], qb.shape[1]
    Hkv, N = kb.shape[1], kb.shape[2]
    ksb, ksh, kst = _strides_rows(kb, "k")
    vsb, vsh, vst = _strides_rows(vb, "v")
    sm = 1.0 / math.sqrt(HEAD_DIM) if sm_scale is None else float(sm_scale)
    if out is None:
        out = torch.empty((B, n_q, HEAD_DIM), dtype=torch.float32, device=q.device)
    ws = ws or Workspace(q.device)
    w, wn = ws.get(int(lib.sikv_dense_workspace_bytes(B, Hkv, n_q, N)))
    _check(lib.sikv_dense_attn(B, Hkv, n_q, N, qb.data_ptr(), kb.data_ptr(), ksb, ksh, kst,
                               vb.data_ptr(), vsb, vsh, vst, ctypes.c_float(sm), out.data_ptr(),
                               w, wn, _stream(q.device), _timer(timer)), "sikv_dense_attn")
    return out


def sikv_kmeans_codebook(cache: Cache, k: torch.Tensor, n_iter: int = 20) -> None:
    """K-means baseline of the sign clustering: n_iter Lloyd iterations from the sign
    vertices over the prefill keys k ([B, Hkv, n_tokens, 128], the ones sikv_encode
    compressed), written to cache.codebook (one iteration = the one-pass codebook)."""
    if cache.codebook is None:
        raise ValueError("the cache has no codebook")
    kb = _bits(k)
    sb, sh, st = _strides_rows(kb, "k")
    d = cache.desc()
    need = int(lib.sikv_workspace_bytes(OP_KMEANS, ctypes.byref(d), 1, 1))
    ws, wsn = cache.ws.get(need)
    _check(lib.sikv_kmeans_codebook(ctypes.byref(d), kb.data_ptr(), sb, sh, st, int(n_iter), ws,
                                    wsn, _stream(cache.device)), "sikv_kmeans_codebook")


def sikv_dense_scores(q: torch.Tensor, k: torch.Tensor, n_tokens: int | None = None,
                      scores: torch.Tensor | None = None, timer: Timer | None = None) -> torch.Tensor:
    """Full dot-product retrieval scores (the comparator of the LUT-GEMV score):
    fp32 [B, Hkv, n_tokens], selection query (sum of each KV head's query group)
    dotted with every bf16 key."""
    qb, kb = _bits(q).contiguous(), _bits(k)
    B, n_q = qb.shape[0], qb.shape[1]
    Hkv = kb.shape[1]
    N = kb.shape[2] if n_tokens is None else int(n_tokens)
    ksb, ksh, kst = _strides_rows(kb, "k")
    if scores is None:
        scores = torch.empty((B, Hkv, N), dtype=torch.float32, device=q.device)
    _check(lib.sikv_dense_scores(B, Hkv, n_q, N, qb.data_ptr(), kb.data_ptr(), ksb, ksh, kst,
                                 scores.data_ptr(), _stream(q.device), _timer(timer)),
           "sikv_dense_scores")
    return scores


def sikv_stream_copy(dst: torch.Tensor, src: torch.Tensor, timer: Timer | None = None) -> None:
    n = src.numel() * src.element_size()
    _check(lib.sikv_stream_copy(dst.data_ptr(), src.data_ptr(), n, _stream(src.device),
                                _timer(timer)), "sikv_stream_copy")
