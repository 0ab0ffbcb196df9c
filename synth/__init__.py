"""Seeded synthetic inputs for decode attention, shared by the tests and the benchmark.

This module draws random numbers and lays them out; it holds none of the
attention arithmetic, and imports neither the HIP library nor the oracle.

Recipe (the same for every case): a CPU ``torch.Generator`` seeded per case;
values drawn as float32 N(0, 1) and cast to fp16/bf16 with round-to-nearest-even
(``Tensor.to``). Draw order: lengths -> page permutation -> q -> K -> V ->
k_new -> v_new. Float8 (e4m3fn) caches: q is bf16; K and V are drawn in
float32 as above, then one descale per (request, KV head) each for K and V is
drawn uniform in [1/64, 1/16], and the stored value is x / descale clamped to
+-448 and cast with round-to-nearest-even (the dequantised value is stored x
descale; unused pages use descale 1/32). Rows past a request's length hold
zeros, NaN or random values (``pad``); paged pools hold exactly the pages the requests use plus
``extra_pages`` unused ones (filled like padding), with physical page ids a
seeded random permutation, and the page table padded with -1.

The five named workloads follow the shapes of the pages' examples:
  c1  unpaged MHA, B=1, Hq=Hkv=32, D=128, 4096 tokens, fp16, 16 splits
  c2  GQA long context, B=1, Hq=32, Hkv=8, 131072 tokens, bf16
  c3  paged batch, B=32, Hq=32, Hkv=8, page 16, lengths U{512..8192}, bf16
  c4  append + NeoX rotary, B=4, Hq=32, Hkv=8, max_seqlen 2048,
      cache_seqlens U{1..2047}, fp16, base 10000, rotary_dim 128
  c5  cascade, 64 requests, Hq=32, Hkv=8, page 64, shared 16384-token prefix,
      suffixes U{256..2048}, bf16
and float8 versions of c2 and c3 (c2f8, c3f8): the same shapes and seeds with
float8 e4m3fn K/V and bf16 queries (also c1f8, c2g2f8 and the cascade c5f8, whose
shared prefix pages are stored at descale 1/32 and read with each request's
descales). Float8 append cases draw k_new / v_new as
bf16 and the descales after them (the caches are quantised as above).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import torch

F16, BF16 = torch.float16, torch.bfloat16
FP8 = torch.float8_e4m3fn


@dataclass
class Case:
    name: str
    dtype: torch.dtype
    B: int
    Hq: int
    Hkv: int
    D: int
    q: torch.Tensor                      # [B, Hq, D]
    k: torch.Tensor                      # contiguous [B, cap, Hkv, D] or pool [P, ps, Hkv, D]
    v: torch.Tensor
    seq_lens: torch.Tensor               # [B] int32 (cascade: suffix lengths; append: cache_seqlens)
    page_size: int = 0
    page_table: Optional[torch.Tensor] = None   # [B, max_pages] int32, -1 padded
    num_splits: int = 0
    # append + rotary
    k_new: Optional[torch.Tensor] = None  # [B, Hkv, D]
    v_new: Optional[torch.Tensor] = None
    rotary_dim: int = 0
    rope_base: float = 10000.0
    rope_cos: Optional[torch.Tensor] = None   # [max_pos, rotary_dim/2] fp32
    rope_sin: Optional[torch.Tensor] = None
    # cascade
    prefix_pages: Optional[torch.Tensor] = None  # [n_prefix_pages] int32
    prefix_len: int = 0
    # float8 caches: per (request, KV head) factors, [B, Hkv] float32
    k_descale: Optional[torch.Tensor] = None
    v_descale: Optional[torch.Tensor] = None
    # [B] int32: request b's row of a contiguous cache; its first valid row
    cache_batch_idx: Optional[torch.Tensor] = None
    cache_leftpad: Optional[torch.Tensor] = None
    meta: dict = field(default_factory=dict)

    @property
    def capacity(self) -> int:
        if self.page_size == 0:
            return self.k.shape[1]
        return self.page_table.shape[1] * self.page_size

    def attended_lens(self) -> torch.Tensor:
        """Tokens each request attends to (length + appended token + shared prefix)."""
        L = self.seq_lens.to(torch.int64)
        if self.k_new is not None:
            L = L + 1
        if self.cache_leftpad is not None:
            L = L - self.cache_leftpad.to(torch.int64)
        return L + self.prefix_len

    def kv_bytes(self) -> int:
        """K+V bytes of the attended rows, each KV head read once (prefix counted once)."""
        e = 1 if self.dtype == FP8 else 2
        per_tok = 2 * self.Hkv * self.D * e
        L = self.seq_lens.to(torch.int64) + (1 if self.k_new is not None else 0)
        if self.cache_leftpad is not None:
            L = L - self.cache_leftpad.to(torch.int64)
        return per_tok * (int(L.sum()) + self.prefix_len)


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


def _randn(g, shape, dtype):
    return torch.randn(shape, generator=g, dtype=torch.float32).to(dtype)


def _q_dtype(dtype):
    return BF16 if dtype == FP8 else dtype


def _kv_draw_dtype(dtype):
    return torch.float32 if dtype == FP8 else dtype


def _descales(g, B: int, Hkv: int):
    kd = torch.empty(B, Hkv, dtype=torch.float32).uniform_(1.0 / 64, 1.0 / 16, generator=g)
    vd = torch.empty(B, Hkv, dtype=torch.float32).uniform_(1.0 / 64, 1.0 / 16, generator=g)
    return kd, vd


def _quantize(x: torch.Tensor, f: torch.Tensor) -> torch.Tensor:
    """float32 x [.., Hkv, D] divided by f (broadcast), clamped to +-448, cast to e4m3fn."""
    return (x / f).clamp(-448.0, 448.0).to(FP8)


def _fill_pad(t: torch.Tensor, mask: torch.Tensor, pad: str, g) -> None:
    """Overwrite t[mask] according to the padding policy (mask broadcast over trailing dims)."""
    if pad == "random" or not bool(mask.any()):
        return
    val = float("nan") if pad == "nan" else 0.0
    t[mask] = torch.tensor(val, dtype=t.dtype)


def rope_tables(max_pos: int, rotary_dim: int, base: float = 10000.0):
    """Caller-side cos/sin tables [max_pos, rotary_dim/2] in fp32 (angles formed in float64)."""
    half = rotary_dim // 2
    inv = base ** (-2.0 * torch.arange(half, dtype=torch.float64) / rotary_dim)
    ang = torch.arange(max_pos, dtype=torch.float64)[:, None] * inv[None, :]
    return torch.cos(ang).to(torch.float32).contiguous(), torch.sin(ang).to(torch.float32).contiguous()


def contiguous_case(seed: int, B: int, Hq: int, Hkv: int, D: int, lens, cap: int,
                    dtype=F16, pad: str = "zero", name: str = "contig", num_splits: int = 0) -> Case:
    g = _gen(seed)
    lens = torch.as_tensor(lens, dtype=torch.int32).reshape(B)
    q = _randn(g, (B, Hq, D), _q_dtype(dtype))
    k = _randn(g, (B, cap, Hkv, D), _kv_draw_dtype(dtype))
    v = _randn(g, (B, cap, Hkv, D), _kv_draw_dtype(dtype))
    rows = torch.arange(cap)[None, :] >= lens[:, None].to(torch.int64)  # [B, cap]
    _fill_pad(k, rows, pad, g)
    _fill_pad(v, rows, pad, g)
    kd = vd = None
    if dtype == FP8:
        kd, vd = _descales(g, B, Hkv)
        k = _quantize(k, kd[:, None, :, None])
        v = _quantize(v, vd[:, None, :, None])
    return Case(name, dtype, B, Hq, Hkv, D, q, k, v, lens, num_splits=num_splits, k_descale=kd, v_descale=vd)


def indexed_case(seed: int, B: int, Hq: int, Hkv: int, D: int, lens, leftpad, cap: int, dtype=BF16,
                 cache_rows: Optional[int] = None, pad: str = "nan", name: str = "indexed") -> Case:
    """Contiguous cache with left padding and, when cache_rows is given, a cache_batch_idx.

    Request b reads rows [leftpad[b], lens[b]) of cache row batch_idx[b] (b without
    cache_rows); batch_idx is a seeded draw of distinct rows. Every other row of
    the cache (padding, past the length, rows no request names) is filled by
    `pad`. Float8 caches: descales per (request, KV head) as in contiguous_case,
    applied to the request's cache row (1/32 for unnamed rows).
    """
    g = _gen(seed)
    lens = torch.as_tensor(lens, dtype=torch.int32).reshape(B)
    lp = torch.as_tensor(leftpad, dtype=torch.int32).reshape(B)
    rows = B if cache_rows is None else cache_rows
    idx = None
    if cache_rows is not None:
        idx = torch.randperm(rows, generator=g)[:B].to(torch.int32)
    q = _randn(g, (B, Hq, D), _q_dtype(dtype))
    k = _randn(g, (rows, cap, Hkv, D), _kv_draw_dtype(dtype))
    v = _randn(g, (rows, cap, Hkv, D), _kv_draw_dtype(dtype))
    mask = torch.ones(rows, cap, dtype=torch.bool)
    for b in range(B):
        r = b if idx is None else int(idx[b])
        mask[r, int(lp[b]):int(lens[b])] = False
    _fill_pad(k, mask, pad, g)
    _fill_pad(v, mask, pad, g)
    kd = vd = None
    if dtype == FP8:
        kd, vd = _descales(g, B, Hkv)
        fk = torch.full((rows, Hkv), 1.0 / 32)
        fv = torch.full((rows, Hkv), 1.0 / 32)
        for b in range(B):
            r = b if idx is None else int(idx[b])
            fk[r], fv[r] = kd[b], vd[b]
        k = _quantize(k, fk[:, None, :, None])
        v = _quantize(v, fv[:, None, :, None])
    return Case(name, dtype, B, Hq, Hkv, D, q, k, v, lens, k_descale=kd, v_descale=vd, cache_batch_idx=idx,
                cache_leftpad=lp)


def multi_query(seed: int, case: Case, q_len: int) -> torch.Tensor:
    """Queries of q_len tokens per request, [B, q_len, Hq, D], drawn like a case's q (its own seed)."""
    g = _gen(seed)
    return _randn(g, (case.B, q_len, case.Hq, case.D), _q_dtype(case.dtype))


def pad_left(case: Case, leftpad, pad: str = "nan") -> Case:
    """Mark rows [0, leftpad[b]) of each request as left padding (filled by `pad`) and record leftpad."""
    lp = torch.as_tensor(leftpad, dtype=torch.int32).reshape(case.B)
    val = float("nan") if pad == "nan" else 0.0
    for b in range(case.B):
        for j in range(int(lp[b])):
            if case.page_size:
                p, s = int(case.page_table[b, j // case.page_size]), j % case.page_size
            else:
                r = b if case.cache_batch_idx is None else int(case.cache_batch_idx[b])
                p, s = r, j
            if case.k.dtype == FP8:
                case.k[p, s] = torch.full_like(case.k[p, s], val, dtype=torch.float32).to(FP8)
                case.v[p, s] = torch.full_like(case.v[p, s], val, dtype=torch.float32).to(FP8)
            else:
                case.k[p, s] = val
                case.v[p, s] = val
    case.cache_leftpad = lp
    return case


def _page_lists(g, lens, ps, extra_pages):
    need = [math.ceil(int(L) / ps) for L in lens]
    pool = sum(need) + extra_pages
    perm = torch.randperm(pool, generator=g).to(torch.int32) if pool > 0 else torch.zeros(0, dtype=torch.int32)
    lists, off = [], 0
    for n in need:
        lists.append(perm[off:off + n])
        off += n
    unused = perm[off:]
    return lists, unused, pool


def paged_case(seed: int, B: int, Hq: int, Hkv: int, D: int, lens, ps: int, dtype=BF16,
               max_pages: Optional[int] = None, extra_pages: int = 0, pad: str = "zero",
               name: str = "paged", num_splits: int = 0, lens_range=None) -> Case:
    g = _gen(seed)
    if lens_range is not None:
        lo, hi = lens_range
        lens = torch.randint(lo, hi + 1, (B,), generator=g, dtype=torch.int64).to(torch.int32)
    else:
        lens = torch.as_tensor(lens, dtype=torch.int32).reshape(B)
    lists, unused, pool = _page_lists(g, lens.tolist(), ps, extra_pages)
    if max_pages is None:
        max_pages = max([len(x) for x in lists] + [1])
    table = torch.full((B, max_pages), -1, dtype=torch.int32)
    for b, pl in enumerate(lists):
        assert len(pl) <= max_pages
        table[b, :len(pl)] = pl
    q = _randn(g, (B, Hq, D), _q_dtype(dtype))
    k = _randn(g, (pool, ps, Hkv, D), _kv_draw_dtype(dtype))
    v = _randn(g, (pool, ps, Hkv, D), _kv_draw_dtype(dtype))
    # padding: slots past each request's length in its last page, and unused pages
    mask = torch.zeros(pool, ps, dtype=torch.bool)
    for b, pl in enumerate(lists):
        L = int(lens[b])
        if len(pl) and L % ps:
            mask[int(pl[-1]), L % ps:] = True
    for p in unused.tolist():
        mask[p, :] = True
    _fill_pad(k, mask, pad, g)
    _fill_pad(v, mask, pad, g)
    kd = vd = None
    if dtype == FP8:
        kd, vd = _descales(g, B, Hkv)
        fk = torch.full((pool, Hkv), 1.0 / 32)  # per page: its request's descales
        fv = torch.full((pool, Hkv), 1.0 / 32)
        for b, pl in enumerate(lists):
            fk[pl.long()] = kd[b]
            fv[pl.long()] = vd[b]
        k = _quantize(k, fk[:, None, :, None])
        v = _quantize(v, fv[:, None, :, None])
    return Case(name, dtype, B, Hq, Hkv, D, q, k, v, lens, page_size=ps, page_table=table,
                num_splits=num_splits, k_descale=kd, v_descale=vd)


def append_case(seed: int, B: int, Hq: int, Hkv: int, D: int, max_seqlen: int, dtype=F16,
                rotary_dim: int = 128, base: float = 10000.0, pad: str = "zero",
                cache_seqlens=None, name: str = "append", page_size: int = 0,
                num_splits: int = 0) -> Case:
    """Decode with KV append: cache_seqlens[b] rows are valid, row cache_seqlens[b] is written."""
    g = _gen(seed)
    if cache_seqlens is None:
        cs = torch.randint(1, max_seqlen, (B,), generator=g, dtype=torch.int64).to(torch.int32)
    else:
        cs = torch.as_tensor(cache_seqlens, dtype=torch.int32).reshape(B)
    if page_size == 0:
        q = _randn(g, (B, Hq, D), _q_dtype(dtype))
        k = _randn(g, (B, max_seqlen, Hkv, D), _kv_draw_dtype(dtype))
        v = _randn(g, (B, max_seqlen, Hkv, D), _kv_draw_dtype(dtype))
        rows = torch.arange(max_seqlen)[None, :] >= cs[:, None].to(torch.int64)
        _fill_pad(k, rows, pad, g)
        _fill_pad(v, rows, pad, g)
        table = None
    else:
        # every request owns enough pages for its appended row
        need = [math.ceil((int(c) + 1) / page_size) for c in cs]
        pool = sum(need)
        perm = torch.randperm(pool, generator=g).to(torch.int32)
        max_pages = math.ceil(max_seqlen / page_size)
        table = torch.full((B, max_pages), -1, dtype=torch.int32)
        off = 0
        mask = torch.zeros(pool, page_size, dtype=torch.bool)
        for b, n in enumerate(need):
            table[b, :n] = perm[off:off + n]
            c = int(cs[b])
            last = int(perm[off + n - 1])
            if c % page_size:
                mask[last, c % page_size:] = True
            elif n > c // page_size:
                mask[last, :] = True
            off += n
        q = _randn(g, (B, Hq, D), _q_dtype(dtype))
        k = _randn(g, (pool, page_size, Hkv, D), _kv_draw_dtype(dtype))
        v = _randn(g, (pool, page_size, Hkv, D), _kv_draw_dtype(dtype))
        _fill_pad(k, mask, pad, g)
        _fill_pad(v, mask, pad, g)
    k_new = _randn(g, (B, Hkv, D), _q_dtype(dtype))
    v_new = _randn(g, (B, Hkv, D), _q_dtype(dtype))
    kd = vd = None
    if dtype == FP8:
        # descales drawn after v_new; a request's pages carry its own
        kd, vd = _descales(g, B, Hkv)
        if page_size == 0:
            k = _quantize(k, kd[:, None, :, None])
            v = _quantize(v, vd[:, None, :, None])
        else:
            fk = torch.empty(k.shape[0], Hkv)
            fv = torch.empty(k.shape[0], Hkv)
            for b in range(B):
                pl = table[b][table[b] >= 0].long()
                fk[pl] = kd[b]
                fv[pl] = vd[b]
            k = _quantize(k, fk[:, None, :, None])
            v = _quantize(v, fv[:, None, :, None])
    cos = sin = None
    if rotary_dim > 0:
        cos, sin = rope_tables(max_seqlen, rotary_dim, base)
    return Case(name, dtype, B, Hq, Hkv, D, q, k, v, cs, page_size=page_size, page_table=table,
                k_new=k_new, v_new=v_new, rotary_dim=rotary_dim, rope_base=base, rope_cos=cos,
                rope_sin=sin, num_splits=num_splits, k_descale=kd, v_descale=vd)


def cascade_case(seed: int, B: int, Hq: int, Hkv: int, D: int, prefix_len: int, ps: int,
                 suffix_range=None, suffix_lens=None, dtype=BF16, pad: str = "zero",
                 extra_pages: int = 0, name: str = "cascade") -> Case:
    """Shared prefix (prefix_len tokens in its own pages) + per-request suffix pages, one pool."""
    g = _gen(seed)
    if suffix_lens is None:
        lo, hi = suffix_range
        sl = torch.randint(lo, hi + 1, (B,), generator=g, dtype=torch.int64).to(torch.int32)
    else:
        sl = torch.as_tensor(suffix_lens, dtype=torch.int32).reshape(B)
    n_pre = math.ceil(prefix_len / ps)
    need = [math.ceil(int(L) / ps) for L in sl]
    pool = n_pre + sum(need) + extra_pages
    perm = torch.randperm(pool, generator=g).to(torch.int32)
    prefix_pages = perm[:n_pre].clone()
    max_pages = max(need + [1])
    table = torch.full((B, max_pages), -1, dtype=torch.int32)
    off = n_pre
    mask = torch.zeros(pool, ps, dtype=torch.bool)
    if prefix_len % ps:
        mask[int(prefix_pages[-1]), prefix_len % ps:] = True
    for b, n in enumerate(need):
        table[b, :n] = perm[off:off + n]
        L = int(sl[b])
        if n and L % ps:
            mask[int(perm[off + n - 1]), L % ps:] = True
        off += n
    for p in perm[off:].tolist():
        mask[p, :] = True
    q = _randn(g, (B, Hq, D), _q_dtype(dtype))
    k = _randn(g, (pool, ps, Hkv, D), _kv_draw_dtype(dtype))
    v = _randn(g, (pool, ps, Hkv, D), _kv_draw_dtype(dtype))
    _fill_pad(k, mask, pad, g)
    _fill_pad(v, mask, pad, g)
    kd = vd = None
    if dtype == FP8:
        # a request's own pages carry its descales; the shared prefix pages (and
        # unused ones) are stored at 1/32 and read with each request's descale
        kd, vd = _descales(g, B, Hkv)
        fk = torch.full((pool, Hkv), 1.0 / 32)
        fv = torch.full((pool, Hkv), 1.0 / 32)
        for b in range(B):
            pl = table[b][table[b] >= 0].long()
            fk[pl] = kd[b]
            fv[pl] = vd[b]
        k = _quantize(k, fk[:, None, :, None])
        v = _quantize(v, fv[:, None, :, None])
    return Case(name, dtype, B, Hq, Hkv, D, q, k, v, sl, page_size=ps, page_table=table,
                prefix_pages=prefix_pages, prefix_len=prefix_len, k_descale=kd, v_descale=vd)


def workload(name: str, pad: str = "zero") -> Case:
    """The five named workloads at their full sizes."""
    if name == "c1":
        return contiguous_case(1, 1, 32, 32, 128, [4096], 4096, F16, pad, "c1", num_splits=16)
    if name == "c1f8":  # c1 with a float8 e4m3fn cache (the vector map kernel)
        return contiguous_case(1, 1, 32, 32, 128, [4096], 4096, FP8, pad, "c1f8", num_splits=16)
    if name == "c2":
        return contiguous_case(2, 1, 32, 8, 128, [131072], 131072, BF16, pad, "c2")
    if name == "c2f8":
        return contiguous_case(2, 1, 32, 8, 128, [131072], 131072, FP8, pad, "c2f8")
    if name == "c2g2f8":  # the long-context request, two query heads per KV head, float8 cache (vector kernel)
        return contiguous_case(2, 1, 16, 8, 128, [131072], 131072, FP8, pad, "c2g2f8")
    if name == "c2g8":  # the long-context request with eight query heads per KV head
        return contiguous_case(2, 1, 64, 8, 128, [131072], 131072, BF16, pad, "c2g8")
    if name == "c3f8":
        return paged_case(3, 32, 32, 8, 128, None, 16, FP8, max_pages=512, pad=pad, name="c3f8",
                          lens_range=(512, 8192))
    if name == "c3":
        return paged_case(3, 32, 32, 8, 128, None, 16, BF16, max_pages=512, pad=pad, name="c3",
                          lens_range=(512, 8192))
    if name == "c4":
        return append_case(4, 4, 32, 8, 128, 2048, F16, rotary_dim=128, base=10000.0, pad=pad,
                           name="c4")
    if name == "c5":
        return cascade_case(5, 64, 32, 8, 128, 16384, 64, suffix_range=(256, 2048), dtype=BF16,
                            pad=pad, name="c5")
    if name == "c5f8":  # c5 with a float8 e4m3fn page pool
        return cascade_case(5, 64, 32, 8, 128, 16384, 64, suffix_range=(256, 2048), dtype=FP8,
                            pad=pad, name="c5f8")
    raise KeyError(name)


WORKLOADS = ("c1", "c2", "c3", "c4", "c5")
