"""Seeded synthetic inputs for the Vegas attention hot path.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic, and it imports nothing else from this package.  Both the
GPU path and the CPU oracle are fed from it (the oracle receives the exact
bits the GPU reads, copied to the host).

Recipe (the same for every workload shape):
  * keys and values ~ N(0, 1), drawn in fp32 and rounded once (RNE) to the
    storage dtype; the gamma+1 new rows of each sequence are drawn the same
    way and carry no plants;
  * per (sequence, KV head) a random unit direction u;
  * planted prefix keys: heavy hitters (+hh_gain*u), attention sinks at the
    first positions (+sink_gain*u), a recency band on the last prefix keys
    (+recency_gain*u); plants add where they overlap;
  * every query row (verification rows and the fresh draft queries) is
    u_{g(h)} + N(0, q_sigma^2);
  * k_b = floor(ratio * L_b) selected positions per sequence.
The pages measure on reasoning and long-document benchmarks whose token
streams are not available here; these shapes stand in for them.
"""
from __future__ import annotations

import dataclasses
import math
from fractions import Fraction
from typing import List, Optional

import torch


@dataclasses.dataclass
class Workload:
    name: str
    dtype: str                    # "f32" or "bf16"
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    gamma: int
    prefix_lens: List[int]        # committed prefix length L_b per sequence
    ratio: Fraction               # k_b = floor(ratio * L_b)
    q_sigma: float
    hh_count: Optional[int] = None        # heavy hitters per sequence (None: hh_frac * L_b)
    hh_frac: Fraction = Fraction(0)
    hh_gain: float = 0.0
    hh_run: int = 1                       # >1: heavy hitters come in runs of this many tokens
    sink_count: int = 0
    sink_gain: float = 0.0
    recency_count: int = 0
    recency_gain: float = 0.0
    layers: int = 1
    draft_steps: Optional[int] = None     # defaults to gamma

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def rows_per_seq(self) -> int:
        return self.gamma + 1

    @property
    def seqlens(self) -> List[int]:
        return [L + self.gamma + 1 for L in self.prefix_lens]

    @property
    def k_per_seq(self) -> List[int]:
        return [int(self.ratio * L) for L in self.prefix_lens]   # floor for non-negative L

    @property
    def n_drafts(self) -> int:
        return self.gamma if self.draft_steps is None else self.draft_steps

    def cu_seqlens(self) -> List[int]:
        out = [0]
        for n in self.seqlens:
            out.append(out[-1] + n)
        return out

    def cu_k(self) -> List[int]:
        out = [0]
        for kb in self.k_per_seq:
            out.append(out[-1] + kb)
        return out

    @property
    def total_kv(self) -> int:
        return sum(self.seqlens)


def _ragged_prefixes(batch: int, lo: int, hi: int, seed: int) -> List[int]:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    u = torch.rand(batch, generator=g, dtype=torch.float64)
    return [int(math.floor(math.exp(math.log(lo) + float(x) * (math.log(hi) - math.log(lo)))))
            for x in u]


def named_workload(i: int, seed: int = 0) -> Workload:
    """The five benchmark/test shapes, 0-based."""
    if i == 0:
        return Workload("tiny-mqa-fp32 B1 Hq4 Hkv1 D64 L1024 gamma3 k5%", "f32", 1, 4, 1, 64, 3,
                        [1024], Fraction(5, 100), q_sigma=0.5, hh_count=10, hh_gain=3.0,
                        draft_steps=3)
    qwen_plants = dict(hh_frac=Fraction(2, 100), hh_gain=2.5, sink_count=4, sink_gain=4.0,
                       recency_count=256, recency_gain=1.5)
    if i == 1:
        return Workload("qwen3-8b-layer B4 Hq32 Hkv8 D128 L32768 gamma4 k5% bf16", "bf16", 4, 32, 8,
                        128, 4, [32768] * 4, Fraction(5, 100), q_sigma=0.7, **qwen_plants)
    if i == 2:
        return Workload("qwen3-8b-128k-step B4 Hq32 Hkv8 D128 L131072 gamma5 k5% bf16 x36 layers",
                        "bf16", 4, 32, 8, 128, 5, [131072] * 4, Fraction(5, 100), q_sigma=0.7,
                        layers=36, **qwen_plants)
    if i == 3:
        return Workload("qwen3-32b-layer B8 Hq64 Hkv8 D128 L65536 gamma6 k10% bf16 clustered",
                        "bf16", 8, 64, 8, 128, 6, [65536] * 8, Fraction(10, 100), q_sigma=0.7,
                        hh_run=64, **qwen_plants)
    if i == 4:
        prefixes = _ragged_prefixes(16, 4096, 131072, seed)
        return Workload("gpt-oss-20b-layer ragged B16 Hq64 Hkv8 D64 L~logU(4K,128K) gamma3 k5% bf16",
                        "bf16", 16, 64, 8, 64, 3, prefixes, Fraction(5, 100), q_sigma=0.7,
                        **qwen_plants)
    raise ValueError(f"no workload {i}")


def custom_workload(dtype: str, batch: int, hq: int, hkv: int, d: int, gamma: int,
                    prefix_lens: List[int], ratio=Fraction(5, 100), q_sigma: float = 0.7,
                    plants: bool = True, draft_steps: Optional[int] = None) -> Workload:
    """An arbitrary shape with the planted structure of the Qwen3-8B layer scaled down."""
    kw = {}
    if plants:
        kw = dict(hh_frac=Fraction(2, 100), hh_gain=2.5, sink_count=min(4, min(prefix_lens)),
                  sink_gain=4.0, recency_count=min(256, min(prefix_lens)), recency_gain=1.5)
    return Workload(f"custom {dtype} B{batch} Hq{hq} Hkv{hkv} D{d} gamma{gamma}", dtype, batch,
                    hq, hkv, d, gamma, list(prefix_lens), Fraction(ratio), q_sigma=q_sigma,
                    draft_steps=draft_steps, **kw)


def _hh_positions(wl: Workload, L: int, gen: torch.Generator) -> torch.Tensor:
    if L <= 0:
        return torch.zeros(0, dtype=torch.long)
    if wl.hh_count is not None:
        n = min(wl.hh_count, L)
    else:
        n = int(wl.hh_frac * L)
    if n == 0:
        return torch.zeros(0, dtype=torch.long)
    if wl.hh_run <= 1:
        return torch.randperm(L, generator=gen)[:n]
    runs = n // wl.hh_run
    slots = L // wl.hh_run
    if runs == 0 or slots < 2:
        return torch.zeros(0, dtype=torch.long)
    chosen = torch.randperm(slots - 1, generator=gen)[:runs]
    shift = int(torch.randint(0, wl.hh_run, (1,), generator=gen))
    starts = chosen * wl.hh_run + shift
    return (starts[:, None] + torch.arange(wl.hh_run)[None, :]).reshape(-1)


def heavy_hitter_positions(wl: Workload, seed: int = 0, layer: int = 0) -> List[torch.Tensor]:
    """The planted heavy-hitter positions of every sequence, as make_inputs draws them for the
    same seed and layer (the only draws of its host-side generator)."""
    cpu_gen = torch.Generator(device="cpu")
    cpu_gen.manual_seed(seed * 1000003 + layer + 7919)
    return [_hh_positions(wl, L, cpu_gen) for L in wl.prefix_lens]


def _unit(n_rows: int, d: int, gen: torch.Generator, device) -> torch.Tensor:
    u = torch.randn(n_rows, d, generator=gen, device=device, dtype=torch.float32)
    return u / u.norm(dim=-1, keepdim=True)


# Where the device KV caches drawn here sit: each layer's K and V share one allocation, V starting
# KV_GAP_BYTES + KV_OFFSET_BYTES past the end of K (rounded up to 2 MB).  Both passes read the K
# and V rows of the same positions together, so how fast a call runs depends on where the two
# tensors sit relative to each other (measured on one MI355X, 128K Qwen3-8B-shaped layer,
# verification with collection):
#   * modulo 2 MB: with V and K congruent, as two large allocations usually are, the same heads'
#     slices of K and V meet in the memory system and two of the eight KV heads read ~4% slower,
#     which sets the end of every call (128K step: 474.7 us per layer-step against 467.2-468.6
#     with V 256, 512 or 768 bytes away);
#   * beyond 2 MB: with V 1 GiB + 10 MiB + 512 B from K a call took 320-323 us, with V 1 GiB +
#     2 MiB + 512 B or 2 GiB + 10 MiB + 512 B away 339-340 us, and two separate allocations read
#     anywhere between the two from layer to layer (two K/V placements interleaved in one process:
#     460.7 against 468.0 us per layer-step).  One allocation keeps the distance what is asked.
# At this workload's size the rule below puts V 1 GiB + 10 MiB + 512 B from K; the 32K and the
# gpt-oss-shaped layers read the same for every distance tried.
KV_OFFSET_BYTES = 512
KV_GAP_BYTES = 8 << 20
_TWO_MB = 2 << 20


def kv_cache_pair(total: int, hkv: int, d: int, dtype, device):
    """Empty K and V caches [total, hkv, d]; on a GPU both live in one allocation, V starting
    KV_GAP_BYTES + KV_OFFSET_BYTES past K's end rounded up to 2 MB, K at a 2 MB boundary (see
    above).  Both are contiguous and 16-byte aligned."""
    dev = torch.device(device)
    if dev.type != "cuda":
        return (torch.empty(total, hkv, d, dtype=dtype, device=dev),
                torch.empty(total, hkv, d, dtype=dtype, device=dev))
    nbytes = total * hkv * d * torch.empty(0, dtype=dtype).element_size()
    vstart = (nbytes + _TWO_MB - 1) // _TWO_MB * _TWO_MB + KV_GAP_BYTES + KV_OFFSET_BYTES
    raw = torch.empty(vstart + nbytes + _TWO_MB, dtype=torch.uint8, device=dev)
    a0 = (-raw.data_ptr()) % _TWO_MB
    k = raw[a0: a0 + nbytes].view(dtype).view(total, hkv, d)
    v = raw[a0 + vstart: a0 + vstart + nbytes].view(dtype).view(total, hkv, d)
    return k, v


def make_inputs(wl: Workload, seed: int = 0, device="cpu", layer: int = 0, out: dict | None = None):
    """Draw one layer's inputs on `device` (a torch device string).

    Returns a dict of torch tensors on `device`:
      q        [batch*(gamma+1), Hq, D]   verification queries
      k, v     [total_kv, Hkv, D]         (kv_cache_pair: K and V in one allocation)
      cu_seqlens_k, cu_k  int32 [batch+1]
      draft_q  [n_drafts, batch, Hq, D]   fresh draft queries, one set per draft step
    If `out` holds preallocated k/v tensors of the right shape they are filled in place.
    """
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed * 1000003 + layer)
    hh_all = heavy_hitter_positions(wl, seed, layer)
    B, Hq, Hkv, D, W = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.gamma + 1
    G = Hq // Hkv
    cu = wl.cu_seqlens()
    total = cu[-1]
    dt = wl.torch_dtype
    res = {} if out is None else out

    def fits(t):
        return t is not None and tuple(t.shape) == (total, Hkv, D) and t.dtype == dt and t.device == dev

    if not (fits(res.get("k")) and fits(res.get("v"))):
        res["k"], res["v"] = kv_cache_pair(total, Hkv, D, dt, dev)
    u = _unit(B * Hkv, D, gen, dev).view(B, Hkv, D)
    for b in range(B):
        s0, s1 = cu[b], cu[b + 1]
        L = wl.prefix_lens[b]
        kf = torch.randn(s1 - s0, Hkv, D, generator=gen, device=dev, dtype=torch.float32)
        gain = torch.zeros(s1 - s0, dtype=torch.float32)
        hh = hh_all[b]
        if hh.numel():
            gain.index_add_(0, hh, torch.full((hh.numel(),), wl.hh_gain))
        if wl.sink_count:
            gain[: min(wl.sink_count, L)] += wl.sink_gain
        if wl.recency_count and L > 0:
            gain[max(0, L - wl.recency_count): L] += wl.recency_gain
        gain = gain.to(dev)
        kf += gain[:, None, None] * u[b][None, :, :]
        res["k"][s0:s1].copy_(kf.to(dt))
        del kf
        vf = torch.randn(s1 - s0, Hkv, D, generator=gen, device=dev, dtype=torch.float32)
        res["v"][s0:s1].copy_(vf.to(dt))
        del vf
    ug = u.repeat_interleave(G, dim=1)                       # [B, Hq, D]
    qf = ug[:, None] + wl.q_sigma * torch.randn(B, W, Hq, D, generator=gen, device=dev)
    res["q"] = qf.reshape(B * W, Hq, D).to(dt).contiguous()
    nd = max(wl.n_drafts, 1)
    df = ug[None] + wl.q_sigma * torch.randn(nd, B, Hq, D, generator=gen, device=dev)
    res["draft_q"] = df.to(dt).contiguous()
    res["cu_seqlens_k"] = torch.tensor(cu, dtype=torch.int32, device=dev)
    res["cu_k"] = torch.tensor(wl.cu_k(), dtype=torch.int32, device=dev)
    return res


def host_bits(t: torch.Tensor):
    """numpy view of a tensor's element bits as the oracle takes them
    (float32 stays float32; bfloat16 becomes its uint16 bit pattern)."""
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    if t.dtype == torch.float32:
        return t.numpy()
    if t.dtype == torch.int32:
        return t.numpy()
    raise TypeError(f"unsupported dtype {t.dtype}")


def page_cache(wl: Workload, inp: dict, page_size: int, seed: int = 0, spare_pages: int = 3,
               drop_contiguous: bool = False) -> dict:
    """Lay the contiguous K/V of `inp` out as a paged cache: the token rows of every sequence
    are cut into pages of `page_size` rows and the pages are scattered over a randomly
    permuted page pool (with a few unused pages).  A data layout only: no values change.

    Returns {"k_pool", "v_pool": [num_pages, page_size, Hkv, D] (kv_cache_pair: on a GPU the V pool
    sits past the K pool in the same allocation), "block_table": int32 [batch, max_pages]
    (unused slots point at pool page 0), "num_pages"}.
    """
    k, v = inp["k"], inp["v"]
    dev = k.device
    cu = wl.cu_seqlens()
    lens = wl.seqlens
    per = [(n + page_size - 1) // page_size for n in lens]
    maxp = max(per)
    num_pages = sum(per) + spare_pages
    g = torch.Generator(device="cpu")
    g.manual_seed(seed * 7919 + page_size)
    perm = torch.randperm(num_pages, generator=g)
    Hkv, D = k.shape[1], k.shape[2]
    out = {"num_pages": num_pages}
    bt = torch.zeros(wl.batch, maxp, dtype=torch.int32)
    used = 0
    for b in range(wl.batch):
        bt[b, : per[b]] = perm[used: used + per[b]].to(torch.int32)
        used += per[b]
    out["block_table"] = bt.to(dev)
    pools = kv_cache_pair(num_pages * page_size, Hkv, D, k.dtype, dev)   # V off K, as the contiguous caches
    for (name, src), pool in zip((("k", k), ("v", v)), pools):
        pool.zero_()
        for b in range(wl.batch):
            t = torch.arange(lens[b], device=dev)
            rows = out["block_table"][b].long()[t // page_size] * page_size + t % page_size
            pool.index_copy_(0, rows, src[cu[b]: cu[b + 1]])
        out[name + "_pool"] = pool.view(num_pages, page_size, Hkv, D)
        if drop_contiguous:
            inp[name] = None
    return out


def make_accept_inputs(batch: int, gamma: int, vocab: int, seed: int = 0, device="cpu", draft_noise: float = 0.6,
                       temperature: float = 1.0) -> dict:
    """Seeded inputs of the acceptance step: target rows p [batch, gamma+1, vocab] and draft
    rows q [batch, gamma, vocab] (softmax of correlated random logits), draft tokens drawn from
    q, and the uniforms the method draws.  Random numbers only."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed * 1000003 + 17)
    base = torch.randn(batch, gamma + 1, vocab, generator=g) * 3.0
    p = torch.softmax(base / temperature, dim=-1)
    noisy = base[:, :gamma] + draft_noise * torch.randn(batch, gamma, vocab, generator=g)
    q = torch.softmax(noisy / temperature, dim=-1)
    draft = (torch.multinomial(q.reshape(-1, vocab), 1, generator=g).reshape(batch, gamma).to(torch.int32)
             if gamma > 0 else torch.zeros(batch, 0, dtype=torch.int32))
    out = {"p": p.float(), "q": q.float(), "draft": draft,
           "u_accept": torch.rand(batch, gamma, generator=g), "u_sample": torch.rand(batch, generator=g)}
    return {k: v.contiguous().to(device) for k, v in out.items()}
