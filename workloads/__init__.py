"""Seeded synthetic inputs for the DSA path, shared by the oracle side and the GPU side.

This module draws random tensors and lays them out; it holds none of the method's
arithmetic.  Both sides receive the very same bytes.

Shapes follow the model the pages describe ("DeepSeek-V3.2" model docs, section 1
"Model Introduction": 128 query heads, KV-LoRA latent 512 + 64 RoPE dims, indexer
64 heads x 128 dims, index_topk 2048; section 5.3 "Rollout & SGLang": bf16 latent
cache in 64-token pages).

Draw recipe (fixed order, so a seed names the inputs exactly):
  * structure (sequence lengths, physical page permutation) from a CPU
    ``torch.Generator`` seeded with ``seed``;
  * values from a ``torch.Generator`` on the target device seeded with ``seed``, in
    the order q^I, k^I, w, q, kv.  Normal draws are fp32 and then rounded to bf16
    (round to nearest even) or quantised to OCP e4m3 with a per-token scale
    amax/448 (round to nearest even; the scale keeps every code finite).
Drawing on the GPU is only a speed measure for the large shapes; the oracle is
always handed copies of the device bytes.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

PAGE = 64
E4M3_MAX = 448.0


@dataclass
class Workload:
    name: str
    mode: str                 # "decode" | "prefill"
    idx_dtype: str            # "f32" | "bf16" | "fp8"
    mla_dtype: str            # "f32" | "bf16"
    H_I: int
    D_I: int
    H: int
    D_qk: int
    D_v: int
    topk: int
    scale: float
    num_seqs: int
    max_row_len: int
    row_seq: torch.Tensor     # int32 [R]
    row_len: torch.Tensor     # int32 [R]
    seq_start: Optional[torch.Tensor]   # int64 [B] (contiguous cache) or None
    page_table: Optional[torch.Tensor]  # int32 [B, max_pages] (paged cache) or None
    page_size: int
    q_idx: torch.Tensor       # [R, H_I, D_I]
    q_scale: Optional[torch.Tensor]     # f32 [R, H_I] (fp8 only)
    k_idx: torch.Tensor       # [N, D_I] or [P, page, D_I]
    k_scale: Optional[torch.Tensor]     # f32 [N] or [P, page] (fp8 only)
    w: torch.Tensor           # f32 [R, H_I]
    q: torch.Tensor           # [R, H, D_qk]
    kv: torch.Tensor          # [N, D_qk] or [P, page, D_qk]
    lens: list = field(default_factory=list)   # per-sequence context lengths (host ints)

    @property
    def num_rows(self) -> int:
        return int(self.row_seq.shape[0])

    @property
    def paged(self) -> bool:
        return self.page_table is not None

    def to(self, device) -> "Workload":
        kw = {}
        for f in self.__dataclass_fields__:
            v = getattr(self, f)
            kw[f] = v.to(device) if isinstance(v, torch.Tensor) else v
        return Workload(**kw)

    def host_rows(self) -> dict:
        """Row description as numpy arrays (for any host-side consumer)."""
        return {
            "row_seq": self.row_seq.cpu().numpy(),
            "row_len": self.row_len.cpu().numpy(),
            "seq_start": None if self.seq_start is None else self.seq_start.cpu().numpy(),
            "page_table": None if self.page_table is None else self.page_table.cpu().numpy(),
            "page_size": self.page_size,
        }


def raw_numpy(t: Optional[torch.Tensor]) -> Optional[np.ndarray]:
    """Host copy of a tensor's bits: bf16 -> uint16, e4m3 -> uint8, others unchanged."""
    if t is None:
        return None
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()


def _normal(shape, gen, device):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)


def _round(x: torch.Tensor, dtype: str) -> torch.Tensor:
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return x.to(torch.bfloat16)
    raise ValueError(dtype)


def quantize_e4m3(x: torch.Tensor, token_dims: int):
    """Per-token OCP e4m3 codes: scale = amax / 448 over all but the first ``token_dims`` dims."""
    red = tuple(range(token_dims, x.dim()))
    amax = x.abs().amax(dim=red, keepdim=True)
    scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    codes = (x / scale).to(torch.float8_e4m3fn)
    return codes, scale.reshape(x.shape[:token_dims])


def _draw_values(wl_shapes: dict, idx_dtype: str, mla_dtype: str, w_div: float, seed: int,
                 device) -> dict:
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    R, H_I, D_I = wl_shapes["q_idx"]
    kshape = wl_shapes["k_idx"]
    out = {}
    qi = _normal((R, H_I, D_I), gen, device)
    ki = _normal(kshape, gen, device)
    if idx_dtype == "fp8":
        out["q_idx"], qs = quantize_e4m3(qi, 1)                  # one scale per query token
        out["q_scale"] = qs[:, None].expand(R, H_I).contiguous()
        out["k_idx"], out["k_scale"] = quantize_e4m3(ki, len(kshape) - 1)
    else:
        out["q_idx"], out["q_scale"] = _round(qi, idx_dtype), None
        out["k_idx"], out["k_scale"] = _round(ki, idx_dtype), None
    del qi, ki
    out["w"] = torch.rand((R, H_I), generator=gen, device=device, dtype=torch.float32) / w_div
    out["q"] = _round(_normal(wl_shapes["q"], gen, device), mla_dtype)
    out["kv"] = _round(_normal(wl_shapes["kv"], gen, device), mla_dtype)
    return out


def decode(lens, *, idx_dtype="bf16", mla_dtype="bf16", paged=False, H_I=64, D_I=128, H=128,
           D_qk=576, D_v=512, topk=2048, scale=None, w_div=8.0, seed=0, device="cpu",
           name="decode") -> Workload:
    """One query token per sequence, attending to its whole cache (own token included)."""
    lens = [int(x) for x in lens]
    if not lens or min(lens) < 1:
        raise ValueError("every sequence needs at least one token")
    B = len(lens)
    sgen = torch.Generator()
    sgen.manual_seed(seed)
    if paged:
        npages = [math.ceil(n / PAGE) for n in lens]
        P = sum(npages)
        perm = torch.randperm(P, generator=sgen).to(torch.int32)
        max_pages = max(npages)
        pt = torch.full((B, max_pages), -1, dtype=torch.int32)
        off = 0
        for b, n in enumerate(npages):
            pt[b, :n] = perm[off:off + n]
            off += n
        kshape, kvshape = (P, PAGE, D_I), (P, PAGE, D_qk)
        seq_start = None
    else:
        starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
        seq_start = torch.from_numpy(starts)
        pt = None
        N = sum(lens)
        kshape, kvshape = (N, D_I), (N, D_qk)
    vals = _draw_values({"q_idx": (B, H_I, D_I), "k_idx": kshape, "q": (B, H, D_qk), "kv": kvshape},
                        idx_dtype, mla_dtype, w_div, seed, device)
    return Workload(
        name=name, mode="decode", idx_dtype=idx_dtype, mla_dtype=mla_dtype, H_I=H_I, D_I=D_I, H=H,
        D_qk=D_qk, D_v=D_v, topk=topk, scale=scale if scale is not None else 1.0 / math.sqrt(192.0),
        num_seqs=B, max_row_len=max(lens),
        row_seq=torch.arange(B, dtype=torch.int32, device=device),
        row_len=torch.tensor(lens, dtype=torch.int32, device=device),
        seq_start=None if seq_start is None else seq_start.to(device),
        page_table=None if pt is None else pt.to(device), page_size=PAGE,
        lens=lens, **vals)


def prefill(L, *, idx_dtype="bf16", mla_dtype="bf16", H_I=64, D_I=128, H=128, D_qk=576, D_v=512,
            topk=2048, scale=None, w_div=8.0, seed=0, device="cpu", name="prefill") -> Workload:
    """One sequence of L tokens; row t attends causally to positions 0..t."""
    L = int(L)
    vals = _draw_values({"q_idx": (L, H_I, D_I), "k_idx": (L, D_I), "q": (L, H, D_qk), "kv": (L, D_qk)},
                        idx_dtype, mla_dtype, w_div, seed, device)
    return Workload(
        name=name, mode="prefill", idx_dtype=idx_dtype, mla_dtype=mla_dtype, H_I=H_I, D_I=D_I, H=H,
        D_qk=D_qk, D_v=D_v, topk=topk, scale=scale if scale is not None else 1.0 / math.sqrt(192.0),
        num_seqs=1, max_row_len=L,
        row_seq=torch.zeros(L, dtype=torch.int32, device=device),
        row_len=torch.arange(1, L + 1, dtype=torch.int32, device=device),
        seq_start=torch.zeros(1, dtype=torch.int64, device=device), page_table=None,
        page_size=PAGE, lens=[L], **vals)


def prefill_batch(lens, *, new=None, idx_dtype="bf16", mla_dtype="bf16", paged=False, H_I=64,
                  D_I=128, H=128, D_qk=576, D_v=512, topk=2048, scale=None, w_div=8.0, seed=0,
                  device="cpu", name="prefill_batch") -> Workload:
    """Several sequences prefilled together: the last new[b] tokens of sequence b (all of them
    when new is None) are query rows, in sequence order; row t of b attends causally to
    positions 0..t of b.  new[b] < lens[b] is a chunk of prefill over a cached prefix."""
    lens = [int(x) for x in lens]
    if not lens or min(lens) < 1:
        raise ValueError("every sequence needs at least one token")
    new = list(lens) if new is None else [int(x) for x in new]
    if len(new) != len(lens) or min(new) < 1 or any(n > l for n, l in zip(new, lens)):
        raise ValueError("each sequence needs 1 .. len query rows")
    B = len(lens)
    R = sum(new)
    N = sum(lens)
    sgen = torch.Generator()
    sgen.manual_seed(seed)
    if paged:
        npages = [math.ceil(n / PAGE) for n in lens]
        P = sum(npages)
        perm = torch.randperm(P, generator=sgen).to(torch.int32)
        pt = torch.full((B, max(npages)), -1, dtype=torch.int32)
        off = 0
        for b, n in enumerate(npages):
            pt[b, :n] = perm[off:off + n]
            off += n
        kshape, kvshape = (P, PAGE, D_I), (P, PAGE, D_qk)
        seq_start = None
    else:
        seq_start = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64))
        pt = None
        kshape, kvshape = (N, D_I), (N, D_qk)
    vals = _draw_values({"q_idx": (R, H_I, D_I), "k_idx": kshape, "q": (R, H, D_qk), "kv": kvshape},
                        idx_dtype, mla_dtype, w_div, seed, device)
    row_seq = torch.cat([torch.full((n,), b, dtype=torch.int32) for b, n in enumerate(new)])
    row_len = torch.cat([torch.arange(l - n + 1, l + 1, dtype=torch.int32)
                         for n, l in zip(new, lens)])
    return Workload(
        name=name, mode="prefill", idx_dtype=idx_dtype, mla_dtype=mla_dtype, H_I=H_I, D_I=D_I, H=H,
        D_qk=D_qk, D_v=D_v, topk=topk, scale=scale if scale is not None else 1.0 / math.sqrt(192.0),
        num_seqs=B, max_row_len=max(lens), row_seq=row_seq.to(device), row_len=row_len.to(device),
        seq_start=None if seq_start is None else seq_start.to(device),
        page_table=None if pt is None else pt.to(device), page_size=PAGE, lens=lens, **vals)


def c5_lengths(seed: int, B: int = 32):
    """Mixed context lengths ~ U[1024, 65536]; sequences 0-1 redrawn from U[1024, 2047]."""
    g = torch.Generator()
    g.manual_seed(seed + 7919)
    lens = torch.randint(1024, 65537, (B,), generator=g)
    lens[:2] = torch.randint(1024, 2048, (2,), generator=g)
    return [int(x) for x in lens]


CONFIGS = {
    1: "tiny fp32 prefill: L=256, indexer 4x32, top-64, MLA 8 heads 80/64, scale 1/sqrt(80)",
    2: "decode 8K bf16: 64 sequences x 8192 ctx, indexer 64x128, top-2048, MLA 128 heads 576/512",
    3: "prefill 16K bf16: 1 sequence, L=16384, causal, indexer 64x128, top-2048, MLA 128x576/512",
    4: "decode 128K: 8 sequences x 131072 ctx, fp8 e4m3 indexer with per-token scales, bf16 latents",
    5: "paged mixed decode: 32 sequences, ctx ~ U[1024, 65536], 64-token pages, bf16",
}


def config(n: int, device="cpu", seed: Optional[int] = None) -> Workload:
    """The five named workloads; seed defaults to 1000 + n."""
    seed = 1000 + n if seed is None else seed
    if n == 1:
        return prefill(256, idx_dtype="f32", mla_dtype="f32", H_I=4, D_I=32, H=8, D_qk=80, D_v=64,
                       topk=64, scale=1.0 / math.sqrt(80.0), w_div=1.0, seed=seed, device=device,
                       name="c1_tiny_fp32_prefill_L256")
    if n == 2:
        return decode([8192] * 64, seed=seed, device=device, name="c2_decode_8k_bf16_b64")
    if n == 3:
        return prefill(16384, seed=seed, device=device, name="c3_prefill_16k_bf16")
    if n == 4:
        return decode([131072] * 8, idx_dtype="fp8", seed=seed, device=device,
                      name="c4_decode_128k_fp8idx_b8")
    if n == 5:
        return decode(c5_lengths(seed), paged=True, seed=seed, device=device,
                      name="c5_paged_mixed_decode_b32")
    raise ValueError(f"no config {n}")


# --------------------------------------------------------------------------- input prep

@dataclass
class PrepBatch:
    """New tokens about to be written into the caches, and their query rows (one per token)."""
    idx_dtype: str            # "bf16" | "fp8": the indexer cache format
    positions: torch.Tensor   # int32 [T]
    cache_rows: torch.Tensor  # int64 [T]: flat cache row of each token (-1: padding)
    cos_sin: torch.Tensor     # f32 [max_pos, 64]: cos then sin of the 32 angles per position
    k_idx_in: torch.Tensor    # bf16 [T, 128]
    kv_in: torch.Tensor       # bf16 [T, 576]
    k_cache: torch.Tensor     # [rows, 128]: bf16, or uint8 e4m3 codes (fp8); random contents
    k_scale: Optional[torch.Tensor]   # f32 [rows] (fp8)
    kv_cache: torch.Tensor    # bf16 [rows, 576]; random contents
    q_idx_in: torch.Tensor    # bf16 [T, 64, 128]
    q: torch.Tensor           # bf16 [T, H, 576]
    seq_start: Optional[torch.Tensor]    # int64 [B] (contiguous cache) or None
    page_table: Optional[torch.Tensor]   # int32 [B, max_pages] (paged cache) or None


def rope_table(max_pos: int, base: float = 10000.0) -> torch.Tensor:
    """A frequency schedule for the tests: angle i of position p is p * base^(-i/32)."""
    i = torch.arange(32, dtype=torch.float64)
    ang = torch.arange(max_pos, dtype=torch.float64)[:, None] * base ** (-i / 32.0)[None, :]
    return torch.cat([ang.cos(), ang.sin()], dim=1).to(torch.float32)


def prep_batch(lens, new, *, idx_dtype="fp8", paged=False, H=128, pad=0, seed=0,
               device="cpu") -> PrepBatch:
    """The last new[b] tokens of sequences of lengths lens[b], their cache rows in a contiguous
    cache (sequences back to back) or a paged one (a random permutation of 64-token pages),
    plus ``pad`` padding tokens (row -1); the caches start with random contents."""
    lens = [int(x) for x in lens]
    new = [int(x) for x in new]
    if len(new) != len(lens) or min(new) < 1 or any(n > l for n, l in zip(new, lens)):
        raise ValueError("each sequence needs 1 .. len new tokens")
    sgen = torch.Generator()
    sgen.manual_seed(seed)
    pos = torch.cat([torch.arange(l - n, l, dtype=torch.int64) for n, l in zip(new, lens)])
    seq = torch.cat([torch.full((n,), b, dtype=torch.int64) for b, n in enumerate(new)])
    if paged:
        pages = [(l + PAGE - 1) // PAGE for l in lens]
        perm = torch.randperm(sum(pages), generator=sgen)
        first = np.concatenate([[0], np.cumsum(pages)[:-1]]).astype(np.int64)
        phys = perm[torch.from_numpy(first)[seq] + pos // PAGE]
        rows = phys * PAGE + pos % PAGE
        n_rows = sum(pages) * PAGE
        page_table = torch.full((len(lens), max(pages)), -1, dtype=torch.int32)
        for b, (f, n) in enumerate(zip(first, pages)):
            page_table[b, :n] = perm[f:f + n].to(torch.int32)
        start = None
    else:
        start = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64))
        rows = start[seq] + pos
        n_rows = sum(lens)
        page_table = None
    rows = torch.cat([rows, torch.full((pad,), -1, dtype=torch.int64)])
    pos = torch.cat([pos, torch.zeros(pad, dtype=torch.int64)]).to(torch.int32)
    T = int(pos.numel())
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    k_idx_in = _normal((T, 128), gen, device).to(torch.bfloat16)
    kv_in = _normal((T, 576), gen, device).to(torch.bfloat16)
    q_idx_in = _normal((T, 64, 128), gen, device).to(torch.bfloat16)
    q = _normal((T, H, 576), gen, device).to(torch.bfloat16)
    kv_cache = _normal((n_rows, 576), gen, device).to(torch.bfloat16)
    if idx_dtype == "fp8":
        codes = torch.randint(0, 0x7F, (n_rows, 128), generator=gen, device=device, dtype=torch.int32)
        sign = torch.randint(0, 2, (n_rows, 128), generator=gen, device=device, dtype=torch.int32)
        k_cache = (codes | (sign << 7)).to(torch.uint8)
        k_scale = torch.rand((n_rows,), generator=gen, device=device, dtype=torch.float32)
    elif idx_dtype == "bf16":
        k_cache = _normal((n_rows, 128), gen, device).to(torch.bfloat16)
        k_scale = None
    else:
        raise ValueError(idx_dtype)
    return PrepBatch(idx_dtype, pos.to(device), rows.to(device),
                     rope_table(max(lens) + 1).to(device), k_idx_in, kv_in, k_cache, k_scale,
                     kv_cache, q_idx_in, q, None if start is None else start.to(device),
                     None if page_table is None else page_table.to(device))


# --------------------------------------------------------------------------- masked MHA mode

@dataclass
class MhaBatch:
    """A prefill batch for the MHA mode: the layout and latent cache of a prefill_batch plus
    per-head 192-dim queries and the up-projections W_UK, W_UV."""
    wl: Workload              # rows, cache layout and the latent cache kv
    q: torch.Tensor           # bf16 [R, H, 192]
    w_uk: torch.Tensor        # bf16 [H, 128, 512]
    w_uv: torch.Tensor        # bf16 [H, 128, 512]
    scale: float


def mha_batch(lens, *, new=None, H=128, H_I=4, paged=False, seed=0, device="cpu") -> MhaBatch:
    """Rows, latent cache and bf16 indexer inputs (H_I heads of 128 dims: the model's 64 where
    the indexer runs, else a tiny unused set) as prefill_batch, then from the same device
    generator stream: q ~ N(0,1), W_UK and W_UV ~ N(0, 1/512) (keys and values of unit scale),
    all bf16."""
    wl = prefill_batch(lens, new=new, paged=paged, H=H, H_I=H_I, D_I=128, seed=seed,
                       device=device, name="mha_batch")
    gen = torch.Generator(device=device)
    gen.manual_seed(seed + 1)
    R = wl.num_rows
    q = _normal((R, H, 192), gen, device).to(torch.bfloat16)
    w_uk = (_normal((H, 128, 512), gen, device) / math.sqrt(512.0)).to(torch.bfloat16)
    w_uv = (_normal((H, 128, 512), gen, device) / math.sqrt(512.0)).to(torch.bfloat16)
    return MhaBatch(wl, q, w_uk, w_uv, 1.0 / math.sqrt(192.0))
