"""Seeded synthetic inputs for the workloads (shared by tests, smoke check and benchmark).

This module draws random tensors and lays them out; it holds none of the method's
arithmetic (no scores, no selection, no attention).  bf16 tensors are produced by
rounding fp32 draws to nearest-even; the oracle receives the same values widened back to
fp32, which is exact.

Workloads (sizes and distributions; "N(0, s2)" means variance s2):
  tiny_prefill      1 sequence, L=256, fp32; indexer H_I=4, d_I=32, q_idx, k_idx ~ N(0,1/32),
                    w ~ U(0,1); attention 4 heads of width 64 with their own k, v,
                    q, k, v ~ N(0,1); top-k 32 (and 256, which selects everything).
  prefill_8k        1 sequence, L=8192, bf16; indexer H_I=64, d_I=128, w ~ N(0,1/64); latent
                    attention: 16 query heads of width 576 over one shared 576-wide row per
                    token whose first 512 columns are the value; activations ~ N(0,1); k=2048.
  prefill_128k      as prefill_8k with L=131072, and 1% of the positions (floor(0.01 L),
                    drawn without replacement) get both their index key and latent row
                    scaled by 4 (salient tokens).
  decode_b64        64 sequences, one new token each, context lengths uniform in
                    [16384, 65536]; paged bf16 caches with 64-token pages and a shuffled
                    block table; shapes as prefill_8k; k=2048.
  decode_b64_128k   as decode_b64 with every context 131072 tokens long.
  decode_rl_sweep   256 sequences, contexts n = 1024 i (i = 1..32); per-sequence budget
                    k = min(n, max(256, floor(rho n))), rho ~ U(0.05, 0.25) per sequence.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import numpy as np
import torch

BASE_SEED = 20261202


@dataclass(frozen=True)
class Shapes:
    H_I: int = 64
    d_I: int = 128
    H: int = 16
    H_kv: int = 1
    d_qk: int = 576
    d_v: int = 512
    latent: bool = True          # value = first d_v columns of the key row
    dtype: str = "bf16"
    idx_std: float = 1.0         # std of q_idx and k_idx
    w_dist: str = "normal"       # "normal": N(0, 1/H_I); "uniform": U(0, 1)
    page_size: int = 64


TINY = Shapes(H_I=4, d_I=32, H=4, H_kv=4, d_qk=64, d_v=64, latent=False, dtype="f32",
              idx_std=1.0 / math.sqrt(32), w_dist="uniform")
LATENT = Shapes()


@dataclass(frozen=True)
class Workload:
    name: str
    shapes: Shapes
    kind: str                    # "prefill" or "decode"
    L: int = 0                   # prefill length
    topk: int = 2048
    salient_frac: float = 0.0
    B: int = 0                   # decode batch
    ctx_range: tuple = (0, 0)    # decode: uniform integer context lengths in [lo, hi]
    rl_sweep: bool = False
    seed_offset: int = 0


WORKLOADS = {
    "tiny_prefill": Workload("tiny_prefill", TINY, "prefill", L=256, topk=32, seed_offset=0),
    "prefill_8k": Workload("prefill_8k", LATENT, "prefill", L=8192, topk=2048, seed_offset=1),
    "decode_b64": Workload("decode_b64", LATENT, "decode", B=64, ctx_range=(16384, 65536),
                           topk=2048, seed_offset=2),
    "prefill_128k": Workload("prefill_128k", LATENT, "prefill", L=131072, topk=2048,
                             salient_frac=0.01, seed_offset=3),
    "decode_rl_sweep": Workload("decode_rl_sweep", LATENT, "decode", B=256, ctx_range=(1024, 32768),
                                topk=8192, rl_sweep=True, seed_offset=4),
    "decode_b64_128k": Workload("decode_b64_128k", LATENT, "decode", B=64,
                                ctx_range=(131072, 131072), topk=2048, seed_offset=5),
}


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _normal(shape, std, g, device, dtype):
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def torch_dtype(s: Shapes):
    return torch.bfloat16 if s.dtype == "bf16" else torch.float32


def _weights(s: Shapes, n, g, device):
    if s.w_dist == "uniform":
        return torch.rand((n, s.H_I), generator=g, device=device, dtype=torch.float32)
    return _normal((n, s.H_I), 1.0 / math.sqrt(s.H_I), g, device, torch.float32)


def prefill_inputs(wl: Workload, device="cuda", seed: int | None = None, L: int | None = None):
    """q [L,H,d_qk], k [L,H_kv,d_qk], v [L,H_kv,d_v] or None, q_idx [L,H_I,d_I], w [L,H_I] fp32,
    k_idx [L,d_I]; plus 'salient' (positions scaled by 4) when the workload has them."""
    s = wl.shapes
    L = wl.L if L is None else L
    seed = BASE_SEED + wl.seed_offset if seed is None else seed
    g = _gen(seed, device)
    dt = torch_dtype(s)
    out = {}
    out["q_idx"] = _normal((L, s.H_I, s.d_I), s.idx_std, g, device, dt)
    out["k_idx"] = _normal((L, s.d_I), s.idx_std, g, device, dt)
    out["w"] = _weights(s, L, g, device)
    out["q"] = _normal((L, s.H, s.d_qk), 1.0, g, device, dt)
    out["k"] = _normal((L, s.H_kv, s.d_qk), 1.0, g, device, dt)
    out["v"] = None if s.latent else _normal((L, s.H_kv, s.d_v), 1.0, g, device, dt)
    if wl.salient_frac > 0:
        n_sal = int(math.floor(wl.salient_frac * L))
        rng = np.random.default_rng(seed + 1)
        pos = np.sort(rng.choice(L, size=n_sal, replace=False))
        p = torch.from_numpy(pos).to(device)
        out["k_idx"][p] *= 4  # exact in bf16 (power of two)
        out["k"][p] *= 4
        out["salient"] = pos
    return out


def decode_contexts(wl: Workload, seed: int | None = None):
    """Per-sequence context lengths (and budgets) of a decode workload."""
    seed = BASE_SEED + wl.seed_offset if seed is None else seed
    rng = np.random.default_rng(seed + 7)
    lo, hi = wl.ctx_range
    if wl.rl_sweep:
        ctx = np.full(wl.B, hi, dtype=np.int64)
        rho = rng.uniform(0.05, 0.25, size=wl.B)
        return ctx, rho
    ctx = rng.integers(lo, hi + 1, size=wl.B, dtype=np.int64)
    return ctx, None


def rl_budget(n: int, rho: np.ndarray) -> np.ndarray:
    """k_b = min(n, max(256, floor(rho_b n))) -- the decode_rl_sweep workload's budget rule."""
    return np.minimum(n, np.maximum(256, np.floor(rho * n).astype(np.int64)))


def decode_inputs(wl: Workload, device="cuda", seed: int | None = None, ctx=None, B: int | None = None):
    """Paged caches sized for the given (or drawn) context lengths.

    Returns q [B,H,d_qk], q_idx [B,H_I,d_I], w [B,H_I] fp32, kv_pages [P,page,H_kv,d_qk],
    v_pages (None for the latent layout), kidx_pages [P,page,d_I], block_table [B,max_blocks]
    int32 (-1 unused), ctx_len [B] int32, topk [B] int32, max_ctx, and rho for the sweep."""
    s = wl.shapes
    seed = BASE_SEED + wl.seed_offset if seed is None else seed
    ctx_np, rho = decode_contexts(wl, seed)
    if ctx is not None:
        ctx_np = np.asarray(ctx, dtype=np.int64)
    if B is not None:
        ctx_np = ctx_np[:B]
        rho = None if rho is None else rho[:B]
    B = len(ctx_np)
    P = s.page_size
    blocks = (ctx_np + P - 1) // P
    n_pages = int(blocks.sum())
    max_ctx = int(ctx_np.max())
    max_blocks = int((max_ctx + P - 1) // P)
    rng = np.random.default_rng(seed + 11)
    perm = rng.permutation(n_pages).astype(np.int32)
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    used = 0
    for b in range(B):
        table[b, :blocks[b]] = perm[used:used + blocks[b]]
        used += blocks[b]
    g = _gen(seed, device)
    dt = torch_dtype(s)
    out = {}
    out["q_idx"] = _normal((B, s.H_I, s.d_I), s.idx_std, g, device, dt)
    out["w"] = _weights(s, B, g, device)
    out["q"] = _normal((B, s.H, s.d_qk), 1.0, g, device, dt)
    out["kidx_pages"] = _normal((n_pages, P, s.d_I), s.idx_std, g, device, dt)
    out["kv_pages"] = _normal((n_pages, P, s.H_kv, s.d_qk), 1.0, g, device, dt)
    out["v_pages"] = None if s.latent else _normal((n_pages, P, s.H_kv, s.d_v), 1.0, g, device, dt)
    out["block_table"] = torch.from_numpy(table).to(device)
    out["ctx_len"] = torch.from_numpy(ctx_np.astype(np.int32)).to(device)
    if rho is not None:
        k = rl_budget(int(ctx_np.max()), rho)
        out["rho"] = rho
    else:
        k = np.full(B, wl.topk, dtype=np.int64)
    out["topk"] = torch.from_numpy(k.astype(np.int32)).to(device)
    out["max_ctx"] = max_ctx
    out["ctx_np"] = ctx_np
    return out


def paged_rows_inputs(wl: Workload, ctx, row_seq, row_pos, device="cuda", seed: int | None = None):
    """Paged caches of len(ctx) sequences (as decode_inputs) and T = len(row_seq) query rows drawn
    like the workload's queries: row t is the token at position row_pos[t] of sequence row_seq[t].
    Adds q [T,H,d_qk], q_idx [T,H_I,d_I], w [T,H_I] (replacing the decode rows), row_seq and
    row_pos [T] int32 on the device and as numpy (rs_np, rp_np)."""
    s = wl.shapes
    seed = BASE_SEED + wl.seed_offset if seed is None else seed
    d = decode_inputs(wl, device, seed=seed, ctx=ctx)
    rs = np.asarray(row_seq, dtype=np.int64)
    rp = np.asarray(row_pos, dtype=np.int64)
    T = len(rs)
    g = _gen(seed + 101, device)
    dt = torch_dtype(s)
    d["q_idx"] = _normal((T, s.H_I, s.d_I), s.idx_std, g, device, dt)
    d["w"] = _weights(s, T, g, device)
    d["q"] = _normal((T, s.H, s.d_qk), 1.0, g, device, dt)
    d["row_seq"] = torch.from_numpy(rs.astype(np.int32)).to(device)
    d["row_pos"] = torch.from_numpy(rp.astype(np.int32)).to(device)
    d["rs_np"], d["rp_np"] = rs, rp
    return d


def acceptance_inputs(T: int, V: int, device="cuda", seed: int | None = None):
    """Dense and sparse next-token logits for T tokens over a vocabulary of V (fp32, [T, V]):
    dense z ~ N(0, 4) per entry; sparse z + d_t e with e ~ N(0, 1) per entry and one perturbation
    scale per token d_t = 1.5 u_t^4, u_t ~ U(0, 1), so that most tokens stay nearly aligned and a
    few diverge (a long tail of low acceptance rates).  Also positions pos [T] int32 = 0..T-1."""
    seed = BASE_SEED + 50 if seed is None else seed
    g = _gen(seed, device)
    dense = torch.randn((T, V), generator=g, device=device, dtype=torch.float32) * 2.0
    u = torch.rand((T, 1), generator=g, device=device, dtype=torch.float32)
    sparse = dense + torch.randn((T, V), generator=g, device=device, dtype=torch.float32) * (1.5 * u ** 4)
    pos = torch.arange(T, dtype=torch.int32, device=device)
    return {"logits_p": dense, "logits_q": sparse, "pos": pos}


def library_config(wl: Workload, max_topk: int | None = None):
    """The library configuration matching a workload's shapes."""
    from indexer_selected_sparse_scores_amd import Config
    s = wl.shapes
    return Config(n_idx_heads=s.H_I, d_idx=s.d_I, n_heads=s.H, n_kv_heads=s.H_kv, d_qk=s.d_qk,
                  d_v=s.d_v, v_from_k=s.latent, page_size=s.page_size,
                  max_topk=max_topk or wl.topk, dtype=s.dtype)


def small(wl: Workload, **kw) -> Workload:
    return replace(wl, **kw)
