"""Seeded synthetic inputs for one QSA layer.

This module only draws random tensors and plants needles; it holds none of the
layer's arithmetic (no rotation, pooling, scoring, selection or attention).
Both the HIP path's tests/bench and the CPU oracle take their inputs from here.

Shapes follow the layer described on the pages (PyTorchKR post "Qwen3.8-Flash-Next,
1/9의 학습 비용으로 Qwen3.7-Plus(397B-A17B) 수준에 도달한 125B-A6B 모델", spec
table rows "Qwen Sparse Attention", "QSA 인덱서", "QSA 예산"): 24 query heads,
2 KV heads, head dim 256; indexer with 4 query heads and one shared key head of
dim 128; budget 512 blocks of 4 tokens.

Layout (token-major, bf16):
  q     [B][L][24][256]     k, v [B][L][2][256]
  q_idx [B][L][4][128]      k_idx [B][L][128]

Values are i.i.d. N(0,1) drawn in fp32 and rounded to bf16 (torch's RNE cast).
Random streams come from torch generators seeded by (workload seed, tensor id,
sequence); a CPU and a GPU generator give different streams, so one workload is
always generated on one device and copied where needed.

Needles: a needle block's 4 tokens get keys sqrt(d)*(c*u + s*xi) and each of its
probe queries gets sqrt(d)*(c*u + s*xi'), with c = 2/sqrt(5), s = 1/sqrt(5)
(cosine 0.8 in expectation), u a unit direction supported on the dims that the
rotary embedding leaves untouched (indexer dims 64..127, core dims 64..255) and
xi, xi' random unit vectors orthogonal to u.  Needle geometry is drawn with a
NumPy generator so it is identical on every device.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

N_Q_HEADS = 24
N_KV_HEADS = 2
HEAD_DIM = 256
ROPE_DIM = 64
N_IDX_HEADS = 4
IDX_DIM = 128
BLOCK = 4

# tensor ids used in seeds
T_Q, T_K, T_V, T_QIDX, T_KIDX, T_NEEDLE = 0, 1, 2, 3, 4, 5

_C = 2.0 / math.sqrt(5.0)   # needle component along the shared direction
_S = 1.0 / math.sqrt(5.0)   # random orthogonal component


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic QSA workload.

    mode 'prefill': `seq_len` tokens, every token is a query.
    mode 'decode' : `seq_len` cached tokens per sequence plus one new token at
                    position `seq_len` (the only query).
    """
    name: str
    mode: str
    batch: int
    seq_len: int
    budget: int
    n_needles: int
    needle_layout: str          # 'random' | 'even'
    seed: int
    yarn_factor: float = 1.0
    recency_blocks: int = 0     # final blocks whose k and k_idx are scaled
    recency_scale: float = 1.0
    chunk: Optional[int] = None  # prefill chunk length (chunked prefill)
    probes_per_needle: int = 8

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    # small prefill, budget 64 blocks, 8 needles at random depths
    "prefill_1k": Workload("qsa_prefill_L1024_K64", "prefill", 1, 1024, 64, 8, "random", 1),
    # prefill with the real budget, 64 evenly spaced needles
    "prefill_32k": Workload("qsa_prefill_L32768_K512", "prefill", 1, 32768, 512, 64, "even", 2),
    # decode, 64 sequences x 131072 cached tokens, 16 needles per sequence
    "decode_128k": Workload("qsa_decode_B64_ctx131072_K512", "decode", 64, 131072, 512, 16, "random", 3),
    # prefill at the native context, 256 needles, last 64 blocks' keys x1.5
    "prefill_256k": Workload("qsa_prefill_L262144_K512", "prefill", 1, 262144, 512, 256, "even", 4,
                             recency_blocks=64, recency_scale=1.5),
    # 1M context with YaRN x4: decode at batch 8 and a chunked prefill
    "decode_1m": Workload("qsa_decode_B8_ctx1048576_K512_yarn4", "decode", 8, 1048576, 512, 256, "random", 5,
                          yarn_factor=4.0),
    "prefill_1m": Workload("qsa_prefill_L1048576_K512_yarn4_chunk65536", "prefill", 1, 1048576, 512, 256,
                           "even", 5, yarn_factor=4.0, chunk=65536),
}


def _seed(*parts: int) -> int:
    ss = np.random.SeedSequence([int(p) for p in parts])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))


def _randn(shape, seed: int, device) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def _unit_on(rng: np.random.Generator, dim: int, lo: int) -> np.ndarray:
    u = np.zeros(dim)
    x = rng.standard_normal(dim - lo)
    u[lo:] = x / np.linalg.norm(x)
    return u


def _noise_orth(rng: np.random.Generator, u: np.ndarray, n: int) -> np.ndarray:
    x = rng.standard_normal((n, u.shape[0]))
    x -= np.outer(x @ u, u)
    x /= np.linalg.norm(x, axis=1, keepdims=True)
    return x


def _needle_vecs(rng, u, n, dim):
    return math.sqrt(dim) * (_C * u[None, :] + _S * _noise_orth(rng, u, n))


@dataclasses.dataclass
class NeedlePlan:
    """Needle geometry for one sequence."""
    blocks: np.ndarray           # int64 [n] needle block indices
    probes: list                 # list of int64 arrays: probe positions per needle
    u_idx: np.ndarray            # [n][128] indexer directions
    u_core: np.ndarray           # [n][2][256] core directions per KV head


def _plan_needles(w: Workload, seq: int, n_tokens: int, n_query_pos: Optional[int]) -> NeedlePlan:
    rng = np.random.default_rng(_seed(w.seed, T_NEEDLE, seq))
    nblk = n_tokens // BLOCK
    n = w.n_needles
    if n == 0 or nblk < 3:
        return NeedlePlan(np.zeros(0, np.int64), [], np.zeros((0, IDX_DIM)), np.zeros((0, 2, HEAD_DIM)))
    if w.needle_layout == "even":
        blocks = np.array([int((k + 0.5) * nblk / n) for k in range(n)], dtype=np.int64)
    else:
        hi = nblk - 2 if w.mode == "prefill" else nblk
        blocks = np.sort(rng.choice(hi, size=min(n, hi), replace=False)).astype(np.int64)
    n = len(blocks)
    if w.mode == "decode":
        # one shared direction per sequence; the new token is the probe
        ui = _unit_on(rng, IDX_DIM, ROPE_DIM)
        uc = np.stack([_unit_on(rng, HEAD_DIM, ROPE_DIM) for _ in range(N_KV_HEADS)])
        u_idx = np.repeat(ui[None], n, 0)
        u_core = np.repeat(uc[None], n, 0)
        probes = [np.array([n_tokens], np.int64)] * n
    else:
        u_idx = np.stack([_unit_on(rng, IDX_DIM, ROPE_DIM) for _ in range(n)])
        u_core = np.stack([np.stack([_unit_on(rng, HEAD_DIM, ROPE_DIM) for _ in range(N_KV_HEADS)])
                           for _ in range(n)])
        used = set()
        probes = []
        L = n_query_pos
        for b in blocks:
            first = BLOCK * (int(b) + 1)
            cand = rng.permutation(np.arange(first, L))
            pick = []
            for p in cand:
                if int(p) not in used:
                    pick.append(int(p))
                    used.add(int(p))
                    if len(pick) == w.probes_per_needle:
                        break
            probes.append(np.array(sorted(pick), np.int64))
    return NeedlePlan(blocks, probes, u_idx, u_core)


def _put(t: torch.Tensor, idx, vals: np.ndarray):
    t[idx] = torch.from_numpy(vals.astype(np.float32)).to(t.device)


def _gen_seq(w: Workload, seq: int, n_tok: int, q_pos: np.ndarray, device, plan: NeedlePlan):
    """fp32 tensors for one sequence: keys for n_tok tokens, queries at q_pos."""
    nq = len(q_pos)
    kk = _randn((n_tok, N_KV_HEADS, HEAD_DIM), _seed(w.seed, T_K, seq), device)
    vv = _randn((n_tok, N_KV_HEADS, HEAD_DIM), _seed(w.seed, T_V, seq), device)
    ki = _randn((n_tok, IDX_DIM), _seed(w.seed, T_KIDX, seq), device)
    qq = _randn((nq, N_Q_HEADS, HEAD_DIM), _seed(w.seed, T_Q, seq), device)
    qi = _randn((nq, N_IDX_HEADS, IDX_DIM), _seed(w.seed, T_QIDX, seq), device)
    if w.recency_blocks and w.recency_scale != 1.0:
        lo = max(0, (n_tok // BLOCK - w.recency_blocks) * BLOCK)
        kk[lo:] *= w.recency_scale
        ki[lo:] *= w.recency_scale
    rng = np.random.default_rng(_seed(w.seed, T_NEEDLE, seq, 1))
    qpos_index = {int(p): i for i, p in enumerate(q_pos)}
    for n, b in enumerate(plan.blocks):
        toks = np.arange(BLOCK * int(b), BLOCK * int(b) + BLOCK)
        _put(ki, torch.from_numpy(toks), _needle_vecs(rng, plan.u_idx[n], BLOCK, IDX_DIM))
        for g in range(N_KV_HEADS):
            kv = _needle_vecs(rng, plan.u_core[n, g], BLOCK, HEAD_DIM)
            kk[torch.from_numpy(toks), g] = torch.from_numpy(kv.astype(np.float32)).to(device)
        for p in plan.probes[n]:
            i = qpos_index.get(int(p))
            if i is None:
                continue
            qi[i] = torch.from_numpy(_needle_vecs(rng, plan.u_idx[n], N_IDX_HEADS, IDX_DIM)
                                     .astype(np.float32)).to(device)
            for g in range(N_KV_HEADS):
                hv = _needle_vecs(rng, plan.u_core[n, g], N_Q_HEADS // N_KV_HEADS, HEAD_DIM)
                qq[i, g * 12:(g + 1) * 12] = torch.from_numpy(hv.astype(np.float32)).to(device)
    return qq, kk, vv, qi, ki


_NAMES = ("q", "k", "v", "q_idx", "k_idx")


def _alloc(B, n_q, n_k, device):
    bf = torch.bfloat16
    return {
        "q": torch.empty((B, n_q, N_Q_HEADS, HEAD_DIM), dtype=bf, device=device),
        "k": torch.empty((B, n_k, N_KV_HEADS, HEAD_DIM), dtype=bf, device=device),
        "v": torch.empty((B, n_k, N_KV_HEADS, HEAD_DIM), dtype=bf, device=device),
        "q_idx": torch.empty((B, n_q, N_IDX_HEADS, IDX_DIM), dtype=bf, device=device),
        "k_idx": torch.empty((B, n_k, IDX_DIM), dtype=bf, device=device),
    }


def prefill_inputs(w: Workload, device="cpu", seq_len: Optional[int] = None, batch: Optional[int] = None):
    """Inputs of a prefill workload: every token is a query.

    Returns a dict with bf16 tensors q, k, v, q_idx, k_idx and the needle plans.
    """
    L = w.seq_len if seq_len is None else seq_len
    B = w.batch if batch is None else batch
    res = _alloc(B, L, L, device)
    plans = []
    qpos = np.arange(L)
    for b in range(B):
        plan = _plan_needles(w, b, L, L)
        for name, t in zip(_NAMES, _gen_seq(w, b, L, qpos, device, plan)):
            res[name][b].copy_(t)
            del t
        plans.append(plan)
    res["needles"] = plans
    return res


def decode_inputs(w: Workload, device="cpu", ctx: Optional[int] = None, batch: Optional[int] = None):
    """Inputs of a decode workload.

    k, v, k_idx hold ctx+1 tokens per sequence: the cached context (positions
    0..ctx-1) and the new token (position ctx).  q, q_idx hold the new token only.
    """
    n_ctx = w.seq_len if ctx is None else ctx
    B = w.batch if batch is None else batch
    res = _alloc(B, 1, n_ctx + 1, device)
    plans = []
    qpos = np.array([n_ctx])
    for b in range(B):
        plan = _plan_needles(w, b, n_ctx, None)
        for name, t in zip(_NAMES, _gen_seq(w, b, n_ctx + 1, qpos, device, plan)):
            res[name][b].copy_(t)
            del t
        plans.append(plan)
    res["needles"] = plans
    return res


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Raw bf16 bit patterns of a tensor as a host uint16 array (no arithmetic)."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def score_rows(seed: int, B: int, L: int, q_offset: int, tie_mode: str = "mixed") -> np.ndarray:
    """Seeded fp32 score matrices [B][L][ceil((q_offset+L)/4)] for testing selection alone.

    Candidate entries (block < floor(p/4)) are >= +0; the rest hold -1.
    tie_mode: 'float'  -- continuous values (no ties);
              'coarse' -- multiples of 0.25 in [0, 8] (many exact ties);
              'zeros'  -- mostly +0 with a few positive values (ties at zero);
              'mixed'  -- rows cycle through the three.
    """
    rng = np.random.default_rng(_seed(seed, 7, B, L, q_offset))
    ncol = (q_offset + L + BLOCK - 1) // BLOCK
    out = np.full((B, L, ncol), -1.0, dtype=np.float32)
    modes = ["float", "coarse", "zeros"]
    for b in range(B):
        for i in range(L):
            o = (q_offset + i) // BLOCK
            if o == 0:
                continue
            mode = modes[(b * L + i) % 3] if tie_mode == "mixed" else tie_mode
            if mode == "float":
                v = np.abs(rng.standard_normal(o)).astype(np.float32) * 10
            elif mode == "coarse":
                v = rng.integers(0, 33, o).astype(np.float32) * 0.25
            else:
                v = np.where(rng.random(o) < 0.05, rng.random(o) * 5, 0.0).astype(np.float32)
            out[b, i, :o] = v
    return out


def gdn_inputs(seed: int, lens, hq: int = 16, hv: int = 48, device="cpu", init_state: bool = False):
    """Seeded inputs of a Gated DeltaNet chunked prefill over packed sequences.

    Head counts default to the GDN row of the pages' spec table (16 QK heads,
    48 V heads, dim 128).  q and k are uniform random unit vectors (normalised
    Gaussians, as the layer's L2 norm leaves them) rounded to bf16; v is N(0,1)
    in bf16; the log gate is g = -exp(N(-3, 1)) (alpha = exp(g) has median
    0.95 and spans fast- and slow-decaying heads); beta = 1/(1+exp(-N(0,1))).
    The optional initial state is N(0, 0.1^2) fp32.  Returns a dict with
    cu_seqlens (int32, [nseq+1]) and q, k [N][hq][128], v [N][hv][128],
    g, beta [N][hv], s0 [nseq][hv][128][128] or None, all on `device`.
    """
    lens = [int(x) for x in lens]
    n = int(sum(lens))
    gen = torch.Generator(device="cpu").manual_seed(_seed(seed, 11, len(lens), n))
    q = torch.randn(n, hq, 128, generator=gen)
    k = torch.randn(n, hq, 128, generator=gen)
    q = (q / q.norm(dim=-1, keepdim=True).clamp_min(1e-6)).to(torch.bfloat16)
    k = (k / k.norm(dim=-1, keepdim=True).clamp_min(1e-6)).to(torch.bfloat16)
    v = torch.randn(n, hv, 128, generator=gen).to(torch.bfloat16)
    g = -torch.exp(torch.randn(n, hv, generator=gen) - 3.0)
    beta = torch.sigmoid(torch.randn(n, hv, generator=gen))
    s0 = torch.randn(len(lens), hv, 128, 128, generator=gen) * 0.1 if init_state else None
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32))
    out = {"cu_seqlens": cu, "lens": lens, "q": q, "k": k, "v": v, "g": g.float(), "beta": beta.float(), "s0": s0}
    return {key: (val.to(device) if isinstance(val, torch.Tensor) else val) for key, val in out.items()}
