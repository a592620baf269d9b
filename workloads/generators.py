"""Seeded generators for verify-step and shortlisted-head inputs.

Every tensor is a pure function of an integer key.  The key is turned into a
64-bit seed by numpy's SeedSequence and drives a torch.Generator on the device
the caller asks for (CPU or GPU).  The same key on different devices gives
different, equally valid streams: callers that compare two implementations
generate once and hand the same bytes to both.

Distributions follow the workloads that the speculative-decoding pages discuss
(vocabularies of 32k-262k tokens; draft distributions that are noisy copies of
the target; a Zipf-like prior over token ids).  Nothing here evaluates the
verify rule itself.  Draft tokens are drawn with the Gumbel-max trick
(argmax of logits/T plus Gumbel noise), which samples softmax(logits/T) exactly
without forming the softmax.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

__all__ = [
    "TAG_TARGET", "TAG_DRAFT_NOISE", "TAG_DRAFT_TOKENS", "TAG_UNIFORMS",
    "TAG_SCORES", "TAG_HIDDEN", "TAG_HEAD_W",
    "WORKLOAD_IDS", "seed_of", "VerifyCase", "HeadCase",
    "normal_logits", "round_to", "noisy_copy", "gumbel_max_tokens",
    "argmax_tokens", "verify_uniforms", "verify_case", "workload_case",
    "head_case", "top_clusters", "bf16_bits", "f32_from_bf16_bits",
    "TAG_KV", "KvCase", "kv_case", "KV_WORKLOAD", "SparseDraftCase", "sparse_draft_case",
]

TAG_TARGET, TAG_DRAFT_NOISE, TAG_DRAFT_TOKENS, TAG_UNIFORMS = 0, 1, 2, 3
TAG_SCORES, TAG_HIDDEN, TAG_HEAD_W = 4, 5, 6
TAG_KV = 7

# Numeric namespaces for the seed keys of the named workloads.
WORKLOAD_IDS = {
    "b1_k4_v32000_f32": 1,
    "b8_k5_v128256_bf16": 2,
    "b64_k4_v151936_bf16": 3,
    "b256_k7_v262144_bf16": 4,
    "shortlist_head_b32_k4_d4096_v128256": 5,
    "kv_commit_b256_k7_p64_e1024_bf16": 6,
}


def seed_of(*key: int) -> int:
    """63-bit seed from an integer tuple via numpy SeedSequence."""
    ss = np.random.SeedSequence([int(k) for k in key])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & np.uint64((1 << 63) - 1))


def _gen(device, key) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(seed_of(*key))
    return g


def normal_logits(shape, std: float, zipf_s: float, key, device="cpu") -> torch.Tensor:
    """float32 logits ~ N(0, std^2), plus an optional log-prior -s*ln(id+1) over the last axis."""
    g = _gen(device, key)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    x.mul_(std)
    if zipf_s:
        V = shape[-1]
        prior = torch.arange(1, V + 1, device=device, dtype=torch.float64).log_().mul_(-zipf_s)
        x.add_(prior.to(torch.float32))
    return x


def round_to(x: torch.Tensor, dtype: str) -> torch.Tensor:
    """Cast float32 values to the storage dtype ('bf16' rounds to nearest even)."""
    if dtype == "bf16":
        return x.to(torch.bfloat16)
    if dtype == "f32":
        return x.to(torch.float32)
    raise ValueError(dtype)


def noisy_copy(base: torch.Tensor, sigma: float, key, dtype: str) -> torch.Tensor:
    """base (any float dtype) + N(0, sigma^2) noise, stored as dtype."""
    g = _gen(base.device, key)
    noise = torch.randn(base.shape, generator=g, device=base.device, dtype=torch.float32)
    noise.mul_(sigma).add_(base.to(torch.float32))
    return round_to(noise, dtype)


def gumbel_max_tokens(logits: torch.Tensor, temperature: float, key, chunk_rows: int = 64) -> torch.Tensor:
    """One token per row of logits[..., V], drawn from softmax(logits/T) by Gumbel-max.

    Works in float64.  Rows whose logits are all -inf get token 0.  Returns int32.
    """
    assert temperature > 0
    V = logits.shape[-1]
    flat = logits.reshape(-1, V)
    g = _gen(logits.device, key)
    out = torch.empty(flat.shape[0], dtype=torch.int64, device=logits.device)
    two53 = float(2 ** 53)
    for r0 in range(0, flat.shape[0], chunk_rows):
        r1 = min(r0 + chunk_rows, flat.shape[0])
        k = torch.randint(0, 2 ** 53, (r1 - r0, V), generator=g, device=logits.device, dtype=torch.int64)
        u = (k.to(torch.float64) + 0.5) / two53          # (0, 1), never 0 or 1
        gum = -torch.log(-torch.log(u))
        score = flat[r0:r1].to(torch.float64) / temperature + gum
        out[r0:r1] = torch.argmax(score, dim=-1)
    return out.reshape(logits.shape[:-1]).to(torch.int32)


def argmax_tokens(logits: torch.Tensor) -> torch.Tensor:
    """Greedy draft tokens: argmax of each row (torch picks the first maximum)."""
    return torch.argmax(logits.to(torch.float32), dim=-1).to(torch.int32)


def verify_uniforms(B: int, K: int, key, device="cpu") -> torch.Tensor:
    """float32 [B, K+1, 2] on the 24-bit grid k/2^24, k in [0, 2^24): [...,0] accept, [...,1] sample."""
    g = _gen(device, key)
    k = torch.randint(0, 1 << 24, (B, K + 1, 2), generator=g, device=device, dtype=torch.int64)
    return (k.to(torch.float32) * (1.0 / (1 << 24))).contiguous()


@dataclasses.dataclass
class VerifyCase:
    target: torch.Tensor        # [B, K+1, V] bf16 or float32
    draft: torch.Tensor         # [B, K, V]
    draft_tokens: torch.Tensor  # int32 [B, K]
    uniforms: torch.Tensor      # float32 [B, K+1, 2]
    temperature: float          # the float32 value both sides use
    dtype: str                  # 'bf16' | 'f32'

    @property
    def B(self):
        return self.target.shape[0]

    @property
    def K(self):
        return self.target.shape[1] - 1

    @property
    def V(self):
        return self.target.shape[2]


def verify_case(B: int, K: int, V: int, dtype: str, *, target_std: float, zipf_s: float,
                sigma: float, temperature: float, key=(0,), device="cpu",
                greedy_drafts: bool = False) -> VerifyCase:
    """Target ~ N(0, std^2) (+ Zipf log-prior), draft = target + N(0, sigma^2),
    draft tokens sampled from softmax(draft/T) (argmax when greedy_drafts)."""
    key = tuple(key)
    tgt32 = normal_logits((B, K + 1, V), target_std, zipf_s, key + (TAG_TARGET,), device)
    target = round_to(tgt32, dtype)
    del tgt32
    draft = noisy_copy(target[:, :K], sigma, key + (TAG_DRAFT_NOISE,), dtype)
    if greedy_drafts:
        tokens = argmax_tokens(draft)
    else:
        tokens = gumbel_max_tokens(draft, float(np.float32(temperature)) if temperature > 0 else 1.0,
                                   key + (TAG_DRAFT_TOKENS,))
    uni = verify_uniforms(B, K, key + (TAG_UNIFORMS,), device)
    return VerifyCase(target.contiguous(), draft.contiguous(), tokens.contiguous(), uni,
                      float(np.float32(temperature)), dtype)


def workload_case(name: str, *, sweep: int = 0, trial: int = 0, device="cpu",
                  greedy: bool = False) -> VerifyCase:
    """The named verify workloads (shapes and distributions of the speculative-decoding pages).

    b1_k4_v32000_f32     : target N(0,2^2), draft sigma 0.5, T=1
    b8_k5_v128256_bf16   : target N(0,3^2)+Zipf(1.1), sigma in (0.2, 1.0)[sweep], T=0.8
                           (greedy=True: argmax drafts, temperature 0)
    b64_k4_v151936_bf16  : target N(0,2^2), sigma in (0.1, 0.5, 1.0, 2.0)[sweep], T=1
    b256_k7_v262144_bf16 : target N(0,3^2)+Zipf(1.1), sigma 0.7, T=1
                           (greedy=True: argmax drafts)
    """
    wid = WORKLOAD_IDS[name]
    key = (0, wid, sweep)
    if name == "b1_k4_v32000_f32":
        return verify_case(1, 4, 32000, "f32", target_std=2.0, zipf_s=0.0, sigma=0.5,
                           temperature=1.0, key=key + (trial,), device=device)
    if name == "b8_k5_v128256_bf16":
        sig = (0.2, 1.0)[sweep]
        return verify_case(8, 5, 128256, "bf16", target_std=3.0, zipf_s=1.1, sigma=sig,
                           temperature=0.0 if greedy else 0.8, key=key + (trial,), device=device,
                           greedy_drafts=greedy)
    if name == "b64_k4_v151936_bf16":
        sig = (0.1, 0.5, 1.0, 2.0)[sweep]
        return verify_case(64, 4, 151936, "bf16", target_std=2.0, zipf_s=0.0, sigma=sig,
                           temperature=1.0, key=key + (trial,), device=device)
    if name == "b256_k7_v262144_bf16":
        return verify_case(256, 7, 262144, "bf16", target_std=3.0, zipf_s=1.1, sigma=0.7,
                           temperature=1.0, key=key + (trial,), device=device, greedy_drafts=greedy)
    raise KeyError(name)


def top_clusters(scores: torch.Tensor, n_sel: int) -> torch.Tensor:
    """Per row: the n_sel highest-scoring cluster ids (ties to the lower id), ascending. int32."""
    # a stable sort of -score puts larger scores first and keeps equal scores in id order
    idx = torch.argsort(-scores.to(torch.float64), dim=-1, stable=True)
    sel = idx[..., :n_sel]
    return torch.sort(sel, dim=-1).values.to(torch.int32).contiguous()


@dataclasses.dataclass
class HeadCase:
    h: torch.Tensor            # bf16 [B, K, d]
    W: torch.Tensor            # bf16 [V, d]
    cluster_ids: torch.Tensor  # int32 [B, n_sel], ascending
    cluster_size: int


def head_case(B=32, K=4, d=4096, V=128256, n_clusters=256, n_sel=16, *, trial=0, device="cpu",
              w_std=0.02) -> HeadCase:
    """Shortlisted drafter head inputs: h ~ N(0,1), W ~ N(0, w_std^2) (both bf16),
    V split into n_clusters contiguous clusters, per-context scores ~ N(0,1), top n_sel clusters."""
    assert V % n_clusters == 0
    wid = WORKLOAD_IDS["shortlist_head_b32_k4_d4096_v128256"]
    key = (0, wid, 0)
    h = normal_logits((B, K, d), 1.0, 0.0, key + (TAG_HIDDEN, trial), device).to(torch.bfloat16)
    W = torch.empty((V, d), dtype=torch.bfloat16, device=device)
    rows = max(1, (1 << 26) // d)
    g = _gen(device, key + (TAG_HEAD_W, trial))
    for r0 in range(0, V, rows):
        r1 = min(V, r0 + rows)
        W[r0:r1] = (torch.randn((r1 - r0, d), generator=g, device=device, dtype=torch.float32)
                    * w_std).to(torch.bfloat16)
    scores = normal_logits((B, n_clusters), 1.0, 0.0, key + (TAG_SCORES, trial), device)
    cids = top_clusters(scores, n_sel)
    return HeadCase(h.contiguous(), W, cids, V // n_clusters)


def bf16_bits(x: torch.Tensor) -> np.ndarray:
    """Raw uint16 bit patterns of a bf16 tensor (copied to host)."""
    assert x.dtype == torch.bfloat16
    return x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def f32_from_bf16_bits(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)




# KV layout of a Llama-3-8B-like target: 32 layers x {key, value} planes,
# 8 KV heads x 128 dims per token and plane, bf16; 128 cache positions.
KV_WORKLOAD = dict(name="kv_commit_b256_k7_p64_e1024_bf16", P=64, B=256, K=7, Lmax=128, E=1024)


@dataclasses.dataclass
class KvCase:
    cache: torch.Tensor      # [P, B, Lmax, E]
    staging: torch.Tensor    # [P, B, K, E]
    cache_len: torch.Tensor  # int32 [B]


def kv_case(P, B, K, Lmax, E, dtype=torch.bfloat16, *, trial=0, device="cpu") -> KvCase:
    """Synthetic KV cache and staging buffer: entries ~ N(0,1) in dtype; each
    sequence's current length uniform on [0, Lmax - K] (room for any commit)."""
    key = (0, 6, 0, TAG_KV, trial)
    g = _gen(device, key)
    cache = torch.empty((P, B, Lmax, E), dtype=dtype, device=device)
    staging = torch.empty((P, B, K, E), dtype=dtype, device=device)
    for p in range(P):
        cache[p] = torch.randn((B, Lmax, E), generator=g, device=device, dtype=torch.float32).to(dtype)
        staging[p] = torch.randn((B, K, E), generator=g, device=device, dtype=torch.float32).to(dtype)
    ln = torch.randint(0, max(1, Lmax - K + 1), (B,), generator=g, device=device, dtype=torch.int64)
    return KvCase(cache, staging, ln.to(torch.int32))


@dataclasses.dataclass
class SparseDraftCase:
    target: torch.Tensor        # [B, K+1, V]
    compact: torch.Tensor       # [B, K, L] draft logits on each position's shortlist, ascending id
    cluster_ids: torch.Tensor   # int32 [B, K, S], first n_sel[i] ascending, the rest -1
    n_sel: list                 # K ints
    cluster_size: int
    dense_draft: torch.Tensor   # [B, K, V]: the same logits at their ids, -inf elsewhere
    draft_tokens: torch.Tensor  # int32 [B, K]
    uniforms: torch.Tensor      # float32 [B, K+1, 2]
    temperature: float
    dtype: str

    @property
    def B(self):
        return self.target.shape[0]

    @property
    def K(self):
        return self.target.shape[1] - 1

    @property
    def V(self):
        return self.target.shape[2]


def sparse_draft_case(B: int, K: int, V: int, cluster_size: int, n_sel, dtype: str = "bf16", *,
                      sigma: float = 0.7, temperature: float = 1.0, key=(8,), device="cpu",
                      target_std: float = 3.0, zipf_s: float = 1.1) -> SparseDraftCase:
    """Per-position shortlists of a context: position i keeps its top n_sel[i]
    clusters (contiguous id ranges of cluster_size) by a N(0,1) score; its draft
    logits there are the target's plus N(0, sigma^2) noise.  Draft tokens are
    sampled from the draft softmax (Gumbel-max on the dense -inf-filled form)."""
    assert V % cluster_size == 0 and len(n_sel) == K
    nc = V // cluster_size
    S = max(n_sel) if K > 0 else 1
    L = S * cluster_size
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    target = normal_logits((B, K + 1, V), target_std, zipf_s, key + (TAG_TARGET,), device)
    noise = normal_logits((B, K, V), sigma, 0.0, key + (TAG_DRAFT_NOISE,), device)
    scores = normal_logits((B, K, nc), 1.0, 0.0, key + (TAG_SCORES,), device)
    cids = torch.full((B, K, S), -1, dtype=torch.int32, device=device)
    compact = torch.zeros((B, K, L), dtype=torch.float32, device=device)
    dense = torch.full((B, K, V), float("-inf"), dtype=torch.float32, device=device)
    full_draft = round_to(target[:, :K] + noise, dtype).float()
    for i in range(K):
        top = torch.topk(scores[:, i], n_sel[i], dim=-1).indices
        top = torch.sort(top, dim=-1).values.to(torch.int32)
        cids[:, i, :n_sel[i]] = top
        ids = (top.long()[:, :, None] * cluster_size + torch.arange(cluster_size, device=device)).reshape(B, -1)
        vals = torch.gather(full_draft[:, i], 1, ids)
        compact[:, i, :ids.shape[1]] = vals
        dense[:, i].scatter_(1, ids, vals)
    target = round_to(target, dtype)
    compact = compact.to(tdt)
    dense = dense.to(tdt)
    tok = gumbel_max_tokens(dense, temperature, key + (TAG_DRAFT_TOKENS,)) if K > 0 else \
        torch.zeros((B, 0), dtype=torch.int32, device=device)
    uni = verify_uniforms(B, K, key + (TAG_UNIFORMS,), device)
    return SparseDraftCase(target, compact, cids, list(n_sel), cluster_size, dense, tok, uni,
                           float(temperature), dtype)
