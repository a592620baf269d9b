"""Comparison of GPU verify outputs with the fp64 oracle (decision-level tie accounting).

A sequence whose oracle result is n takes min(n + 1, K) accept decisions and
one sampled (or argmax) token: those are the decisions counted.  Outputs must
match the oracle exactly, except that a disagreement is *excused* when it sits
within 1e-6 of the oracle's decision boundary:

- an accept decision: |u - min(1, ratio)| < 1e-6 at the first position where
  the two accepted lengths differ;
- a sampled token: the oracle's sampled distribution puts less than 1e-6 of
  its mass (normalised by S) between u*S and the cumulative interval of the
  token the GPU picked (``probe_gap`` of the oracle, given the GPU's token).
  So the GPU's token must be the oracle's neighbour across a near-tie, not
  merely any token while the oracle's own pick is close to a boundary.

Once a sequence disagrees, its later decisions are not compared.  Any other
disagreement fails.  Excused disagreements are also totalled over the whole
test session (``SESSION``) and must stay below 1e-4 of the decisions taken.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

import oracle

TIE_BAND = 1e-6
PROB_RTOL = 1e-5
MAX_EXCUSED_RATE = 1e-4


@dataclasses.dataclass
class Report:
    decisions: int = 0
    excused: int = 0
    failures: list = dataclasses.field(default_factory=list)
    prob_max_rel: float = 0.0

    def merge(self, o: "Report"):
        self.decisions += o.decisions
        self.excused += o.excused
        self.failures += o.failures
        self.prob_max_rel = max(self.prob_max_rel, o.prob_max_rel)

    @property
    def excused_rate(self):
        return self.excused / max(1, self.decisions)

    def allowed_excused(self):
        """Per-call allowance: the session rate, but at least one near-tie per call."""
        return max(1, int(MAX_EXCUSED_RATE * self.decisions))


# every sampling comparison of the session adds to this
SESSION = Report()

# The probabilities are fp32 outputs: below the smallest normal fp32 (2^-126)
# they cannot carry PROB_RTOL relative precision (subnormals hold fewer bits,
# and values under 2^-149 are zero).  There both sides must be below 2^-126;
# above it the error is relative.
FLT_MIN = 2.0 ** -126


def prob_rel_error(gpu, orc) -> float:
    """Largest relative error of GPU probabilities against the oracle's, with
    values where both sides lie below FLT_MIN counted as equal (and a GPU
    value at or above FLT_MIN where the oracle's is below counted as 1)."""
    g = np.asarray(gpu, np.float64)
    o = np.asarray(orc, np.float64)
    tiny_o = np.abs(o) < FLT_MIN
    bad_tiny = tiny_o & (np.abs(g) >= FLT_MIN)
    rel = np.abs(g[~tiny_o] - o[~tiny_o]) / np.abs(o[~tiny_o])
    worst = float(np.max(rel)) if rel.size else 0.0
    return max(worst, 1.0 if bad_tiny.any() else 0.0)


def decisions_taken(orc_len, K):
    """Accept decisions up to and including the first rejection, plus the sample."""
    n = np.asarray(orc_len, np.int64)
    return int(np.where(n < 0, 0, np.minimum(n + 1, K) + 1).sum())


def probe_tokens(gpu_len, gpu_out):
    """The GPU's emitted token at its own position n (-1 for a faulty sequence)."""
    gl = np.asarray(gpu_len)
    go = np.asarray(gpu_out)
    pos = np.clip(gl, 0, go.shape[1] - 1)
    tok = go[np.arange(gl.shape[0]), pos]
    return np.where(gl >= 0, tok, -1).astype(np.int32)


def compare(gpu_len, gpu_out, orc, K, greedy=False, gpu_pt=None, gpu_pd=None, seq_ids=None) -> Report:
    """Compare GPU outputs with an oracle result.  In sample mode the oracle must
    have been run with probe_token=probe_tokens(gpu_len, gpu_out)."""
    gl = np.asarray(gpu_len)
    go = np.asarray(gpu_out)
    B = gl.shape[0]
    rep = Report(decisions=decisions_taken(orc["accepted_len"], K))
    ids = np.arange(B) if seq_ids is None else np.asarray(seq_ids)
    for b in range(B):
        nl, no = int(gl[b]), int(orc["accepted_len"][b])
        same = nl == no and np.array_equal(go[b], orc["out_tokens"][b])
        if same:
            continue
        if nl < 0 or no < 0:
            rep.failures.append((int(ids[b]), "faulty flag differs", nl, no))
            continue
        if greedy:
            rep.failures.append((int(ids[b]), "greedy mismatch", go[b].tolist(), orc["out_tokens"][b].tolist()))
            continue
        if nl != no:
            i = min(nl, no)
            margin = float(orc["accept_margin"][b, i])
            what = f"accept decision at {i}"
        else:
            ob = orc["out_tokens"][b]
            if not (np.array_equal(go[b, :no], ob[:no]) and np.array_equal(go[b, no + 1:], ob[no + 1:])):
                rep.failures.append((int(ids[b]), "tokens other than the sample differ", go[b].tolist(), ob.tolist()))
                continue
            if "probe_gap" not in orc:
                raise ValueError("sample disagreements need the oracle run with the GPU's tokens as probe_token")
            margin = float(orc["probe_gap"][b])
            what = f"sample at {no} (gpu token {int(go[b, no])}, oracle {int(ob[no])})"
        if margin < TIE_BAND:
            rep.excused += 1
        else:
            rep.failures.append((int(ids[b]), what, margin, go[b].tolist(), orc["out_tokens"][b].tolist()))
    if not greedy:
        SESSION.decisions += rep.decisions
        SESSION.excused += rep.excused
    if gpu_pt is not None:
        for gp, key in ((gpu_pt, "p_target"), (gpu_pd, "p_draft")):
            g = np.asarray(gp, np.float64)
            o = orc[key]
            ok = np.isfinite(o)
            if not np.array_equal(np.isfinite(g), ok):
                rep.failures.append(("probability NaN pattern differs", key))
                continue
            if ok.any():
                rep.prob_max_rel = max(rep.prob_max_rel, prob_rel_error(g[ok], o[ok]))
    return rep


def run_gpu(case, mode="sample", return_probs=True, **kw):
    import speculative_sampling_verification_vocab_amd as sv
    dev = torch.device("cuda", 0)
    tgt = case.target.to(dev)
    dr = case.draft.to(dev) if case.draft is not None else None
    tok = case.draft_tokens.to(dev)
    uni = case.uniforms.to(dev)
    res = sv.spec_verify(tgt, dr, tok, uni, case.temperature if mode != "greedy" else 0.0, mode,
                         return_probs=return_probs, **kw)
    torch.cuda.synchronize()
    return [r.cpu().numpy() for r in res]


def run_oracle(case, mode="sample", threads=None, gpu=None):
    """The oracle on a case; gpu = (accepted_len, out_tokens) of the GPU run
    supplies the probe tokens for the sample comparison."""
    threads = threads or oracle.default_threads()
    probe = probe_tokens(gpu[0], gpu[1]) if gpu is not None and mode != "greedy" else None
    return oracle.verify(case.target, case.draft, case.draft_tokens, case.uniforms,
                         case.temperature, mode=oracle.GREEDY if mode == "greedy" else oracle.SAMPLE,
                         threads=threads, probe_token=probe)


def check_case(case, mode="sample", max_excused_rate=None):
    """Run both sides on one case and return the report (asserting no failure)."""
    out = run_gpu(case, mode)
    orc = run_oracle(case, mode, gpu=out)
    if mode == "greedy":
        rep = compare(out[0], out[1], orc, case.K, greedy=True)
    else:
        rep = compare(out[0], out[1], orc, case.K, gpu_pt=out[2], gpu_pd=out[3])
    assert not rep.failures, rep.failures[:5]
    if mode == "sample":
        assert rep.prob_max_rel <= PROB_RTOL, rep.prob_max_rel
        assert rep.excused <= rep.allowed_excused(), (rep.excused, rep.decisions)
    if max_excused_rate is not None:
        assert rep.excused_rate <= max_excused_rate, (rep.excused, rep.decisions)
    return rep, out, orc
