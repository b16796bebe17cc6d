"""Seeded synthetic inputs for the speculative-decoding verify step.

This module only draws random inputs. It holds none of the verify method's
arithmetic (no softmax, no acceptance test, no residual sampling), and both the
HIP path's tests and the fp64 oracle consume what it produces.

Five workloads are defined, each a shape plus a recipe for the logits:

* ``b1_k4_v1000_f32``    B=1,   k=4, V=1000,   fp32, T=1.0, sampling.
  Target logits iid N(0, 2^2); draft = target + N(0, 0.5^2).
* ``b8_k5_v32000_f32``   B=8,   k=5, V=32000,  fp32, T=0.7, sampling.
  Target N(0, 3^2) plus +8 at one random index per row; draft = 0.8*target + N(0, 1).
* ``b64_k5_v151936_bf16`` B=64, k=5, V=151936, bf16, T=1.0, sampling.
  Target N(0, 2.5^2) plus +6 at 5 distinct random indices per row; draft =
  target + N(0, 1); exactly round(0.2*B*k) draft rows (chosen without
  replacement) are replaced by fresh N(0, 2.5^2) rows to force rejections.
* ``b256_k3_v128256_bf16_greedy`` B=256, k=3, V=128256, bf16, greedy.
  Target N(0, 2^2) plus a margin spike +U(0, 4) added to the row's argmax;
  draft tokens = target argmax, with exactly round(0.3*B*k) positions (chosen
  without replacement) replaced by a uniformly random id. No draft logits and
  no uniforms are used in greedy mode.
* ``b512_k8_v262144_bf16`` B=512, k=8, V=262144, bf16, T=0.8, sampling.
  Target N(0, 2^2) plus +5 at 10 distinct random indices; draft = target + N(0, 0.7^2).

Common rules: logits are drawn in float32 and, for bf16 workloads, rounded to
bfloat16 (round to nearest even). Target rows i = 0..k (row k is the bonus
row); draft rows i = 0..k-1. In sampling mode each draft token is drawn from
softmax(draft_row / T) of the *stored* (rounded) draft row, by the Gumbel-max
construction (argmax of d/T plus Gumbel noise), which is an exact sampler for
that categorical distribution. Uniforms are float32 in [0, 1).

Ragged drafts (``draft_lengths``): per-row draft counts for any workload,
kb = the number of successes before the first failure of independent trials
that continue with probability 0.8, capped at k (a drafter that stops when its
own confidence drops, with a per-step continuation rate near the acceptance
rates the pages quote), from a generator seeded from (workload, seed,
"draft_len"). The logits, tokens and uniforms are those of ``make``.

Confidence-gate rows (``make_gate``): n ready distributions of V logits, iid
N(0, 2^2), then one token t per row set to the row maximum plus U(0, 20) (the
70B-class model in the pre-positioning paper shows decision-point gaps from
below 2 to about 20), with t drawn from the admissible set A with probability
0.9 and uniformly otherwise; A is 64 distinct token ids drawn once per
(n, V, seed). Rounded to bfloat16 for bf16 rows. ``admit_bits`` packs a token
list into the V-bit mask the gate reads (bit j & 31 of word j >> 5).

Every batch row b is drawn from its own generator seeded from (workload, seed,
b), so any subset of rows can be regenerated alone; the global choices (which
draft rows are replaced, which greedy positions are replaced) come from one
extra generator seeded from (workload, seed).
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional

import torch

SAMPLE = 0
GREEDY = 1


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    k: int
    V: int
    dtype: str          # "f32" or "bf16"
    T: float            # temperature (ignored in greedy mode)
    mode: int           # SAMPLE or GREEDY
    recipe: str         # human-readable recipe

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def logit_bytes(self) -> int:
        """Bytes of logits the verify step must read once (target + draft)."""
        rows = self.B * (self.k + 1)
        if self.mode == SAMPLE:
            rows += self.B * self.k
        return rows * self.V * self.elem_bytes

    def with_batch(self, B: int) -> "Workload":
        return dataclasses.replace(self, B=B)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("b1_k4_v1000_f32", 1, 4, 1000, "f32", 1.0, SAMPLE,
                 "target N(0,2^2); draft = target + N(0,0.5^2)"),
        Workload("b8_k5_v32000_f32", 8, 5, 32000, "f32", 0.7, SAMPLE,
                 "target N(0,3^2) + 8 at one index; draft = 0.8*target + N(0,1)"),
        Workload("b64_k5_v151936_bf16", 64, 5, 151936, "bf16", 1.0, SAMPLE,
                 "target N(0,2.5^2) + 6 at 5 indices; draft = target + N(0,1); "
                 "20% of draft rows replaced by N(0,2.5^2)"),
        Workload("b256_k3_v128256_bf16_greedy", 256, 3, 128256, "bf16", 1.0, GREEDY,
                 "target N(0,2^2) + U(0,4) on the argmax; tokens = argmax, 30% random"),
        Workload("b512_k8_v262144_bf16", 512, 8, 262144, "bf16", 0.8, SAMPLE,
                 "target N(0,2^2) + 5 at 10 indices; draft = target + N(0,0.7^2)"),
    ]
}

# The workload the throughput figure is quoted on.
HEADLINE = "b64_k5_v151936_bf16"


def _seed(*parts) -> int:
    h = hashlib.sha256("/".join(str(p) for p in parts).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device, *parts) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(*parts))
    return g


def _normal(shape, std, g, device):
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std


def _boost(rows, count, amount, g, device):
    """Add `amount` at `count` distinct random indices of every row (in place)."""
    n, V = rows.shape
    for r in range(n):
        idx = torch.randperm(V, generator=g, device=device)[:count]
        rows[r, idx] += amount
    return rows


def _gumbel_tokens(draft_rows, T, g, device):
    """One draw per row from softmax(draft_rows / T), via Gumbel-max."""
    u = torch.rand(draft_rows.shape, generator=g, device=device, dtype=torch.float64)
    u = u.clamp_min(1e-300)
    gumbel = -torch.log(-torch.log(u))
    return torch.argmax(draft_rows.double() / T + gumbel, dim=1).to(torch.int32)


def _global_choice(w: Workload, seed: int, device):
    """Workload-wide choices drawn before any row: replaced draft rows / positions."""
    g = _gen(device, w.name, seed, "global")
    n = w.B * w.k
    if w.name.startswith("b64_k5"):
        nrep = int(round(0.2 * n))
        return torch.randperm(n, generator=g, device=device)[:nrep].cpu()
    if w.mode == GREEDY:
        nrep = int(round(0.3 * n))
        pos = torch.randperm(n, generator=g, device=device)[:nrep].cpu()
        ids = torch.randint(0, w.V, (nrep,), generator=g, device=device).cpu()
        return pos, ids
    return None


def _rows_for_batch(w: Workload, seed: int, b: int, glob, device):
    """Float32 target [k+1,V], float32 draft [k,V] (or None), tokens [k], uniforms [k+1,2]."""
    g = _gen(device, w.name, seed, b)
    k, V = w.k, w.V
    n = k + 1
    if w.name == "b1_k4_v1000_f32":
        tgt = _normal((n, V), 2.0, g, device)
        dft = tgt[:k] + _normal((k, V), 0.5, g, device)
    elif w.name == "b8_k5_v32000_f32":
        tgt = _boost(_normal((n, V), 3.0, g, device), 1, 8.0, g, device)
        dft = 0.8 * tgt[:k] + _normal((k, V), 1.0, g, device)
    elif w.name == "b64_k5_v151936_bf16":
        tgt = _boost(_normal((n, V), 2.5, g, device), 5, 6.0, g, device)
        dft = tgt[:k] + _normal((k, V), 1.0, g, device)
        fresh = _normal((k, V), 2.5, g, device)
        for i in range(k):
            if (b * k + i) in glob:
                dft[i] = fresh[i]
    elif w.name == "b256_k3_v128256_bf16_greedy":
        tgt = _normal((n, V), 2.0, g, device)
        spike = torch.rand((n,), generator=g, device=device, dtype=torch.float32) * 4.0
        am = torch.argmax(tgt, dim=1)
        tgt[torch.arange(n, device=device), am] += spike
        dft = None
    elif w.name == "b512_k8_v262144_bf16":
        tgt = _boost(_normal((n, V), 2.0, g, device), 10, 5.0, g, device)
        dft = tgt[:k] + _normal((k, V), 0.7, g, device)
    else:
        raise KeyError(w.name)

    tgt = tgt.to(w.torch_dtype)
    if dft is not None:
        dft = dft.to(w.torch_dtype)

    if w.mode == GREEDY:
        tok = torch.argmax(tgt[:k].float(), dim=1).to(torch.int32)  # first max on ties
        pos, ids = glob
        for j in range(pos.numel()):
            p = int(pos[j])
            if p // k == b:
                tok[p % k] = int(ids[j])
        uni = None
    else:
        tok = _gumbel_tokens(dft.float(), w.T, g, device) if k > 0 else \
            torch.zeros((0,), dtype=torch.int32, device=device)
        uni = torch.rand((n, 2), generator=g, device=device, dtype=torch.float32)
    return tgt, dft, tok, uni


def make(w: Workload | str, seed: int = 0, device="cpu", rows: Optional[range] = None):
    """Generate the inputs of workload `w` for `seed`.

    Returns a dict with ``target`` [B,k+1,V], ``draft`` [B,k,V] (None in greedy
    mode), ``tokens`` [B,k] int32, ``uniforms`` [B,k+1,2] float32 (None in
    greedy mode), plus ``T`` and ``mode``. With ``rows`` only those batch rows
    are generated (identical to the same rows of the full draw).
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    device = torch.device(device)
    glob = _global_choice(w, seed, device)
    if isinstance(glob, torch.Tensor):
        glob = set(int(x) for x in glob)
    rows = range(w.B) if rows is None else rows
    nb = len(rows)
    target = torch.empty((nb, w.k + 1, w.V), dtype=w.torch_dtype, device=device)
    draft = None if w.mode == GREEDY else \
        torch.empty((nb, w.k, w.V), dtype=w.torch_dtype, device=device)
    tokens = torch.empty((nb, w.k), dtype=torch.int32, device=device)
    uniforms = None if w.mode == GREEDY else \
        torch.empty((nb, w.k + 1, 2), dtype=torch.float32, device=device)
    for j, b in enumerate(rows):
        t, d, tok, u = _rows_for_batch(w, seed, b, glob, device)
        target[j] = t
        if draft is not None:
            draft[j] = d
            uniforms[j] = u
        tokens[j] = tok
    return {"target": target, "draft": draft, "tokens": tokens, "uniforms": uniforms,
            "T": w.T, "mode": w.mode, "workload": w}


RAGGED_CONTINUE = 0.8


def draft_lengths(w: Workload | str, seed: int = 0, device="cpu", p: float = RAGGED_CONTINUE):
    """Per-row draft lengths int32 [B] in [0, k]: successes before the first
    failure of trials that continue with probability p, capped at k."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    g = _gen("cpu", w.name, seed, "draft_len")
    trials = torch.rand((w.B, max(w.k, 1)), generator=g, dtype=torch.float64) < p
    run = torch.cumprod(trials.to(torch.int64), dim=1).sum(dim=1)
    return run.clamp(max=w.k).to(torch.int32).to(device)


GATE_V = 128256            # a 70B-class model's vocabulary
GATE_A = 64                # admissible single-token answers


def make_gate(n: int, V: int = GATE_V, seed: int = 0, dtype: str = "bf16", device="cpu"):
    """Ready distributions logits [n, V] and the admissible token ids (int64 [GATE_A])."""
    g = _gen("cpu", "gate", n, V, seed)
    A = torch.randperm(V, generator=g)[:min(GATE_A, V)]
    x = torch.randn((n, V), generator=g, dtype=torch.float32) * 2.0
    inA = torch.rand(n, generator=g) < 0.9
    pick_a = A[torch.randint(0, A.numel(), (n,), generator=g)]
    pick_u = torch.randint(0, V, (n,), generator=g)
    t = torch.where(inA, pick_a, pick_u)
    s = torch.rand(n, generator=g) * 20.0
    x[torch.arange(n), t] = x.max(dim=1).values + s
    td = torch.float32 if dtype == "f32" else torch.bfloat16
    return x.to(td).to(device), A


def admit_bits(tokens, V: int) -> torch.Tensor:
    """int32 [(V + 31) // 32] mask with bit (j & 31) of word j >> 5 set for each token j."""
    words = [0] * ((V + 31) // 32)
    for j in (int(t) for t in tokens):
        words[j >> 5] |= 1 << (j & 31)
    return torch.tensor([w - (1 << 32) if w >= (1 << 31) else w for w in words], dtype=torch.int32)


LMHEAD_D = 4096            # hidden size of the 8B-class models with these vocabularies


def make_lmhead(B: int, k: int, V: int, d: int = LMHEAD_D, seed: int = 0, device="cpu"):
    """An int8 LM head and the k + 1 hidden states of B batch rows.

    weight [V, d] int8 ~ round(N(0, 30^2)) clipped to [-127, 127]; hidden row m
    (= b*(k+1) + i) leans towards a planted vocabulary row: round(N(0, 30^2) +
    beta * weight[planted]) clipped, beta ~ U(0.055, 0.094), which lifts the
    planted logit by about 3.5 to 6 standard deviations of the others (at
    d = 4096), so it is
    the argmax of most rows but not all. Scales: hidden U(0.5, 1.5) / 2^7,
    weight U(0.9, 1.1) / 2^7 (float32). Draft tokens are the planted rows of
    positions 0..k-1 with 30% replaced by uniform random ids.
    """
    g = _gen(device, "lmhead", B, k, V, d, seed)
    M = B * (k + 1)
    w = torch.randn((V, d), generator=g, device=device).mul_(30.0).round_().clamp_(-127, 127)
    planted = torch.randint(0, V, (M,), generator=g, device=device)
    beta = torch.rand((M, 1), generator=g, device=device) * 0.039 + 0.055
    h = torch.randn((M, d), generator=g, device=device).mul_(30.0)
    h.add_(beta * w[planted]).round_().clamp_(-127, 127)
    hs = (torch.rand(M, generator=g, device=device) + 0.5) / 128.0
    ws = (torch.rand(V, generator=g, device=device) * 0.2 + 0.9) / 128.0
    tok = planted.view(B, k + 1)[:, :k].clone()
    swap = torch.rand((B, k), generator=g, device=device) < 0.3
    rnd = torch.randint(0, V, (B, k), generator=g, device=device)
    tok = torch.where(swap, rnd, tok).to(torch.int32)
    return {"hidden": h.to(torch.int8), "hidden_scale": hs.float(), "weight": w.to(torch.int8),
            "weight_scale": ws.float(), "tokens": tok, "B": B, "k": k, "V": V, "d": d}


def make_lmhead_sample(B: int, k: int, V: int, d: int = LMHEAD_D, seed: int = 0, device="cpu",
                       draft_head: bool = False):
    """make_lmhead's target head and rows, plus a draft's hidden rows and uniforms.

    Draft hidden row b*k + i is the target's row b*(k+1) + i mixed with fresh
    noise: round(0.8 * h_t + N(0, 18^2)) clipped, so the draft leans to the
    same planted row, less sharply. With draft_head, the draft has a head of
    its own: the target's weights plus round(N(0, 12^2)), clipped, with its own
    scales. Draft tokens are the planted rows with 30% replaced by uniform
    random ids (as make_lmhead); uniforms [B, k+1, 2] ~ U[0, 1) float32.
    """
    x = make_lmhead(B, k, V, d, seed=seed, device=device)
    g = _gen(device, "lmhead_sample", B, k, V, d, seed)
    ht = x["hidden"].view(B, k + 1, d)[:, :k].reshape(B * k, d).float()
    hd = (ht * 0.8 + torch.randn((B * k, d), generator=g, device=device) * 18.0).round_().clamp_(-127, 127)
    x["draft_hidden"] = hd.to(torch.int8)
    x["draft_hidden_scale"] = x["hidden_scale"].view(B, k + 1)[:, :k].reshape(B * k).clone() * 1.25
    if draft_head:
        wd = x["weight"].float() + torch.randn((V, d), generator=g, device=device) * 12.0
        x["draft_weight"] = wd.round_().clamp_(-127, 127).to(torch.int8)
        x["draft_weight_scale"] = (torch.rand(V, generator=g, device=device) * 0.2 + 0.9) / 128.0
    else:
        x["draft_weight"] = None
        x["draft_weight_scale"] = None
    x["uniforms"] = torch.rand((B, k + 1, 2), generator=g, device=device, dtype=torch.float32)
    return x
