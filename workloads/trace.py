"""Seeded synthetic request traces for span-prefill scheduling.

Stand-in for the page's RAG serving runs (MiniPIC §4: a multi-hop QA set on
a Llama-3-8B-architecture model, neither present): every request lists a few
retrieved spans drawn from a shared pool, then its own final prompt, then a
number of output tokens; requests arrive over time.  Values are N(0, 1),
rounded to bf16; nothing here is model data and nothing here computes
attention.

Token data: every span token and every private (prompt or output) token of
a request has its own q [Hq][d], k~ [Hkv][d] and v [Hkv][d], drawn in the
order: spans' K, V, q (span by span), then requests' K, V, q (request by
request), from ``default_rng(data_seed)``.  Structure comes from
``default_rng(100 + data_seed)``: span lengths (whole 16-token blocks),
which spans each request lists and in which order, prompt and output
lengths, arrival steps.
"""

from __future__ import annotations

import dataclasses

import numpy as np

from .synth import _draw


@dataclasses.dataclass
class Trace:
    name: str
    hq: int
    hkv: int
    d: int
    base: float
    span_lens: list            # tokens per span (multiples of 16)
    requests: list             # (arrival_step, [span ids], prompt_len, output_len)
    q: np.ndarray              # [n_tokens][Hq][d] bf16 bits: every token's query
    k: np.ndarray              # [n_tokens][Hkv][d] unrotated keys
    v: np.ndarray              # [n_tokens][Hkv][d]
    span_base: np.ndarray      # first token index of each span
    req_base: np.ndarray       # first token index of each request's private tokens
    description: str = ""
    dtype: str = "bf16"

    def span_tokens(self, r: int) -> int:
        return int(sum(self.span_lens[s] for s in self.requests[r][1]))

    def composed_len(self, r: int) -> int:
        _, _, p, o = self.requests[r]
        return self.span_tokens(r) + p + o

    def span_token_index(self, s: int, i):
        return self.span_base[s] + np.asarray(i, np.int64)

    def request_token_index(self, r: int, c):
        """Global token index of composed slot(s) c of request r (spans first, then private)."""
        c = np.asarray(c, np.int64)
        out = np.empty(c.shape, np.int64)
        off = 0
        for s in self.requests[r][1]:
            m = (c >= off) & (c < off + self.span_lens[s])
            out[m] = self.span_base[s] + (c[m] - off)
            off += self.span_lens[s]
        m = c >= off
        out[m] = self.req_base[r] + (c[m] - off)
        return out

    @property
    def n_tokens(self) -> int:
        return int(self.k.shape[0])


def make_trace(name: str = "small", data_seed: int = 11, n_spans: int = 6, n_req: int = 8,
               span_blocks=(2, 5), spans_per_req=(1, 3), prompt=(2, 40), output=(0, 6),
               arrival_every: int = 2, arrivals_per_wave: int = 2, hq: int = 32, hkv: int = 8,
               d: int = 128, base: float = 500000.0, values: bool = True) -> Trace:
    """A trace; the ranges are inclusive (low, high).

    Requests arrive in waves of ``arrivals_per_wave`` every ``arrival_every``
    steps.  values=False draws no token data (zero views of the right shape),
    for host-only use.
    """
    srng = np.random.default_rng(100 + data_seed)
    span_lens = [16 * int(srng.integers(span_blocks[0], span_blocks[1] + 1))
                 for _ in range(n_spans)]
    reqs = []
    for r in range(n_req):
        k = int(srng.integers(spans_per_req[0], spans_per_req[1] + 1))
        sids = [int(x) for x in srng.choice(n_spans, size=k, replace=False)]
        p = int(srng.integers(max(prompt[0], 0 if k else 1), prompt[1] + 1))
        o = int(srng.integers(output[0], output[1] + 1))
        reqs.append(((r // arrivals_per_wave) * arrival_every, sids, p, o))
    span_base = np.zeros(n_spans, np.int64)
    span_base[1:] = np.cumsum(span_lens)[:-1]
    n_span_tok = int(sum(span_lens))
    priv = [p + o for _, _, p, o in reqs]
    req_base = n_span_tok + np.concatenate([[0], np.cumsum(priv)[:-1]]).astype(np.int64)
    n_tok = n_span_tok + int(sum(priv))
    if values:
        drng = np.random.default_rng(data_seed)
        ks, vs, qs = [], [], []
        for n in list(span_lens) + priv:
            ks.append(_draw(drng, (n, hkv, d), "bf16"))
            vs.append(_draw(drng, (n, hkv, d), "bf16"))
            qs.append(_draw(drng, (n, hq, d), "bf16"))
        k, v, q = np.concatenate(ks), np.concatenate(vs), np.concatenate(qs)
    else:
        z = np.zeros((), np.uint16)
        k = v = np.broadcast_to(z, (n_tok, hkv, d))
        q = np.broadcast_to(z, (n_tok, hq, d))
    desc = (f"{n_req} requests in waves of {arrivals_per_wave} every {arrival_every} steps, each "
            f"{spans_per_req[0]}-{spans_per_req[1]} of {n_spans} shared spans "
            f"({span_blocks[0] * 16}-{span_blocks[1] * 16} tokens) + a {prompt[0]}-{prompt[1]} "
            f"token final prompt + {output[0]}-{output[1]} output tokens; {hq}q/{hkv}kv heads, "
            f"d {d}, bf16")
    return Trace(name=name, hq=hq, hkv=hkv, d=d, base=base, span_lens=span_lens, requests=reqs,
                 q=q, k=k, v=v, span_base=span_base, req_base=req_base, description=desc)


# The benchmark trace: RAG-style requests, each listing 4 of 64 shared
# 1024-token spans (the chunked-prefill shape) + a 256-token final prompt +
# 32 output tokens, arriving 8 at a time every 8 steps while earlier
# requests decode.
RAG_TRACE = dict(name="rag", data_seed=21, n_spans=64, n_req=64, span_blocks=(64, 64),
                 spans_per_req=(4, 4), prompt=(256, 256), output=(32, 32), arrival_every=8,
                 arrivals_per_wave=8)
