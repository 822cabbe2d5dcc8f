"""The denoising round, the per-block loop, the commit pass and prefill.

  * Round input (self-conditioning): the previous round's distribution is fed
    back through an adapter on the tied embedding, so each round starts from
    the model's last guess ([ORL-blog] "What shipped"; [ORL-brief] item 2;
    [ORL-zicq] "Technical Mechanism Analysis").  Reading: an open row's input
    is m + W_sc (p.E) with m a mask embedding vector and W_sc a bias-free d x d
    adapter; in the first round of a block there is no previous distribution
    and the input is m; a committed row's input is its token's embedding.
  * Round: forward the block, head statistics, commit ([ORL-blog] "What
    shipped": each round gives a distribution over the unresolved tokens, and
    the block is committed after enough rounds).
  * Loop: rounds repeat until no position is open or max_rounds is reached;
    the continue decision is taken after every round ([ORL-blog] "What
    shipped", on the engine's whole-block loop).
  * Commit pass (reading; the pages do not say how a finished block's K/V is
    produced): one more forward of the clean committed tokens writes the
    block's K/V into the prefix cache, so later blocks attend to the committed
    text, not to a round's partly-masked inputs.  Prompt prefill is the same
    pass over each block of the prompt (block-causal attention).
Pinned by tests/test_oracle_loop.py.
"""
from __future__ import annotations

import dataclasses

import numpy as np

from .numerics import Prec
from .block import forward_block, rmsnorm, attention, rope, swiglu
from .head import head_rowstats
from .commit import CommitRule, commit, FLAG_NONFINITE


class OracleModel:
    """Weights of one model as oracle floats, converted lazily from storage.

    source: a mapping name -> stored array (synth.Weights or a dict), plus the
    shape.  Layer weights are converted on each access unless cache_layers is
    set, so a 36-layer bf16 model never sits in float64 all at once.
    """

    def __init__(self, shape, source, prec: Prec, cache_layers: bool = True, overrides=None):
        self.shape = shape
        self.src = source
        self.prec = prec
        self._cache = {} if cache_layers else None
        self.overrides = dict(overrides or {})

    def get(self, name):
        if name in self.overrides:
            return np.asarray(self.overrides[name], dtype=self.prec.compute)
        if self._cache is not None and name in self._cache:
            return self._cache[name]
        v = self.prec.w(self.src[name])
        if self._cache is not None:
            self._cache[name] = v
        return v

    def emb_stored(self):
        if "emb" in self.overrides:
            return self.overrides["emb"]
        return self.src["emb"]

    def emb_rows(self, ids):
        return self.prec.w(np.asarray(self.emb_stored())[np.asarray(ids)])

    def layer(self, i):
        names = ["attn_norm", "wq", "wk", "wv", "wo", "ffn_norm"]
        if not self.shape.moe:
            names += ["wg", "wu", "wd"]
        else:
            names += ["router"]
        return {n: self.get(f"l{i}.{n}") for n in names}


@dataclasses.dataclass
class KVCache:
    k: list
    v: list
    length: int = 0

    @classmethod
    def empty(cls, shape, cap, dtype=np.float64):
        z = lambda: np.zeros((shape.hkv, cap, shape.head_dim), dtype)  # noqa: E731
        return cls([z() for _ in range(shape.n_layers)], [z() for _ in range(shape.n_layers)], 0)

    def copy(self):
        return KVCache([a.copy() for a in self.k], [a.copy() for a in self.v], self.length)


def selfcond(model: OracleModel, tokens, committed, pe_prev, prec: Prec):
    """Round input x [B, d]: E[tok] for committed rows, m + W_sc (p.E) for open rows."""
    B = len(committed)
    d = model.shape.d
    m = model.get("mask_emb")
    x = np.empty((B, d), prec.compute)
    open_rows = [i for i in range(B) if not committed[i]]
    done_rows = [i for i in range(B) if committed[i]]
    if done_rows:
        x[done_rows] = model.emb_rows(np.asarray(tokens)[done_rows])
    if open_rows:
        if pe_prev is None:
            x[open_rows] = m
        else:
            pe = prec.act(np.asarray(pe_prev)[open_rows])
            x[open_rows] = m + pe @ model.get("w_sc").T
    return x


def final_hidden(model: OracleModel, h, prec: Prec):
    return prec.act(rmsnorm(h, model.get("final_norm"), model.shape.eps))


@dataclasses.dataclass
class RoundResult:
    x: np.ndarray
    hn: np.ndarray
    stats: dict
    committed_now: list
    flags: int


def denoise_round(model: OracleModel, kv: KVCache, tokens, committed, pe_prev, round_idx: int,
                  rule: CommitRule, prec: Prec, want_logits: bool = False) -> RoundResult:
    """One round: self-cond input, forward with block K/V written at [L, L+B),
    head statistics of the open rows, commit.  tokens/committed change in place."""
    L = kv.length
    x = selfcond(model, tokens, committed, pe_prev, prec)
    h = forward_block(model, x, kv, L, prec)
    hn = final_hidden(model, h, prec)
    st = head_rowstats(hn, model.emb_stored(), committed, prec, want_logits=want_logits)
    mp_open = st["maxprob"]
    flags = 0
    open_rows = [i for i in range(len(committed)) if not committed[i]]
    if any(not (np.isfinite(st["lse"][i]) and np.isfinite(st["entropy"][i])) for i in open_rows):
        flags |= FLAG_NONFINITE
    now, f2 = commit(rule, mp_open, st["argmax"], committed, tokens, round_idx)
    return RoundResult(x, hn, st, now, flags | f2)


@dataclasses.dataclass
class BlockResult:
    tokens: np.ndarray
    rounds: int
    n_new: list
    flags: int
    trace: list  # per round: (open rows at start, RoundResult)


def commit_pass(model: OracleModel, kv: KVCache, tokens, prec: Prec):
    """Forward the clean tokens of the block at [L, L+B), write their K/V, L += B."""
    L = kv.length
    x = model.emb_rows(tokens)
    forward_block(model, x, kv, L, prec, skip_last_ffn=True)
    kv.length = L + len(tokens)


def decode_block(model: OracleModel, kv: KVCache, rule: CommitRule, prec: Prec,
                 keep_trace: bool = False, want_logits: bool = False) -> BlockResult:
    """Decode one block of B fully-masked positions after the cached prefix."""
    B = model.shape.block
    tokens = np.zeros(B, np.int32)
    committed = np.zeros(B, np.uint8)
    pe_prev = None
    n_new = []
    flags = 0
    trace = []
    r = 0
    while r < rule.max_rounds and not committed.all():
        open_before = committed.copy()
        res = denoise_round(model, kv, tokens, committed, pe_prev, r, rule, prec, want_logits)
        n_new.append(len(res.committed_now))
        flags |= res.flags
        pe_prev = res.stats["pe"]
        if keep_trace:
            trace.append((open_before, res))
        r += 1
    commit_pass(model, kv, tokens, prec)
    return BlockResult(tokens.copy(), r, n_new, flags, trace)


def prefill(model: OracleModel, kv: KVCache, ids, prec: Prec):
    """Commit passes over consecutive blocks of the prompt (len % B == 0)."""
    B = model.shape.block
    ids = np.asarray(ids, dtype=np.int32)
    assert len(ids) % B == 0
    for a in range(0, len(ids), B):
        commit_pass(model, kv, ids[a:a + B], prec)


def generate(model: OracleModel, prompt, n_blocks: int, rule: CommitRule, prec: Prec,
             cap=None, keep_trace: bool = False):
    """Prefill the prompt, then decode n_blocks blocks.  Returns (tokens, blocks, kv)."""
    B = model.shape.block
    cap = cap or (len(prompt) + B * (n_blocks + 1))
    kv = KVCache.empty(model.shape, cap, prec.compute)
    prefill(model, kv, prompt, prec)
    out = []
    blocks = []
    for _ in range(n_blocks):
        br = decode_block(model, kv, rule, prec, keep_trace=keep_trace)
        out.append(br.tokens)
        blocks.append(br)
    return np.concatenate(out) if out else np.zeros(0, np.int32), blocks, kv


def blockcausal_reference(model: OracleModel, ids, prec: Prec):
    """K/V of every layer for a whole token sequence computed in one pass with a
    block-causal mask (position i sees j iff j // B <= i // B), without a cache.
    Used to pin the cached commit-pass/prefill path.  Dense models only.
    Returns (k, v) lists of [Hkv, N, D]."""
    s = model.shape
    B = s.block
    ids = np.asarray(ids)
    N = len(ids)
    pos = np.arange(N)
    blk = pos // B
    allowed = blk[None, :] <= blk[:, None]                     # [N(query), N(key)]
    x = model.emb_rows(ids)
    ks, vs = [], []
    for li in range(s.n_layers):
        lw = model.layer(li)
        a = prec.act(rmsnorm(x, lw["attn_norm"], s.eps))
        q = prec.act(rope((a @ lw["wq"].T).reshape(N, s.hq, s.head_dim), pos, s.rope_base))
        k = prec.act(rope((a @ lw["wk"].T).reshape(N, s.hkv, s.head_dim), pos, s.rope_base))
        v = prec.act((a @ lw["wv"].T).reshape(N, s.hkv, s.head_dim))
        ks.append(k.transpose(1, 0, 2).copy())
        vs.append(v.transpose(1, 0, 2).copy())
        o = np.empty((N, s.hq, s.head_dim), prec.compute)
        group = s.hq // s.hkv
        for h in range(s.hq):
            g = h // group
            sc = (q[:, h, :] @ k[:, g, :].T) / np.sqrt(s.head_dim)
            sc = np.where(allowed, sc, -np.inf)
            sc = sc - sc.max(axis=1, keepdims=True)
            p = np.exp(sc)
            p = p / p.sum(axis=1, keepdims=True)
            o[:, h, :] = p @ v[:, g, :]
        hres = x + prec.act(o.reshape(N, -1)) @ lw["wo"].T
        f = prec.act(rmsnorm(hres, lw["ffn_norm"], s.eps))
        x = hres + prec.act(swiglu(f @ lw["wg"].T, f @ lw["wu"].T)) @ lw["wd"].T
    return ks, vs
