"""Continuous-batching replay through the library (join/leave pin).

Follows the request flow of the TGI architecture page's call-flow diagrams:
a first request is prefilled and decoded; a second joins with its own
prefill and both decode; the first finishes and its blocks are freed; a
third joins and is cleared at once; the second decodes to its stop length.
The library's host block manager (pka_bm_*, a LIFO free list) hands freed
blocks out again immediately and produces every slot mapping and block
table, and freed blocks are NaN-poisoned, so a stale block-table entry or a read past a
sequence's end shows up as a wrong or non-finite output.  Every step is
checked against the fp64 oracle over each request's contiguous history.
The second variant prefills the second prompt in chunks that run in the same
mixed step as the first request's decodes (prefill chunking: TGI router
deep-dive, the prefill-chunking paragraph of the scheduling-loop section).
"""
import numpy as np
import pytest
import torch

import paged_kv_attention_append_amd as pka
from oracle import attention as A
from paged_kv_attention_append_amd import workloads as W

from gpu_harness import compare, say

pytestmark = pytest.mark.gpu

HQ, HKV, D = 8, 2, 128
NUM_BLOCKS = 24
BF = torch.bfloat16


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


class Request:
    def __init__(self, rid, prompt, max_len, rng):
        self.rid, self.prompt, self.max_len = rid, prompt, max_len
        self.k = W.round_to_dtype(rng.standard_normal((max_len, HKV, D), dtype=np.float32), W.BF16)
        self.v = W.round_to_dtype(rng.standard_normal((max_len, HKV, D), dtype=np.float32), W.BF16)
        self.q = W.round_to_dtype(rng.standard_normal((max_len, HQ, D), dtype=np.float32), W.BF16)
        self.len = 0  # tokens in the cache


class Server:
    """Host side of one attention layer: the library's block manager (request
    id = sequence id) + library calls."""

    def __init__(self):
        self.cache = pka.KVCache.allocate(NUM_BLOCKS, HKV, D, BF, fill=float("nan"))
        self.bm = pka.BlockManager(NUM_BLOCKS, 4, NUM_BLOCKS)

    def slots_for(self, req, start, stop):
        assert self.bm.seq_len(req.rid) == start
        return self.bm.append([req.rid], [stop - start])

    def release(self, req):
        kp = self.cache.k_pool.view(NUM_BLOCKS, HKV, 16, D)
        vp = self.cache.v_pool.view(NUM_BLOCKS, HKV, 16, D)
        for b in self.bm.release(req.rid):
            kp[int(b)].fill_(float("nan"))
            vp[int(b)].fill_(float("nan"))

    def append(self, req, start, stop):
        slots = self.slots_for(req, start, stop)
        pka.kv_append(self.cache, torch.from_numpy(req.k[start:stop]).to(BF).cuda(),
                      torch.from_numpy(req.v[start:stop]).to(BF).cuda(), torch.from_numpy(slots).cuda())
        req.len = stop

    def tables(self, reqs):
        bt, lens = self.bm.tables([r.rid for r in reqs])
        assert list(lens) == [r.len for r in reqs]
        return torch.from_numpy(bt).cuda()

    def prefill(self, req):
        say(f"prefill r{req.rid} ({req.prompt} tokens)")
        self.append(req, 0, req.prompt)
        cu = np.array([0, req.prompt], np.int32)
        out = pka.attn_prefill_varlen(torch.from_numpy(req.q[:req.prompt]).to(BF).cuda(),
                                      torch.from_numpy(req.k[:req.prompt]).to(BF).cuda(),
                                      torch.from_numpy(req.v[:req.prompt]).to(BF).cuda(),
                                      torch.from_numpy(cu).cuda(), torch.from_numpy(cu))
        ref = A.attention_seq(req.q[:req.prompt], req.k[:req.prompt], req.v[:req.prompt])
        compare(out, ref, W.BF16, f"replay prefill r{req.rid}")

    def decode(self, reqs):
        say("decode " + ",".join(f"r{r.rid}@{r.len}" for r in reqs))
        for r in reqs:
            self.append(r, r.len, r.len + 1)
        q = torch.from_numpy(np.stack([r.q[r.len - 1] for r in reqs])).to(BF).cuda()
        kvl = np.array([r.len for r in reqs], np.int32)
        out = pka.attn_decode_paged(q, self.cache, self.tables(reqs), torch.from_numpy(kvl).cuda(), int(kvl.max()))
        ref = np.stack([A.attention_seq(r.q[r.len - 1:r.len], r.k[:r.len], r.v[:r.len])[0] for r in reqs])
        compare(out, ref, W.BF16, "replay decode")

    def mixed(self, decodes, chunk_req, chunk):
        """Decodes of `decodes` plus the next `chunk` prompt tokens of chunk_req."""
        start = chunk_req.len
        stop = min(chunk_req.prompt, start + chunk)
        say(f"mixed: decode {[r.rid for r in decodes]} + r{chunk_req.rid} rows {start}..{stop}")
        for r in decodes:
            self.append(r, r.len, r.len + 1)
        self.append(chunk_req, start, stop)
        reqs = list(decodes) + [chunk_req]
        qs = [r.q[r.len - 1:r.len] for r in decodes] + [chunk_req.q[start:stop]]
        ql = np.array([len(x) for x in qs], np.int32)
        cu = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
        kvl = np.array([r.len for r in reqs], np.int32)
        out = pka.attn_mixed_step(torch.from_numpy(np.concatenate(qs)).to(BF).cuda(), self.cache,
                                  torch.from_numpy(cu).cuda(), torch.from_numpy(cu), torch.from_numpy(kvl).cuda(),
                                  torch.from_numpy(kvl), self.tables(reqs))
        ref = np.concatenate([A.attention_seq(qq, r.k[:r.len], r.v[:r.len]) for qq, r in zip(qs, reqs)])
        compare(out, ref, W.BF16, "replay mixed")


def _script(chunked: bool):
    rng = np.random.default_rng(77)
    r1 = Request(1, 37, 44, rng)
    r2 = Request(2, 70, 96, rng)
    r3 = Request(3, 20, 21, rng)
    srv = Server()
    srv.prefill(r1)
    srv.decode([r1])
    srv.decode([r1])
    if chunked:
        while r2.len < r2.prompt:          # r2's prompt in chunks, alongside r1's decodes
            srv.mixed([r1], r2, 32)
    else:
        srv.prefill(r2)
    srv.decode([r1, r2])
    srv.release(r1)                         # r1 finished: free (and poison) its blocks
    srv.decode([r2])
    srv.prefill(r3)                         # takes r1's blocks (LIFO)
    srv.release(r3)                         # cleared at once
    while r2.len < r2.max_len:
        srv.decode([r2])
    assert r2.len == r2.max_len
    torch.cuda.synchronize()


def test_replay_join_leave():
    _script(chunked=False)


def test_replay_join_leave_with_prefill_chunking():
    _script(chunked=True)
