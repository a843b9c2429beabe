"""Stream order of the fused layer.

The prepare phase may run its stream pass over K and V on a second stream
that the library keeps (fixed selector, causal window, separate Kn),
forked from the caller's stream and joined back to it with events. These
tests check that a call stays ordered on the caller's stream:
  * on a non-default stream, right after work on that stream that writes
    its inputs, with the output read on that stream right after;
  * replayed from a captured graph, with eager work between the replays.
The same kernels on the same inputs are deterministic, so every result must
equal the eager result on the default stream bit for bit. Parity of these
calls with the oracle is covered by the variant and attention tests.
"""
import pytest
import torch

import sparse_rank_attention_rola_amd as sd
from workloads import synthetic
from gpu_util import dev_bf16, dev_f32, say

pytestmark = pytest.mark.gpu

CFG = synthetic.AttnConfig("frames-780", 1, 2, 128, 6, 10, 13, 128, 64, 0.70, 32)
K_KEEP = 4
FRAME = CFG.Hg * CFG.Wg
# (selector, chunk tokens, window): the side-stream paths and the serial one
CASES = [("fixed", 0, 0), ("topk", 2 * FRAME, 2), ("topk", 0, 0)]


def _id(c):
    return f"{c[0]}-ct{c[1]}-w{c[2]}"


def _inputs():
    Qb, Kb, Vb = synthetic.gen_qkv(CFG, 0)
    Pqb, Pkb = synthetic.gen_lowrank_params(CFG)
    g = synthetic.gen_gate(CFG, amplified=True)
    lr = sd.LowrankParams(dev_bf16(Pqb), dev_bf16(Pkb))
    return dev_bf16(Qb), dev_bf16(Kb), dev_bf16(Vb), dev_f32(g), lr


class _Layer:
    def __init__(self, case):
        select, ct, window = case
        self.var = dict(select=select, chunk_tokens=ct, window=window)
        self.Q, self.K, self.V, self.g, self.lr = _inputs()
        self.grid = (CFG.T, CFG.Hg, CFG.Wg)
        nq = -(-CFG.L // CFG.block_q)
        self.idx_shape = (CFG.B, CFG.H, nq, K_KEEP)

    def buffers(self):
        ws = sd.rola_workspace(self.Q, self.lr, K_KEEP, grid=self.grid, block_q=CFG.block_q, **self.var)
        return ws, torch.empty_like(self.Q), torch.empty(self.idx_shape, dtype=torch.int32, device="cuda")

    def call(self, K, V, ws, out, idx):
        return sd.sd_rola_attention(self.Q, K, V, self.g, self.lr, K_KEEP, grid=self.grid, block_q=CFG.block_q,
                                    out=out, idx_out=idx, workspace=ws, **self.var)

    def eager(self):
        ws, out, idx = self.buffers()
        self.call(self.K, self.V, ws, out, idx)
        torch.cuda.synchronize()
        return out.clone(), idx.clone()


@pytest.mark.parametrize("case", CASES, ids=_id)
def test_call_on_a_caller_stream(case):
    say(f"caller stream {_id(case)}")
    lay = _Layer(case)
    ref_o, ref_i = lay.eager()
    ws, out, idx = lay.buffers()
    Kc, Vc = torch.empty_like(lay.K), torch.empty_like(lay.V)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    for rep in range(3):
        with torch.cuda.stream(s):
            # inputs written on the caller's stream just before the call
            Kc.zero_()
            Vc.zero_()
            Kc.copy_(lay.K)
            Vc.copy_(lay.V)
            lay.call(Kc, Vc, ws, out, idx)
            got_o, got_i = out.clone(), idx.clone()  # read on the caller's stream just after
            out.zero_()
        torch.cuda.synchronize()
        assert torch.equal(got_i, ref_i), f"block map, call {rep}"
        assert torch.equal(got_o, ref_o), f"output, call {rep}"


@pytest.mark.parametrize("case", CASES, ids=_id)
def test_graph_replays(case):
    say(f"graph replays {_id(case)}")
    lay = _Layer(case)
    ref_o, ref_i = lay.eager()
    ws, out, idx = lay.buffers()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        lay.call(lay.K, lay.V, ws, out, idx)
    for rep in range(3):
        out.zero_()  # eager work between the replays
        idx.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, ref_i), f"block map, replay {rep}"
        assert torch.equal(out, ref_o), f"output, replay {rep}"


def test_calls_from_two_host_threads():
    # the side stream is shared by the calls on a device; a mutex orders the
    # host side of their fork/join, each call stays ordered on its own stream
    import threading

    say("two host threads, fixed selector")
    lay = _Layer(CASES[0])
    ref_o, ref_i = lay.eager()
    results, errors = {}, []

    def worker(t):
        try:
            s = torch.cuda.Stream()
            ws, out, idx = lay.buffers()
            got = []
            with torch.cuda.stream(s):
                for _ in range(4):
                    lay.call(lay.K, lay.V, ws, out, idx)
                    got.append((out.clone(), idx.clone()))
            s.synchronize()
            results[t] = got
        except Exception as e:  # reported by the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors
    for t in range(2):
        for n, (o, i) in enumerate(results[t]):
            assert torch.equal(i, ref_i), f"thread {t} call {n}: block map"
            assert torch.equal(o, ref_o), f"thread {t} call {n}: output"
