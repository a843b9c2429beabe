"""The allocation-free fused layer against the fused layer with a workspace.

sd_rola_attention_noalloc runs the same kernels as sd_rola_attention, in
stream order on the caller's stream, on the library's static device
scratch instead of a caller workspace. The kernels are deterministic, so
its output and block map must equal those of sd_rola_attention on the same
inputs bit for bit (sd_rola_attention's own parity with the oracle is
covered by the attention, variant and full-size tests). Three calls run in
a row, the later ones on a smaller layer, so that each finds the previous
call's contents in the scratch. Shapes whose workspace exceeds the static
buffer are rejected before any device work.
"""
import pytest
import torch

import sparse_rank_attention_rola_amd as sd
from workloads import synthetic
from gpu_util import dev_bf16, dev_f32, say

pytestmark = pytest.mark.gpu

K720 = synthetic.WAN14B_720P
SMALL = synthetic.AttnConfig("frames-780", 1, 2, 128, 6, 10, 13, 128, 64, 0.70, 32)


def _device_inputs(cfg, seed):
    # the 14B 720P layer at full size: drawn on the device (seeded), since
    # both sides of the comparison run the library's kernels
    gen = torch.Generator(device="cuda").manual_seed(seed)
    shape = (cfg.B, cfg.L, cfg.H, cfg.d)
    Q, K, V = (torch.randn(shape, generator=gen, device="cuda").to(torch.bfloat16) for _ in range(3))
    Pqb, Pkb = synthetic.gen_lowrank_params(cfg, seed)
    g = synthetic.gen_gate(cfg, seed, amplified=True)
    return Q, K, V, dev_f32(g), sd.LowrankParams(dev_bf16(Pqb), dev_bf16(Pkb))


def _host_inputs(cfg, seed):
    Qb, Kb, Vb = synthetic.gen_qkv(cfg, seed)
    Pqb, Pkb = synthetic.gen_lowrank_params(cfg, seed)
    g = synthetic.gen_gate(cfg, seed, amplified=True)
    return dev_bf16(Qb), dev_bf16(Kb), dev_bf16(Vb), dev_f32(g), sd.LowrankParams(dev_bf16(Pqb), dev_bf16(Pkb))


def _both(cfg, inputs, k_keep, **var):
    Q, K, V, g, lr = inputs
    grid = (cfg.T, cfg.Hg, cfg.Wg)
    nq = -(-cfg.L // cfg.block_q)
    idx_ref = torch.empty((cfg.B, cfg.H, nq, k_keep), dtype=torch.int32, device="cuda")
    ref = sd.sd_rola_attention(Q, K, V, g, lr, k_keep, grid=grid, block_q=cfg.block_q, idx_out=idx_ref, **var)
    out = torch.full_like(Q, float("nan"))
    idx = torch.full_like(idx_ref, -7)
    sd.sd_rola_attention_noalloc(Q, K, V, g, lr, k_keep, out, grid=grid, block_q=cfg.block_q, idx_out=idx, **var)
    torch.cuda.synchronize()
    return ref, idx_ref, out, idx


def _same(ref, idx_ref, out, idx, name):
    n_out = int((out.view(torch.int16) != ref.view(torch.int16)).sum())
    n_idx = int((idx != idx_ref).sum())
    say(f"{name}: {n_out} output and {n_idx} block-map entries differ")
    assert n_out == 0 and n_idx == 0


def test_noalloc_equals_workspace_entry_two_calls():
    k720 = sd.sd_keep_count(K720.sparsity, -(-K720.L // 64))
    say(f"no-alloc call 1: {K720.name} B={K720.B} H={K720.H} L={K720.L} k={k720}")
    _same(*_both(K720, _device_inputs(K720, 3), k720), "720P layer")
    say(f"no-alloc call 2: {SMALL.name} H={SMALL.H} L={SMALL.L} k=4")
    _same(*_both(SMALL, _host_inputs(SMALL, 1), 4), "780-token layer")
    say("no-alloc call 3: 780-token layer, chunked selection with a causal window")
    frame = SMALL.Hg * SMALL.Wg
    _same(*_both(SMALL, _host_inputs(SMALL, 2), 4, chunk_tokens=2 * frame, window=2), "780-token chunked layer")


def test_noalloc_rejects_shapes_beyond_the_static_buffer():
    # 720P at 50% sparsity keeps 590 blocks per row: its workspace (about
    # 158 MiB) exceeds the 128 MiB buffer
    cfg = K720
    Q = torch.empty((1, cfg.L, cfg.H, cfg.d), dtype=torch.bfloat16, device="cuda")
    Pqb, Pkb = synthetic.gen_lowrank_params(cfg, 0)
    lr = sd.LowrankParams(dev_bf16(Pqb), dev_bf16(Pkb))
    g = torch.zeros((1, cfg.L), dtype=torch.float32, device="cuda")
    out = torch.zeros_like(Q)
    k = sd.sd_keep_count(0.5, -(-cfg.L // 64))
    with pytest.raises(sd.SdError) as e:
        sd.sd_rola_attention_noalloc(Q, Q, Q, g, lr, k, out, grid=(cfg.T, cfg.Hg, cfg.Wg), block_q=cfg.block_q)
    assert e.value.status == sd.SD_ERR_UNSUPPORTED
    assert "static buffer" in str(e.value)
    torch.cuda.synchronize()
    assert int(out.view(torch.int16).count_nonzero()) == 0  # nothing ran
