"""The entry points are safe to capture in a HIP graph: they allocate,
synchronise and memset nothing, so a captured decode (split kernel + merge
kernel) and a captured prefill replay to the eager result bit for bit.  Each
graph is replayed several times with new inputs copied into its static
buffers and with eager work and synchronisations between the replays, and
every replay is compared."""
import pytest
import torch

from gpu_common import gpu_available, say

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _replays(capture_fn, make_inputs, static, n=3):
    g = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        capture_fn()                      # warm-up outside the graph, on the capture stream
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=stream):
        out = capture_fn()
    results = []
    for i in range(n):
        fresh = make_inputs(100 + i)
        for k, t in fresh.items():
            static[k].copy_(t)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        results.append((out.clone(), fresh))
        _ = torch.randn(1024, device="cuda").sum().item()  # eager work between replays
    return results


def test_decode_split_and_merge_in_a_graph():
    import transformer_attention_flash_amd as plx
    from transformer_attention_flash_amd import synth
    B, Hq, Hkv, L, d = 4, 8, 4, 1000, 128
    say("graph: decode B=4 Hq=8 Hkv=4 L=1000 d=128, 256-key chunks (split + merge)")
    static = synth.make_decode(B, Hq, Hkv, L, d, torch.bfloat16, "cuda", seed=0)
    ws = torch.empty(plx.decode_workspace_size(B, Hq, Hkv, d, L, keys_per_split=256), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty_like(static["q"])

    def run():
        return plx.decode(static["q"], static["k"], static["v"], static["rho"], out=out, keys_per_split=256,
                          workspace=ws)

    def make(seed):
        return synth.make_decode(B, Hq, Hkv, L, d, torch.bfloat16, "cuda", seed=seed)

    for got, x in _replays(run, make, static):
        want = plx.decode(x["q"], x["k"], x["v"], x["rho"], keys_per_split=256)
        torch.cuda.synchronize()
        assert torch.equal(got, want)


def test_prefill_in_a_graph():
    import transformer_attention_flash_amd as plx
    from transformer_attention_flash_amd import synth
    B, Hq, Hkv, T, d = 1, 4, 2, 300, 128
    say("graph: prefill B=1 Hq=4 Hkv=2 T=300 d=128")
    static = synth.make_prefill(B, Hq, Hkv, T, d, torch.bfloat16, "cuda", seed=0)
    out = torch.empty_like(static["q"])

    def run():
        return plx.prefill(static["q"], static["k"], static["v"], static["rho"], out=out)

    def make(seed):
        return synth.make_prefill(B, Hq, Hkv, T, d, torch.bfloat16, "cuda", seed=seed)

    for got, x in _replays(run, make, static):
        want = plx.prefill(x["q"], x["k"], x["v"], x["rho"])
        torch.cuda.synchronize()
        assert torch.equal(got, want)
