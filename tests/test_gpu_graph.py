"""The decode step captured into a HIP graph (needs an MI355X): mla_decode
allocates nothing and sets no memory, so a serving loop can capture it once and
replay it.  Every replay, with eager calls and synchronisations between them,
must give the eager step's output bit for bit, on the 32K ragged DeepSeek-V3
shape (the 64-head matrix-core kernel) and a small fp32 case (the generic
kernel), each over a cache copy that differs from the eager call's."""
import sys

import pytest
import torch

from head_latent_attention_10_amd import _lib
from head_latent_attention_10_amd.device import Decoder, DeviceInputs
from mla_inputs import CONFIGS, generate

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.load_library()


@pytest.mark.parametrize("name", ["dsv3_ragged_32k", "tiny_fp32"])
def test_decode_graph_replays_match_eager(name):
    print(f"graph replay {name}", flush=True)
    sys.stdout.flush()
    inp = generate(CONFIGS[name])
    dev = DeviceInputs(inp)
    dec = Decoder(dev)
    p = dec.p
    c2 = dev.c_kv.clone()  # the graph reads a second copy of the pool

    def call(c_kv, stream):
        _lib.mla_decode(p, dev.q, c_kv, dev.c_kv_scale, dev.k_rope, dev.block_table, dev.seq_lens,
                        dev.W_UK, dev.W_UV, dec.out, dec.workspace, dec.ws_bytes, stream)

    call(dev.c_kv, torch.cuda.current_stream())
    torch.cuda.synchronize()
    want = dec.out.clone()
    # warm up on a side stream before capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(c2, side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(3):
            call(c2, torch.cuda.current_stream())
    for rep in range(4):
        dec.out.fill_(0)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(dec.out.view(torch.uint8), want.view(torch.uint8)), rep
        # eager work between replays, on the workspace the graph uses
        call(dev.c_kv, torch.cuda.current_stream())
        torch.cuda.synchronize()
        assert torch.equal(dec.out.view(torch.uint8), want.view(torch.uint8)), rep
