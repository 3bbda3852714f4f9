"""A captured forward replays correctly: several replays of a HIP graph holding
one layer forward, with eager work and synchronizations in between, each give
the eager result byte for byte: the decode path (8-row tiles; split K at one
token, with two strips per wave and K-chunks on the Mixtral shape; 16-row
tiles in two K-chunks; the Zipf-skewed layer with its tiles grouped by XCD;
at T = 2048 with the MFMA router, its group-sum pass and the multi-block
grouping), and the large-batch path with int4 and staged (int8/bf16) tiers."""

import numpy as np
import pytest

from tests._harness import Setup, log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cid,T", [(2, 32), (1, 64), (3, 512), (4, 2048), (4, 1), (5, 1),
                                   (6, 128), (3, 64)])
def test_graph_replay_matches_eager(cid, T):
    import torch
    st = Setup(cid, T=T)
    layer = st.gpu_layer()
    x, wr, b = st.dev_inputs()
    log(f"graph replay cfg{cid} T={T}")
    y_eager = layer.forward(x, wr, b, out_dtype=torch.float32).clone()
    torch.cuda.synchronize()
    ref = y_eager.cpu().numpy().view(np.uint32)
    ws = layer.workspace(T, x.device)
    y = torch.empty_like(y_eager)
    layer.forward(x, wr, b, y=y, workspace=ws)      # warm up on the side stream
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.bind_forward(x, wr, b, y, workspace=ws, stream=torch.cuda.current_stream())()
    for rep in range(4):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy().view(np.uint32), ref), f"replay {rep}"
        # unrelated eager work between replays
        z = layer.forward(x, wr, b, out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        assert z.shape == y.shape
