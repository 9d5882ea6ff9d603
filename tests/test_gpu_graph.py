"""The decode step captured in a HIP graph (torch.cuda.CUDAGraph over the
library's launches on the capture stream): every replay, over several input
sets copied into the captured input buffers, with unrelated eager work and
synchronisations between the replays, is bit for bit the eagerly issued
step on the same inputs.  The launches allocate nothing and record no
memset, so the step is capturable as a serving loop would capture it.
"""
import sys

import numpy as np
import pytest
import torch

import dsa_inputs

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from sparse_attention_indexer_topk_amd.pipeline import DecodePath  # noqa: E402


def snapshot(path):
    t = [path.cand, path.slots, path.counts, path.pout, path.plse, path.out, path.lse]
    if path.prologue is not None:
        t += [path.kv_c_out, path.k_pe_out, path.cache]
    return [x.clone() for x in t]


def same(a, b):
    """Bit for bit (as bytes: -inf scores and empty partials compare too)."""
    return all(torch.equal(x.contiguous().view(torch.uint8), y.contiguous().view(torch.uint8))
               for x, y in zip(a, b))


@pytest.mark.parametrize("name", ["decode_s", "fp8_s"])
def test_step_replays_bit_identical_in_a_hip_graph(name):
    print(f"[graph] case {name}", file=sys.stderr, flush=True)
    c = dsa_inputs.make(name)
    path = DecodePath(**dsa_inputs.device_arrays(c))
    dev = path.logits.device
    sets = [(path.logits.clone(), path.q.clone())]
    for s in range(1, 3):
        lg, qq = dsa_inputs.redraw_logits_q(c, s)
        sets.append((torch.from_numpy(lg).to(dev),
                     torch.from_numpy(qq.view(np.int16)).to(dev).view(torch.bfloat16)))

    def load(i):
        path.logits.copy_(sets[i][0])
        path.q.copy_(sets[i][1])

    # eager references (the prologue rewrites the same cache slots with the
    # same rows every step, so the references stay valid across replays)
    refs = []
    for i in range(len(sets)):
        load(i)
        path.step()
        torch.cuda.synchronize()
        refs.append(snapshot(path))

    # warm-up on a side stream, as torch asks before a capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        path.step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        path.step()
    torch.cuda.synchronize()

    noise = torch.randn(512, 512, device=dev)
    for rep in range(3):
        for i in range(len(sets)):
            load(i)
            g.replay()
            torch.cuda.synchronize()
            assert same(snapshot(path), refs[i]), f"replay {rep}, input set {i} differs"
            # unrelated eager work between replays
            noise = torch.tanh(noise @ noise.T * 1e-3)
            torch.cuda.synchronize()
