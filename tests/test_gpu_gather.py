"""yoco_gather_last on the GPU against the oracle, bit for bit."""

import json
import os

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_helpers import DeviceWorkload, dev, say
from yoco_shared_kv_gather_amd import binding as yb
from yoco_shared_kv_gather_amd import synth

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _bits(t):
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32).cpu().numpy()


def test_pages_example_rows():
    say("gather: pages' logits-indices example")
    fx = json.load(open(os.path.join(GOLDEN, "vllm_logits_indices_example.json")))
    cu = torch.tensor(fx["printed"]["query_start_loc"], dtype=torch.int32, device=dev())
    hidden = torch.randn(28, 64, device=dev())
    out, idx = yb.gather_last(hidden, cu)
    torch.cuda.synchronize()
    assert idx.cpu().tolist() == fx["derived_for_last_token_gather"]["last_index"]
    ref, ridx = oracle.gather_last(_bits(hidden), fx["printed"]["query_start_loc"])
    assert np.array_equal(_bits(out), ref) and np.array_equal(idx.cpu().numpy(), ridx)


def test_schedule_steps():
    sched = json.load(open(os.path.join(GOLDEN, "vllm_schedule_example.json")))
    for step in sched["steps"]:
        say(f"gather: scheduling step {step['step']}")
        cu = torch.tensor(step["cu_seqlens"], dtype=torch.int32, device=dev())
        hidden = torch.randn(int(step["cu_seqlens"][-1]), 256, device=dev())
        out, idx = yb.gather_last(hidden, cu)
        torch.cuda.synchronize()
        assert idx.cpu().tolist() == step["last_row"]
        assert torch.equal(out, hidden[idx.long()])


@pytest.mark.parametrize("cid,size", [(1, "full"), (2, "small"), (4, "small"), (4, "full"), (3, "edge")])
def test_workload_gather_bit_exact(cid, size):
    say(f"gather: workload {cid} {size}")
    meta = synth.make_metadata(cid, size)
    d = dev()
    hidden = torch.empty((meta.num_tokens, meta.geom.hidden), dtype=synth.torch_dtype(meta.geom), device=d)
    hidden.view(torch.int16 if hidden.element_size() == 2 else torch.int32).random_(-30000, 30000)
    cu = torch.from_numpy(meta.cu_seqlens).to(d)
    out, idx = yb.gather_last(hidden, cu)
    torch.cuda.synchronize()
    ref, ridx = oracle.gather_last(_bits(hidden), meta.cu_seqlens)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert np.array_equal(_bits(out), ref)


def test_empty_requests_and_nan_payloads():
    say("gather: empty requests, NaN payloads")
    d = dev()
    bits = torch.randint(-2 ** 31, 2 ** 31 - 1, (9, 12), dtype=torch.int32, device=d)
    bits[3, 0] = 0x7FC01234
    hidden = bits.view(torch.float32)
    cu = torch.tensor([0, 2, 2, 4, 9, 9], dtype=torch.int32, device=d)
    out, idx = yb.gather_last(hidden, cu)
    torch.cuda.synchronize()
    ref, ridx = oracle.gather_last(bits.cpu().numpy(), cu.cpu().numpy())
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert np.array_equal(out.view(torch.int32).cpu().numpy(), ref)
