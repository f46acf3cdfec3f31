"""GPU parity of mscl_reduce_scatter and mscl_allgather against the oracle.

ReduceScatter is bit-exact against oracle.reduce_scatter (same accumulation
rule); AllGather is a bit copy, checked against oracle.allgather on arbitrary
bit patterns (NaN payloads included).  Both the 16-byte vector path and the
element path (block boundaries not 16-byte aligned, or base pointers only
element-aligned) are covered, in place and out of place, plus a full-size
case at the 128 MiB prefill shape.
"""

import numpy as np
import pytest
import torch

import gpu_helpers as G
import oracle_pins as P
from allreduce_emulated_peer_amd import mscl as M
from allreduce_emulated_peer_amd import workloads as W
from oracle import allreduce as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    M.load()
    yield


def random_bits(R, n, dtype, seed):
    g = np.random.default_rng(seed)
    width = 32 if dtype == "fp32" else 16
    return [P.from_bits(g.integers(0, 2 ** width, size=n, dtype=np.uint64).astype(
        np.uint32 if width == 32 else np.uint16), dtype) for _ in range(R)]


def flat_device(xs, dtype, lead=0):
    """One device allocation per rank, each buffer starting `lead` elements in
    (lead = 1 gives element-aligned but not 16-byte aligned pointers)."""
    out = []
    for x in xs:
        t = G.to_device(np.concatenate([np.zeros(lead, dtype=x.dtype), x]) if lead else x, dtype)
        out.append(t[lead:] if lead else t)
    return out


RS_COUNTS = (1, 3, 4, 8, 9, 64, 1000, 4099, 65536)


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
def test_reduce_scatter_small(dtype):
    for R in (1, 2, 3, 8, 16):
        for rc in RS_COUNTS:
            xs = P.rand_inputs(R, R * rc, dtype, seed=R * 100 + rc, scale=16.0)
            want = O.reduce_scatter(xs, dtype)
            for lead in (0, 1):
                G.channel(R)
                ins = flat_device(xs, dtype, lead)
                outs = [G.poison_like(ins[0][:rc]) for _ in range(R)]
                G.note(f"reduce_scatter {dtype} R={R} rc={rc} lead={lead}")
                M.reduce_scatter([t.data_ptr() for t in ins], [t.data_ptr() for t in outs], rc, G.CODES[dtype], R,
                                 torch.cuda.current_stream().cuda_stream)
                torch.cuda.synchronize()
                for r in range(R):
                    got = G.to_host_bits(outs[r], dtype)
                    wb = O.bits_of(want[r], dtype)
                    assert np.all(O.ulp_distance(got, wb, dtype) == 0), f"{dtype} R={R} rc={rc} lead={lead} block {r}"


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_reduce_scatter_in_place(dtype):
    for R, rc in ((4, 4096), (8, 1001), (16, 65536)):
        xs = P.rand_inputs(R, R * rc, dtype, seed=rc)
        want = O.reduce_scatter(xs, dtype)
        ins = [G.to_device(x, dtype) for x in xs]
        outs = [ins[r][r * rc:(r + 1) * rc] for r in range(R)]  # block r of inputs[r]
        G.channel(R)
        G.note(f"reduce_scatter in place {dtype} R={R} rc={rc}")
        M.reduce_scatter([t.data_ptr() for t in ins], [t.data_ptr() for t in outs], rc, G.CODES[dtype], R,
                         torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        for r in range(R):
            assert np.array_equal(G.to_host_bits(outs[r], dtype), O.bits_of(want[r], dtype))


AG_COUNTS = (1, 2, 7, 8, 16, 1000, 4099, 65536)


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
def test_allgather_small(dtype):
    for R in (1, 2, 3, 8, 16):
        for sc in AG_COUNTS:
            xs = random_bits(R, sc, dtype, seed=R * 1000 + sc)
            want = O.bits_of(O.allgather(xs, dtype)[0], dtype)
            for lead in (0, 1):
                G.channel(R)
                ins = flat_device(xs, dtype, lead)
                outs = [G.poison_like(torch.empty(R * sc, dtype=ins[0].dtype, device="cuda")) for _ in range(R)]
                G.note(f"allgather {dtype} R={R} sc={sc} lead={lead}")
                M.allgather([t.data_ptr() for t in ins], [t.data_ptr() for t in outs], sc, G.CODES[dtype], R,
                            torch.cuda.current_stream().cuda_stream)
                torch.cuda.synchronize()
                for p in range(R):
                    assert np.array_equal(G.to_host_bits(outs[p], dtype), want), f"{dtype} R={R} sc={sc} lead={lead} out {p}"


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_allgather_in_place(dtype):
    for R, sc in ((2, 8), (8, 4097), (16, 65536)):
        xs = random_bits(R, sc, dtype, seed=sc)
        want = O.bits_of(O.allgather(xs, dtype)[0], dtype)
        outs = []
        for r in range(R):
            o = G.poison_like(torch.empty(R * sc, dtype=G.TORCH_DTYPES[dtype], device="cuda"))
            o[r * sc:(r + 1) * sc].copy_(G.to_device(xs[r], dtype))
            outs.append(o)
        ins = [outs[r][r * sc:(r + 1) * sc] for r in range(R)]  # inputs[r] = block r of outputs[r]
        G.channel(R)
        G.note(f"allgather in place {dtype} R={R} sc={sc}")
        M.allgather([t.data_ptr() for t in ins], [t.data_ptr() for t in outs], sc, G.CODES[dtype], R,
                    torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        for p in range(R):
            assert np.array_equal(G.to_host_bits(outs[p], dtype), want)


def test_full_size_prefill_shape():
    """R = 8 bf16: ReduceScatter of the 128 MiB prefill buffers (16 MiB blocks)
    and AllGather of those blocks back into 128 MiB outputs; the round trip
    equals the AllReduce."""
    w = W.prefill_bf16()
    xs = W.generate_all(w)
    R, rc = w.nranks, w.count // w.nranks
    ins = [G.to_device(x, "bf16") for x in xs]
    blocks = [torch.empty(rc, dtype=torch.bfloat16, device="cuda") for _ in range(R)]
    G.channel(R)
    stream = torch.cuda.current_stream().cuda_stream
    G.note("reduce_scatter 8 x 128 MiB")
    M.reduce_scatter([t.data_ptr() for t in ins], [t.data_ptr() for t in blocks], rc, M.BFLOAT16, R, stream)
    want = O.allreduce(xs, "bf16")
    torch.cuda.synchronize()
    for r in range(R):
        G.assert_matches_oracle_on_device([blocks[r]], want[r * rc:(r + 1) * rc], "bf16", f"block {r}")
    outs = [torch.empty(w.count, dtype=torch.bfloat16, device="cuda") for _ in range(R)]
    G.note("allgather 8 x 16 MiB -> 8 x 128 MiB")
    M.allgather([t.data_ptr() for t in blocks], [t.data_ptr() for t in outs], rc, M.BFLOAT16, R, stream)
    torch.cuda.synchronize()
    G.assert_matches_oracle_on_device(outs, want, "bf16", "reduce_scatter + allgather")


def test_allreduce_tensors_wrapper():
    """The torch convenience wrapper: dtype from the tensors, torch's current
    stream by default, an explicit stream, in place."""
    R, n = 4, 50_001
    w = W.custom(R, "bf16", n, "normal", seed_index=21)
    xs = W.generate_all(w)
    want = O.bits_of(O.allreduce(xs, "bf16"), "bf16")
    G.channel(R)
    ins = [G.to_device(x, "bf16") for x in xs]
    outs = [G.poison_like(t) for t in ins]
    G.note("allreduce_tensors R=4 bf16 default stream")
    M.allreduce_tensors(ins, outs)
    torch.cuda.synchronize()
    for o in outs:
        assert np.array_equal(G.to_host_bits(o, "bf16"), want)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    G.note("allreduce_tensors R=4 bf16 explicit stream, in place")
    M.allreduce_tensors(ins, ins, algo=M.ALGO_TWO_SHOT, stream=s)
    s.synchronize()
    for t in ins:
        assert np.array_equal(G.to_host_bits(t, "bf16"), want)


def test_process_exits_cleanly_with_a_running_proxy():
    """A process that used the port channel and exits without destroying its
    channel set must still exit normally: the library stops every proxy
    thread at exit, before the HIP runtime tears down."""
    import os
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = (
        "import torch\n"
        "from allreduce_emulated_peer_amd import mscl as M\n"
        "M.channel_create(4, 0)\n"
        "x = [torch.ones(1 << 16, device='cuda', dtype=torch.bfloat16) for _ in range(4)]\n"
        "y = [torch.empty_like(t) for t in x]\n"
        "M.allreduce_tensors(x, y, algo=M.ALGO_TWO_SHOT_PORT)\n"
        "torch.cuda.synchronize()\n"
        "assert bool((y[3] == 4).all())\n"
        "print('done', flush=True)\n"
    )
    G.note("subprocess: port call, then exit with the proxy running")
    r = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr[-2000:]
    assert "done" in r.stdout
    assert "terminate" not in r.stderr and "Segmentation" not in r.stderr
