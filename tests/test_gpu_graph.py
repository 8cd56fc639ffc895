"""The library's calls captured into a HIP graph: every replay, with the
program's own eager work and synchronizations in between, must reproduce the
eager result bit for bit.  Every call below is deterministic: row scans and
reductions combine in a fixed order for a given size and pointer alignment,
and the device scans here are integer or min/max scans and select, whose
results are exact whatever order the look-back combines descriptors in.  (A
floating-add device scan is not in this list: its look-back may take a
predecessor's inclusive prefix or its aggregate, depending on timing, so its
last bits can differ from run to run, within the float tolerance.)  Each call
resets its descriptors with a fill kernel rather than hipMemsetAsync, so it
can sit in a graph."""
import numpy as np
import pytest
import torch

import stream_compaction_amd as sc
import workloads

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    dev = torch.device("cuda")
    rows, n = 64, 3001
    nd, ns = 1_000_003, 700_001
    x = torch.empty((rows, n), dtype=torch.bfloat16, device=dev)
    xi = torch.empty(nd, dtype=torch.int32, device=dev)
    xf = torch.empty(nd, dtype=torch.float32, device=dev)
    pay = torch.empty(ns, dtype=torch.float32, device=dev)
    fl = torch.empty(ns, dtype=torch.uint8, device=dev)
    y1 = torch.empty_like(x)
    y2 = torch.empty_like(xi)
    y3 = torch.empty_like(xf)
    y4 = torch.full_like(pay, -1.0)
    y5 = torch.empty_like(xi)
    y6 = torch.empty(1, dtype=torch.float32, device=dev)
    y7 = torch.empty_like(x)
    s6 = torch.empty(sc.reduce_device_scratch_bytes(nd, "f32"), dtype=torch.uint8, device=dev)
    num = torch.empty(1, dtype=torch.int32, device=dev)
    s2 = torch.empty(sc.scan_device_scratch_bytes(nd, "i32"), dtype=torch.uint8, device=dev)
    s3 = torch.empty(sc.scan_device_scratch_bytes(nd, "f32"), dtype=torch.uint8, device=dev)
    s4 = torch.empty(sc.select_compact_scratch_bytes(ns), dtype=torch.uint8, device=dev)

    def fill(rep):
        bits = workloads.normal_bf16((rows, n), 100 + rep)
        x.copy_(torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16))
        xi.copy_(torch.from_numpy(workloads.uniform_ints(nd, 0, 15, 200 + rep)))
        xf.copy_(torch.from_numpy(workloads.uniform_f32(nd, 300 + rep, -1e6, 1e6)))
        p, f = workloads.payload_f32(ns, 400 + rep), workloads.bernoulli_flags(ns, 0.3, 500 + rep)
        pay.copy_(torch.from_numpy(p))
        fl.copy_(torch.from_numpy(f))

    def calls():
        sc.scan_rows(x, "add", True, out=y1)
        sc.scan_device(xi, "add", out=y2, scratch=s2)
        sc.scan_device(xf, "max", out=y3, scratch=s3)
        sc.select_compact(pay, fl, out=y4, num_out=num, scratch=s4)
        sc.scan_device_inclusive(xi, "add", out=y5, scratch=s2)
        sc.reduce_device(xf, "add", out=y6, scratch=s6)
        sc.scan_rows(x, "mul", False, out=y7)

    fill(0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()                                 # eager warm-up off the default stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    for rep in range(1, 5):
        fill(rep)                               # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (y1, y2, y3, y4, num, y5, y6, y7)]
        e1 = sc.scan_rows(x, "add", True)
        e2 = sc.scan_device(xi, "add")
        e3 = sc.scan_device(xf, "max")
        e4, en = sc.select_compact(pay, fl, out=torch.full_like(pay, -1.0))
        e5 = sc.scan_device_inclusive(xi, "add")
        e6 = sc.reduce_device(xf, "add")
        e7 = sc.scan_rows(x, "mul", False)
        torch.cuda.synchronize()
        assert torch.equal(got[5], e5), rep
        assert torch.equal(got[6].view(torch.int32), e6.view(torch.int32)), rep
        assert torch.equal(got[7].view(torch.int16), e7.view(torch.int16)), rep
        assert torch.equal(got[0].view(torch.int16), e1.view(torch.int16)), rep
        assert torch.equal(got[1], e2), rep
        assert torch.equal(got[2].view(torch.int32), e3.view(torch.int32)), rep
        k = int(en.item())
        assert int(got[4].item()) == k, rep
        # the prefix is the result; past it the graph's buffer holds earlier replays' output
        assert torch.equal(got[3][:k].view(torch.int32), e4[:k].view(torch.int32)), rep
