"""Concurrent use as the boundary documents it: one handle per stream.  Two host
threads, each with its own handle and its own (default-priority) stream, enqueue
calls at the same time; the split-H variant is forced on both, so each call also
uses its handle's workspace.  Every output is checked against the oracle."""
import threading

import numpy as np
import pytest
import torch

import residual_add_rmsnorm_arrms_amd as A
import synth
from tests.gpu_util import assert_parity, inputs, reference, say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


@pytest.mark.parametrize("variant", [A.ARRMS_VARIANT_SPLITH, A.ARRMS_VARIANT_ROW])
def test_two_threads_two_handles_two_streams(variant):
    say("case concurrency variant=%d" % variant)
    W, T, H, calls = 4, 48, 4096, 25
    jobs = []
    for j in range(2):
        x, r, w = inputs(W, T, H, seed=900 + j)
        op = A.FusedReduceResidualRMSNorm(max_world=W, max_tokens=T, max_hidden=H, device=0)
        op.set_variant(variant)
        outs = [(torch.empty((T, H), dtype=torch.bfloat16, device=DEV),
                 torch.empty((T, H), dtype=torch.bfloat16, device=DEV)) for _ in range(calls)]
        jobs.append(dict(x=x, r=r, w=w, xd=x.to(DEV), rd=r.to(DEV), wd=w.to(DEV), op=op, stream=torch.cuda.Stream(),
                         outs=outs, error=None))
    torch.cuda.synchronize()
    barrier = threading.Barrier(2)

    def work(job):
        try:
            torch.cuda.set_device(DEV)
            barrier.wait()
            for ro, no in job["outs"]:
                job["op"](job["xd"], job["rd"], job["wd"], 1e-6, ro, no, stream=job["stream"])
        except Exception as e:  # reported by the main thread
            job["error"] = e

    threads = [threading.Thread(target=work, args=(job,)) for job in jobs]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not any(t.is_alive() for t in threads), "a host thread did not finish"
    torch.cuda.synchronize()
    for j, job in enumerate(jobs):
        assert job["error"] is None, job["error"]
        ref = reference(job["x"], job["r"], job["w"], 1e-6)
        first = None
        for k, (ro, no) in enumerate(job["outs"]):
            got_ro, got_no = synth.bits(ro.cpu()), synth.bits(no.cpu())
            if first is None:
                first = (got_ro, got_no)
                assert_parity(got_ro, got_no, ref, "concurrent job %d" % j)
            else:  # every call of a job gives the same bits
                assert np.array_equal(got_ro, first[0]) and np.array_equal(got_no, first[1]), (j, k)
        job["op"].close()
