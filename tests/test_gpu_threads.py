"""Several host threads calling the library at once, each on its own HIP stream.

The entry points keep per-thread error state and a per-device cache of the compute-unit
count; none of this may mix up concurrent callers.  Each thread runs a fixed sequence (a
colwise GEMM with GELU, a rowwise partial, a 5-row weight-streaming call with 60 KiB of
staged activations, an 8-row split-K call, a SUM and an invalid call) several times; every result must equal the same sequence run alone on
the default stream, bit for bit, and each thread must see its own error message."""
import threading

import numpy as np
import pytest
import torch

import synth_inputs as si
import tensor_sharded_linear_amd as tsl
from helpers import bits_to_dev

pytestmark = pytest.mark.gpu


def _inputs(seed):
    rng = np.random.default_rng(seed)
    x = bits_to_dev(si.normal_bf16(rng, (640, 1024)))
    w = bits_to_dev(si.normal_bf16(rng, (512, 1024), 1 / 32))
    w2 = bits_to_dev(si.normal_bf16(rng, (256, 512), 1 / 23))
    b = bits_to_dev(si.normal_bf16(rng, (512,)))
    c = bits_to_dev(si.normal_bf16(rng, (8, 6144)))
    wa = bits_to_dev(si.normal_bf16(rng, (1024, 6144), 1 / 78))
    return x, w, w2, b, c, wa


def _sequence(inp, stream):
    x, w, w2, b, c, wa = inp
    with torch.cuda.stream(stream):
        h = tsl.tp_linear_colwise(x, w, b, act="gelu_tanh", stream=stream)
        p0 = tsl.tp_linear_rowwise(h, w2, stream=stream)
        p1 = tsl.tp_linear_rowwise(h, w2.flip(0).contiguous(), stream=stream)
        s = tsl.tp_partial_combine([p0, p1], "sum", stream=stream)
        y = tsl.tp_linear_colwise(c[:5], wa, stream=stream)   # 5 rows x 6144: 60 KiB of LDS
        z = tsl.tp_linear_colwise(c, wa, act="gelu_tanh", stream=stream)   # 8 rows: split-K
    stream.synchronize()
    return [t.clone() for t in (h, p0, s, y, z)]


def test_concurrent_threads_on_separate_streams():
    inputs = [_inputs(100 + i) for i in range(4)]
    ref = [_sequence(inp, torch.cuda.current_stream()) for inp in inputs]
    results = [None] * 4
    errors = [None] * 4
    failures = []

    def worker(i):
        try:
            s = torch.cuda.Stream()
            out = None
            for _ in range(5):
                out = _sequence(inputs[i], s)
                with pytest.raises(ValueError):
                    tsl.tp_linear_colwise(inputs[i][0], inputs[i][1][:500])   # N % 16 != 0
                errors[i] = tsl.tp_last_error()
            results[i] = out
        except Exception as e:  # noqa: BLE001 -- reported below with the thread index
            failures.append((i, repr(e)))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(4)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not failures, failures
    for i in range(4):
        for a, b in zip(results[i], ref[i]):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)), i
        assert errors[i].startswith("tp_linear_colwise") and "16" in errors[i], errors[i]
