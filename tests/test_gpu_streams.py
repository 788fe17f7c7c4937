"""Streams and the per-device descriptor cache.

The library keeps up to kSlotCache descriptor lists on each device (and as
many validated lists per thread) and reuses one when the same list is passed
again; a list moved to another stream waits for the last launch that read it.
These tests run steps on side streams and push lists out of the cache (with
enough one-block filler lists stepped in between), and check every result
against the oracle.
"""

import os
import re

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import DevTensorSet, compare_state, log, oracle_step
from precision_optimizer_step_amd import opt8
from workloads import gen

pytestmark = pytest.mark.gpu

M8 = oracle.MODE_8BIT


@pytest.fixture(scope="module", autouse=True)
def device():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible AMD GPU")
    torch.cuda.set_device(0)
    opt8.opt8_init_codebooks()


def _bf16(rng, n, sigma):
    return gen.to_bf16_bits((rng.standard_normal(n) * sigma).astype(np.float32))


def _make(rng, n, tid, seed):
    p, g = _bf16(rng, n, 0.02), _bf16(rng, n, 1e-3)
    m, v, am, av = gen.random_state_8bit(seed, tid, n)
    return DevTensorSet(M8, p, g, m, v, am, av, tensor_id=tid), [p, m, v, am, av]


def _hp(step):
    return oracle.Hparams(lr=1e-3, weight_decay=0.01, step=step, seed=77)


def _slot_cache():
    """The cache size the library is built with (opt8_host_limits.h)."""
    path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "precision_optimizer_step_amd", "csrc", "opt8_host_limits.h")
    return int(re.search(r"kSlotCache = (\d+);", open(path).read()).group(1))


def _fillers(count, first_id):
    """`count` one-tensor lists of one 2,048-element block each, carved from shared buffers:
    stepped only to push other lists out of the cache, never checked."""
    dev = torch.device("cuda:0")
    n = 2048
    bufs = (torch.zeros(count * n, dtype=torch.bfloat16, device=dev),
            torch.zeros(count * n, dtype=torch.bfloat16, device=dev),
            torch.full((count * n,), 127, dtype=torch.uint8, device=dev),
            torch.zeros(count * n, dtype=torch.uint8, device=dev),
            torch.zeros(count, dtype=torch.float32, device=dev),
            torch.zeros(count, dtype=torch.float32, device=dev))
    P, G, M, V, AM, AV = bufs
    lists = [opt8.tensor_array([opt8.make_tensor(P.data_ptr() + 2 * n * i, G.data_ptr() + 2 * n * i,
                                                 M.data_ptr() + n * i, V.data_ptr() + n * i,
                                                 AM.data_ptr() + 4 * i, AV.data_ptr() + 4 * i,
                                                 tensor_id=first_id + i, mode=M8, numel=n)])
             for i in range(count)]
    return lists, bufs


def _launch(sets, hp, stream):
    descs = [s.desc() for s in sets]
    opt8.opt8_adamw_step(descs, opt8.make_hparams(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay,
                                                  hp.step, hp.seed), stream=stream)


def test_side_streams_and_a_list_moving_between_streams():
    """One list stepped on side stream 1 and, with no host synchronisation in between, on side
    stream 2: the second launch must wait for the first through the library's event (the
    streams themselves are unordered).  Another list runs on the current stream.  Results are
    checked against two oracle steps."""
    rng = np.random.default_rng(5)
    a = [_make(rng, 2048 * 6 + 100, 10 + i, 3) for i in range(3)]
    b = [_make(rng, 2048 * 4, 20 + i, 4) for i in range(2)]
    sa, sta = [x[0] for x in a], [x[1] for x in a]
    sb, stb = [x[0] for x in b], [x[1] for x in b]
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    stats = {}
    for t in range(1, 7, 2):
        _launch(sa, _hp(t), s1)
        _launch(sa, _hp(t + 1), s2)          # ordered after the s1 launch by the library
        _launch(sb, _hp(t), None)
        _launch(sb, _hp(t + 1), None)
        torch.cuda.synchronize()
        for sets, states in ((sa, sta), (sb, stb)):
            for k, (s, st) in enumerate(zip(sets, states)):
                want = oracle_step(s, oracle_step(s, st, _hp(t)), _hp(t + 1))
                compare_state(f"streams steps {t},{t + 1}/t{s.tensor_id}", s.read(), want, M8, stats)
                states[k] = want
    log(f"side streams: mismatches {sum(stats.values())}")
    assert sum(stats.values()) == 0


def test_more_lists_than_cached_slots():
    """Six lists stepped for three rounds, with more filler lists than the cache holds
    stepped after each of them (no host synchronisation in between), so every list is evicted
    and uploaded again each round and slots are rewritten while earlier launches are queued;
    results equal the oracle's."""
    rng = np.random.default_rng(6)
    lists = []
    for li in range(6):
        items = [_make(rng, 2048 * (1 + li) + 37 * li, 100 + 10 * li + k, 8 + li) for k in range(2)]
        lists.append(([x[0] for x in items], [x[1] for x in items]))
    fill, keep = _fillers(_slot_cache() + 8, 5000)
    fhp = opt8.make_hparams(1e-3, 0.9, 0.999, 1e-8, 0.0, 1, 5)
    stats = {}
    for rnd in range(3):
        hp = _hp(rnd + 1)
        for sets, _ in lists:
            _launch(sets, hp, None)
            for f in fill:
                opt8.opt8_adamw_step(f, fhp)
        torch.cuda.synchronize()
        for li, (sets, states) in enumerate(lists):
            for k, (s, st) in enumerate(zip(sets, states)):
                want = oracle_step(s, st, hp)
                compare_state(f"cache round {rnd} list {li}/t{s.tensor_id}", s.read(), want, M8, stats)
                states[k] = want
    log(f"descriptor cache: mismatches {sum(stats.values())}")
    del keep
    assert sum(stats.values()) == 0


def test_concurrent_host_threads():
    """Two host threads, each with its own stream, three lists of its own and more filler
    lists than half the cache holds, launch four rounds of steps with no host synchronisation
    until both have finished: the calls share the device's descriptor cache (evicting each
    other's lists) and must still give each list the oracle's result."""
    import threading

    rng = np.random.default_rng(9)
    groups = []
    for th in range(2):
        lists = []
        for li in range(3):
            items = [_make(rng, 2048 * (2 + li) + 501 * th + 13, 300 + 20 * (3 * th + li) + k, 30 + li)
                     for k in range(2)]
            lists.append(([x[0] for x in items], [x[1] for x in items]))
        groups.append(lists)
    half = _slot_cache() // 2 + 4
    fillers = [_fillers(half, 6000 + th * half) for th in range(2)]
    fhp = opt8.make_hparams(1e-3, 0.9, 0.999, 1e-8, 0.0, 1, 5)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    errors = []

    def worker(th):
        try:
            for rnd in range(4):
                for sets, _ in groups[th]:
                    _launch(sets, _hp(rnd + 1), streams[th])
                for f in fillers[th][0]:
                    opt8.opt8_adamw_step(f, fhp, stream=streams[th])
        except Exception as e:   # re-raised in the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(th,)) for th in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    stats = {}
    for th, lists in enumerate(groups):
        for li, (sets, states) in enumerate(lists):
            for s, st in zip(sets, states):
                want = st
                for rnd in range(4):
                    want = oracle_step(s, want, _hp(rnd + 1))
                compare_state(f"thread {th} list {li}/t{s.tensor_id}", s.read(), want, M8, stats)
    log(f"concurrent host threads: mismatches {sum(stats.values())}")
    assert sum(stats.values()) == 0


def test_graph_capture_is_refused():
    """A step called on a stream that is being captured into a HIP graph returns
    OPT8_E_CAPTURE before anything is queued (the capture ends empty and nothing changes);
    the same step called eagerly afterwards gives the oracle's result."""
    import ctypes

    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipStreamBeginCapture.argtypes = [ctypes.c_void_p, ctypes.c_int]
    hip.hipStreamEndCapture.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p)]
    hip.hipGraphDestroy.argtypes = [ctypes.c_void_p]
    rng = np.random.default_rng(11)
    s, st = _make(rng, 2048 * 2 + 5, 900, 12)
    hp = _hp(1)
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    relaxed = 2   # hipStreamCaptureModeRelaxed
    assert hip.hipStreamBeginCapture(side.cuda_stream, relaxed) == 0
    rc = opt8.opt8_adamw_step([s.desc()], opt8.make_hparams(hp.lr, hp.beta1, hp.beta2, hp.eps,
                                                             hp.weight_decay, hp.step, hp.seed),
                              stream=side, check=False)
    msg = opt8.opt8_last_error()
    graph = ctypes.c_void_p()
    assert hip.hipStreamEndCapture(side.cuda_stream, ctypes.byref(graph)) == 0
    if graph.value:
        assert hip.hipGraphDestroy(graph) == 0
    assert rc == opt8.OPT8_E_CAPTURE, (rc, msg)
    assert "captured" in msg, msg
    torch.cuda.synchronize()
    for got, want in zip(s.read(), st):
        assert np.array_equal(got, want), "a refused step must leave every buffer unchanged"
    _launch([s], hp, None)
    torch.cuda.synchronize()
    stats = {}
    compare_state("after a refused capture", s.read(), oracle_step(s, st, hp), M8, stats)
    assert sum(stats.values()) == 0
