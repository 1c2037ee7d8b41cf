"""The probes (include/a2av_probe.h) run and move what they say: the copy
probe's output equals its input, the write probe fills its buffer with 0xA5,
the read probe writes nothing, the launch probe writes its bytes and nothing
past them, regular or cooperative; bad arguments are refused."""
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from all_movement_amd import a2av  # noqa: E402
from all_movement_amd import workloads as wl  # noqa: E402
from tests.gpu_harness import DEV, say  # noqa: E402


@pytest.fixture(autouse=True)
def _gpu_or_skip():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("nbytes", [16, 131072 - 16, (3 << 20) + 48, 64 << 20])
def test_probes_move_what_they_say(nbytes):
    src = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    wl.fill_random_(src, 77)
    dst = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    stream = torch.cuda.current_stream(DEV).cuda_stream
    say("probe bytes", nbytes)
    for _ in range(2):                      # twice: the tile counter is cleared each launch
        assert a2av.a2av_probe_stream(a2av.PROBE_COPY, src.data_ptr(), dst.data_ptr(), nbytes, 0,
                                      stream) == a2av.OK
        torch.cuda.synchronize()
        assert torch.equal(src, dst)
    dst.zero_()
    assert a2av.a2av_probe_stream(a2av.PROBE_READ, src.data_ptr(), None, nbytes, 0,
                                  stream) == a2av.OK
    assert a2av.a2av_probe_stream(a2av.PROBE_READ, src.data_ptr(), dst.data_ptr(), nbytes, 7,
                                  stream) == a2av.OK
    torch.cuda.synchronize()
    assert int(dst.count_nonzero()) == 0
    assert a2av.a2av_probe_stream(a2av.PROBE_WRITE, None, dst.data_ptr(), nbytes, 0,
                                  stream) == a2av.OK
    torch.cuda.synchronize()
    assert bool((dst == 0xA5).all())


def test_probe_rejects_bad_arguments():
    buf = torch.empty(4096, dtype=torch.uint8, device=DEV)
    p = buf.data_ptr()
    run = lambda kind=a2av.PROBE_COPY, s=p, d=p + 2048, n=1024, w=0: (  # noqa: E731
        a2av.a2av_probe_stream(kind, s, d, n, w, None))
    assert run(kind=3) == a2av.ERR_INVALID_ARGS
    assert run(s=None) == a2av.ERR_NULLPTR
    assert run(kind=a2av.PROBE_WRITE, d=None) == a2av.ERR_NULLPTR
    assert run(n=0) == a2av.ERR_INVALID_ARGS
    assert run(n=1000) == a2av.ERR_INVALID_ARGS
    assert run(s=p + 4) == a2av.ERR_INVALID_ARGS
    assert run(w=-1) == a2av.ERR_INVALID_ARGS


@pytest.mark.parametrize("coop", [0, 1])
@pytest.mark.parametrize("nbytes", [0, 16, (1 << 20) + 32, 64 << 20])
def test_launch_probe_writes_its_bytes(coop, nbytes):
    buf = torch.zeros(nbytes + 4096, dtype=torch.uint8, device=DEV)
    stream = torch.cuda.current_stream(DEV).cuda_stream
    say("launch probe", coop, nbytes)
    for w in (0, 64):
        assert a2av.a2av_probe_launch(coop, buf.data_ptr(), nbytes, w, stream) == a2av.OK
        torch.cuda.synchronize()
        assert bool((buf[:nbytes] == 0xA5).all())
        assert int(buf[nbytes:].count_nonzero()) == 0
    assert a2av.a2av_probe_launch(coop, None, 0, 0, stream) == a2av.OK
    torch.cuda.synchronize()


def test_launch_probe_rejects_bad_arguments():
    buf = torch.empty(4096, dtype=torch.uint8, device=DEV)
    p = buf.data_ptr()
    run = lambda coop=0, d=p, n=1024, w=0: a2av.a2av_probe_launch(coop, d, n, w, None)  # noqa: E731
    assert run(coop=2) == a2av.ERR_INVALID_ARGS
    assert run(coop=-1) == a2av.ERR_INVALID_ARGS
    assert run(d=None) == a2av.ERR_NULLPTR
    assert run(n=-16) == a2av.ERR_INVALID_ARGS
    assert run(n=1000) == a2av.ERR_INVALID_ARGS
    assert run(n=1 << 31) == a2av.ERR_INVALID_ARGS
    assert run(d=p + 4) == a2av.ERR_INVALID_ARGS
    assert run(w=-1) == a2av.ERR_INVALID_ARGS
