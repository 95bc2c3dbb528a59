"""The HBM read-ceiling probe (mpk_stream_read) reads every byte it is given:
a buffer of zeros leaves the sink word alone, and a buffer whose only
non-zero word makes one lane's XOR equal the probe's constant has the probe
store that constant (for any launch shape, since the word's unit is read by
whichever workgroup takes it)."""
import pytest

import persistent_task_runtime_amd as mpk

pytestmark = pytest.mark.gpu

MAGIC = 0x6A09E667


@pytest.mark.parametrize("workgroups", [1, 256, 1000])
def test_stream_read_touches_every_unit(rocm_device, workgroups):
    import torch

    n = 64 * 128 * 1024  # 64 units of 128 KiB
    buf = torch.zeros(n // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    print("stream_read zeros: workgroups %d, %d bytes" % (workgroups, n), flush=True)
    mpk.mpk_stream_read(buf.data_ptr(), n, workgroups, sink.data_ptr(), stream)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0
    # one word in the last unit: only a complete read finds it
    buf[n // 4 - 3] = MAGIC
    print("stream_read planted word: workgroups %d" % workgroups, flush=True)
    mpk.mpk_stream_read(buf.data_ptr(), n, workgroups, sink.data_ptr(), stream)
    torch.cuda.synchronize()
    assert int(sink.item()) & 0xFFFFFFFF == MAGIC
