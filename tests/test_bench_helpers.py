"""Host logic of bench.py that its JSON line depends on: the counter summaries
behind roofline.traffic are read back, and dropped once the kernels they were
taken on change."""
import os
import shutil

import bench


def test_committed_traffic_summaries_match_sources():
    # both summaries in profiles/ were taken on the kernels as committed
    assert bench.measured_traffic() is not None
    assert bench.measured_traffic(bench.PREFILL_TRAFFIC_FILE, bench.PREFILL_SOURCES) is not None


def test_traffic_is_dropped_when_sources_change(tmp_path):
    root = tmp_path / "repo"
    for rel in bench.DECODE_SOURCES:
        dst = root / rel
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(bench.ROOT, rel), dst)
    summary = tmp_path / "traffic.txt"
    digest_of = lambda: bench.sources_digest([str(root / r) for r in bench.DECODE_SOURCES])
    summary.write_text(f"# comment: 1\nbytes_per_call: 1234\nsources_sha256_16: {digest_of()}\n")
    srcs = [str(root / r) for r in bench.DECODE_SOURCES]
    assert bench.measured_traffic(str(summary), srcs) == 1234
    with open(srcs[0], "a") as f:            # any edit of a kernel source
        f.write("\n// edited\n")
    assert bench.measured_traffic(str(summary), srcs) is None
    assert bench.measured_traffic(str(tmp_path / "missing.txt"), srcs) is None


class _Recorder:
    """Stands in for the binding: records the calls a decode step makes."""
    ACC_BUFS = 8

    def __init__(self):
        self.calls = []

    @staticmethod
    def MoeLayer(*args):
        return args

    @staticmethod
    def decode_workspace_bytes(layer, T):
        return 256

    def decode_layer_acc(self, L, x, logits, table, acc_out, acc_clear=None, prev=None, **kw):
        self.calls.append(("layer", L, x, acc_out, acc_clear, prev))

    def decode_acc_finish(self, x, acc, y=None):
        self.calls.append(("finish", x, acc, y))


def test_decode_step_buffer_rotation():
    """The timed decode step (one accumulate-mode call per layer): every call
    adds into a buffer that is zero (cleared by the call before, or zero from
    the start), forms the previous layer's y from that layer's x and buffer,
    and the finish forms the last y; after a step the first buffer is zero
    again, so the next step can start."""
    import torch
    import synth
    rec = _Recorder()
    shape = synth.LayerShape(8, 2, 64, 32, True)
    n = 6
    pools = [(torch.zeros((9, 1), dtype=torch.uint8), torch.zeros(8, dtype=torch.int32), 8,
              synth.FMT_Q2SM) for _ in range(n)]
    xs = [torch.zeros((1, 64)) for _ in range(n)]
    chain = bench.DecodeChain(torch, rec, shape, pools, 1, "cpu", xs, acc=True)
    for step in range(2):
        zero = {id(b): True for b in chain.accs} if step == 0 else zero
        rec.calls.clear()
        chain.step([None] * n)
        layers = [c for c in rec.calls if c[0] == "layer"]
        assert len(layers) == n and rec.calls[-1][0] == "finish"
        for l, (_, L, x, acc_out, acc_clear, prev) in enumerate(layers):
            assert x is xs[l]
            assert zero[id(acc_out)], f"layer {l} adds into a buffer that is not zero"
            zero[id(acc_out)] = False
            assert acc_clear is not acc_out
            assert prev is None or acc_clear is not prev[1], "a call clears what it reads"
            if acc_clear is not None:
                zero[id(acc_clear)] = True
            if l == 0:
                assert prev is None
            else:
                px, pacc, py = prev
                assert px is xs[l - 1] and pacc is layers[l - 1][3] and py is chain.y
        _, fx, facc, fy = rec.calls[-1]
        assert fx is xs[-1] and facc is layers[-1][3] and fy is chain.y
        assert zero[id(layers[0][3])], "the next step's first buffer is not cleared"
