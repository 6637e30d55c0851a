"""Host logic of bench.py that its JSON line depends on: the counter summaries
behind roofline.traffic are read back, and dropped once the kernels they were
taken on change."""
import os
import shutil

import bench


def test_committed_traffic_summaries_match_sources():
    # the summaries in profiles/ were taken on the kernels as committed
    assert bench.measured_traffic() is not None
    assert bench.measured_traffic(bench.VERIFY_TRAFFIC_FILE, bench.DECODE_SOURCES) is not None
    assert bench.measured_traffic(bench.PREFILL_TRAFFIC_FILE, bench.PREFILL_SOURCES) is not None
    m = bench.mfma_busy_counters()
    assert m is not None and 0 < m["gate_up"] < 1 and 0 < m["down"] < 1


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


class _FakeBinding:
    """Stands in for the binding: a one-layer decode_stack call returns
    y = 2 x + layer number; full calls are recorded."""

    def __init__(self):
        self.calls = []

    @staticmethod
    def MoeLayer(*args):
        return args

    @staticmethod
    def new_stack_workspace(layers, T):
        import torch
        return torch.zeros(256, dtype=torch.uint8)

    def decode_stack(self, layers, x, logits, tables, addends=None, ys=None, ws=None,
                     routing=False):
        if len(layers) == 1:
            ys.copy_(2 * x + layers[0][4])
            return {"y": ys}
        self.calls.append((layers, x, logits, tables, addends, ys, ws, routing))
        return {"y": ys}


def test_stack_step_addends_and_calls(monkeypatch):
    """The timed step: addends a_l = xs[l] - y_{l-1}(xs[l-1]) per logit set,
    entry 0 zero; each step is one moe_decode_stack call over every layer
    with its own logit and addend set, writing only the last layer's y."""
    import torch
    import synth
    monkeypatch.setattr(torch.cuda, "synchronize", lambda: None)
    fake = _FakeBinding()
    shape = synth.LayerShape(8, 2, 64, 32, True)
    n = 5
    pools = [(torch.zeros((9, 1), dtype=torch.uint8), torch.zeros(8, dtype=torch.int32), 8, l)
             for l in range(n)]        # the layer number stands in the format field
    xs = [torch.full((1, 64), float(l + 1)) for l in range(n)]
    sets = [torch.zeros((n, 1, 8)) + g for g in range(2)]
    step = bench.StackStep(torch, fake, shape, pools, 1, "cpu", xs[0], sets)
    step.set_addends(xs)
    assert len(step.add_sets) == 2
    for adds in step.add_sets:
        assert adds.shape == (n, 1, 64)
        assert torch.equal(adds[0], torch.zeros((1, 64)))
        for l in range(1, n):
            assert torch.equal(adds[l], xs[l] - (2 * xs[l - 1] + (l - 1)))
    for g in range(2):
        step.step(g)
        layers, x, logits, tables, addends, ys, ws, routing = fake.calls[-1]
        assert len(layers) == n and x is xs[0] and logits is sets[g]
        assert addends is step.add_sets[g] and ys is step.y and ys.shape == (1, 64)
        assert ws is step.ws and not routing
