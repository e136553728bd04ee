"""The layer under HIP graph capture.

Every entry point only launches kernels on the caller's stream: no
allocation, no memset, no copy and no host read of device data, so a whole
step can be captured once and replayed.  These tests capture the forward
(moe_forward) and the training step (moe_forward_train + moe_backward),
replay each graph several times with eager work and synchronisations in
between, change the inputs in place between replays, and require every
replay to equal an eager call on the same inputs bit for bit (every kernel
sums in a fixed order, so the two runs perform the same arithmetic).
Eager parity with the oracle is covered by the other GPU tests.
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_logit_amd as moe
import moe_inputs
from _gpu import dev, host, problem_of, torch_dtype

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

# outputs defined on their first offsets[E] rows only (the kept assignments)
KEPT_ROWS = {"src_token", "u", "h", "y_perm"}


def route_buffers(case):
    T, E, k = case.T, case.E, case.k
    return {"topk_idx": torch.empty(T, k, dtype=torch.int32, device="cuda"),
            "topk_w": torch.empty(T, k, dtype=torch.float32, device="cuda"),
            "counts": torch.empty(E, dtype=torch.int32, device="cuda"),
            "offsets": torch.empty(E + 1, dtype=torch.int32, device="cuda"),
            "slot": torch.empty(T, k, dtype=torch.int32, device="cuda"),
            "src_token": torch.empty(T * k, dtype=torch.int32, device="cuda")}


def second_inputs(case, inp):
    """The same weights with the tokens (and given logits) of another seed,
    for in-place updates of the captured buffers."""
    other = moe_inputs.make(case.with_(seed=case.seed + 7919), weights=False, bias_override=inp.get("bg"))
    out = dict(inp)
    out["x"] = other["x"]
    if case.logits == "given":
        out["logits"] = other["logits"]
    return out


def snapshot(bufs):
    torch.cuda.synchronize()
    return {n: host(t).copy() for n, t in bufs.items()}


def scribble(bufs):
    """Overwrite every output eagerly, so a replay that skipped a write shows."""
    for t in bufs.values():
        if t.dtype.is_floating_point:
            t.fill_(float("nan"))
        else:
            t.fill_(-3)


def assert_same(got, ref, what):
    P = int(ref["offsets"][-1])
    for n in ref:
        a, b = got[n], ref[n]
        assert a.shape == b.shape, f"{what}: {n} shape"
        if n in KEPT_ROWS:
            a, b = a[:P], b[:P]
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"{what}: {n} differs from eager"


class Forward:
    """Device buffers of one forward; inputs can be reloaded in place."""

    def __init__(self, case, inp):
        self.case, self.p = case, problem_of(case)
        T, d, E = case.T, case.d, case.E
        self.x, self.W1, self.W2 = dev(inp["x"]), dev(inp["W1"]), dev(inp["W2"])
        self.gate = case.logits == "gate"
        self.Wg = dev(inp["Wg"]) if self.gate else None
        self.bg = dev(inp["bg"]) if self.gate and inp["bg"] is not None else None
        self.logits = torch.empty(T, E, dtype=torch.float32, device="cuda") if self.gate else dev(inp["logits"])
        self.info = route_buffers(case)
        self.y = torch.empty(T, d, dtype=torch_dtype(case), device="cuda")
        self.ws = torch.empty(moe.moe_workspace_size(self.p), dtype=torch.uint8, device="cuda")

    def load(self, inp):
        self.x.copy_(dev(inp["x"]))
        if not self.gate:
            self.logits.copy_(dev(inp["logits"]))

    def outputs(self):
        out = dict(self.info)
        out["y"] = self.y
        if self.gate:
            out["logits"] = self.logits
        return out

    def run(self, stream):
        moe.moe_forward(self.p, self.x, self.Wg, self.bg, self.W1, self.W2, self.y, logits=self.logits,
                        info=self.info, ws=self.ws, stream=stream)


def capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # one eager call on the capture stream first
        fn(s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fn(s)
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("name", list(moe_inputs.SMALL))
def test_forward_graph_replay(name):
    case = moe_inputs.get(name)
    print(f"[graph forward] {name} T={case.T} d={case.d} E={case.E} k={case.k} F={case.F}", flush=True)
    inp_a = moe_inputs.make(case)
    inp_b = second_inputs(case, inp_a)

    # eager references on separate buffers
    refs = []
    for inp in (inp_a, inp_b):
        f = Forward(case, inp)
        f.run(torch.cuda.current_stream())
        refs.append(snapshot(f.outputs()))
        del f

    f = Forward(case, inp_a)
    g = capture(f.run)
    for rep, (inp, ref) in enumerate([(inp_a, refs[0]), (inp_b, refs[1]), (inp_a, refs[0])]):
        f.load(inp)
        scribble(f.outputs())
        torch.cuda.synchronize()
        g.replay()
        got = snapshot(f.outputs())
        assert_same(got, ref, f"replay {rep}")
        # eager work between replays: an unrelated kernel and a copy on the default stream
        torch.randn(1024, device="cuda").sum().item()


class TrainStep:
    """Buffers of moe_forward_train + moe_backward for one case."""

    def __init__(self, case, inp, losses):
        self.case, self.p, self.losses = case, problem_of(case), losses
        T, d, E, k, F = case.T, case.d, case.E, case.k, case.F
        n1 = 2 * F if case.act == "swiglu" else F
        dt = torch_dtype(case)
        self.f = Forward(case, inp)
        self.saved = {"u": torch.empty(T * k, n1, dtype=dt, device="cuda"),
                      "h": torch.empty(T * k, F, dtype=dt, device="cuda"),
                      "y_perm": torch.empty(T * k, d, dtype=dt, device="cuda")}
        self.dy = dev(moe_inputs.make_dy(case))
        self.grads = {"dx": torch.empty(T, d, dtype=dt, device="cuda"),
                      "dWg": torch.empty(E, d, dtype=torch.float32, device="cuda"),
                      "dbg": torch.empty(E, dtype=torch.float32, device="cuda"),
                      "dW1": torch.empty(E, n1, d, dtype=torch.float32, device="cuda"),
                      "dW2": torch.empty(E, d, F, dtype=torch.float32, device="cuda")}
        self.bws = torch.empty(moe.moe_backward_workspace_size(self.p), dtype=torch.uint8, device="cuda")

    def outputs(self):
        out = self.f.outputs()
        out.update(self.saved)
        out.update(self.grads)
        return out

    def run(self, stream):
        f, gr = self.f, self.grads
        moe.moe_forward_train(self.p, f.x, f.Wg, f.bg, f.W1, f.W2, f.y, f.logits, f.info, self.saved, f.ws,
                              stream=stream)
        moe.moe_backward(self.p, self.dy, f.x, f.Wg, f.W1, f.W2, f.logits, f.info, self.saved, gr["dx"],
                         gr["dWg"], gr["dbg"], gr["dW1"], gr["dW2"], self.bws, stream=stream,
                         aux_coef=self.losses[0], z_coef=self.losses[1])


TRAIN = [("mixtral_s", (0.0, 0.0)), ("skywork_m_s", (0.01, 0.001)), ("tiny_fp32", (0.0, 0.0))]


@pytest.mark.parametrize("name,losses", TRAIN, ids=[n for n, _ in TRAIN])
def test_training_step_graph_replay(name, losses):
    case = moe_inputs.get(name)
    print(f"[graph train] {name} T={case.T} d={case.d} E={case.E} k={case.k} F={case.F} losses={losses}",
          flush=True)
    inp_a = moe_inputs.make(case)
    inp_b = second_inputs(case, inp_a)
    refs = []
    for inp in (inp_a, inp_b):
        t = TrainStep(case, inp, losses)
        t.run(torch.cuda.current_stream())
        refs.append(snapshot(t.outputs()))
        del t

    t = TrainStep(case, inp_a, losses)
    g = capture(t.run)
    for rep, (inp, ref) in enumerate([(inp_a, refs[0]), (inp_b, refs[1]), (inp_b, refs[1])]):
        t.f.load(inp)
        scribble(t.outputs())
        torch.cuda.synchronize()
        g.replay()
        got = snapshot(t.outputs())
        assert_same(got, ref, f"replay {rep}")
        torch.randn(1024, device="cuda").sum().item()
