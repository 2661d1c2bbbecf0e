"""The binding's tensor checks (no GPU): the C ABI receives raw pointers only, so a wrong
dtype, shape, stride or device must be rejected in Python before any pointer is passed.
Each case below changes one tensor of an otherwise valid argument set."""
import pytest
import torch

from chunked_linear_recurrence_amd import ssd


def _layer(dtype=torch.bfloat16, b=2, L=300, H=4, P=16, N=32, G=2):
    return dict(x=torch.zeros(b, L, H, P, dtype=dtype), dt=torch.zeros(b, L, H, dtype=dtype),
                A=torch.zeros(H), B=torch.zeros(b, L, G, N, dtype=dtype),
                C=torch.zeros(b, L, G, N, dtype=dtype), D=torch.zeros(H),
                init_state=torch.zeros(b, H, P, N), y=torch.zeros(b, L, H, P, dtype=dtype),
                final_state=torch.zeros(b, H, P, N), workspace=torch.zeros(64, dtype=torch.uint8))


LAYER_BAD = {
    "A float64": ("A", lambda t: t.double(), "A has dtype"),
    "D float64": ("D", lambda t: t.double(), "D has dtype"),
    "dt float32 with bf16 x": ("dt", lambda t: t.float(), "dt has dtype"),
    "B float32 with bf16 x": ("B", lambda t: t.float(), "B has dtype"),
    "x float16": ("x", lambda t: t.half(), "x has dtype"),
    "x non-contiguous head slice": ("x", lambda t: torch.zeros(2, 300, 8, 16, dtype=t.dtype)[:, :, ::2],
                                    "x must be contiguous"),
    "C shape": ("C", lambda t: t[:, :-1].contiguous(), "C has shape"),
    "dt shape": ("dt", lambda t: t[:, :, :-1].contiguous(), "dt has shape"),
    "A shape": ("A", lambda t: torch.zeros(5), "A has shape"),
    "init bf16": ("init_state", lambda t: t.bfloat16(), "init_state has dtype"),
    "init shape": ("init_state", lambda t: t[:, :, :, :-1].contiguous(), "init_state has shape"),
    "final transposed": ("final_state", lambda t: t.transpose(2, 3), "final_state has shape"),
    "y shape": ("y", lambda t: t[:1].contiguous(), "y has shape"),
    "workspace float": ("workspace", lambda t: t.float(), "workspace has dtype"),
}


@pytest.mark.parametrize("case", sorted(LAYER_BAD))
def test_layer_rejections(case):
    name, change, msg = LAYER_BAD[case]
    args = _layer()
    args[name] = change(args[name])
    with pytest.raises(ValueError, match=msg):
        ssd.check_layer_args(**args)


def test_valid_layer_on_cpu_is_rejected_for_its_device():
    with pytest.raises(ValueError, match="CUDA device"):
        ssd.check_layer_args(**_layer())
    with pytest.raises(ValueError, match="CUDA device"):
        ssd.check_layer_args(**_layer(dtype=torch.float32))
    args = _layer()
    with pytest.raises(ValueError, match="CUDA device"):
        ssd.fwd(args["x"], args["dt"], args["A"], args["B"], args["C"], args["D"], args["init_state"], 64)


def test_optional_tensors_may_be_none():
    args = _layer()
    for k in ("D", "init_state", "y", "final_state", "workspace"):
        args[k] = None
    with pytest.raises(ValueError, match="CUDA device"):     # everything else is valid
        ssd.check_layer_args(**args)


def _stack(nl=3, b=1, L=200, H=2, P=16, N=32, G=1, dtype=torch.bfloat16):
    return dict(x0=torch.zeros(b, L, H, P, dtype=dtype), dt=torch.zeros(b, L, H, dtype=dtype),
                A=torch.zeros(nl, H), B=torch.zeros(b, L, G, N, dtype=dtype),
                C=torch.zeros(b, L, G, N, dtype=dtype), D=torch.zeros(nl, H),
                layer_states=torch.zeros(nl, b, H, P, N))


@pytest.mark.parametrize("name,change,msg", [
    ("A", lambda t: t[0].contiguous(), "A has shape"),
    ("D", lambda t: t[:2].contiguous(), "D has shape"),
    ("layer_states", lambda t: t[:2].contiguous(), "layer_states has shape"),
    ("layer_states", lambda t: t.double(), "layer_states has dtype"),
    ("dt", lambda t: t.float(), "dt has dtype"),
])
def test_stack_rejections(name, change, msg):
    args = _stack()
    args[name] = change(args[name])
    with pytest.raises(ValueError, match=msg):
        ssd.check_stack_args(**args)
    with pytest.raises(ValueError, match=msg):
        ssd.segmented(args["x0"], args["dt"], args["A"], args["B"], args["C"], args["D"],
                      args["layer_states"], 64, 64)


@pytest.mark.parametrize("name,change,msg", [
    ("state", lambda t: t.bfloat16(), "state has dtype"),
    ("dt", lambda t: t[:, :1].contiguous(), "dt has shape"),
    ("B", lambda t: t.float(), "B has dtype"),
    ("x", lambda t: torch.zeros(2, 4, 32, dtype=t.dtype)[:, :, ::2], "x must be contiguous"),
])
def test_step_rejections(name, change, msg):
    b, H, P, N = 2, 4, 16, 32
    args = dict(x=torch.zeros(b, H, P, dtype=torch.bfloat16), dt=torch.zeros(b, H, dtype=torch.bfloat16),
                A=torch.zeros(H), B=torch.zeros(b, 1, N, dtype=torch.bfloat16),
                C=torch.zeros(b, 1, N, dtype=torch.bfloat16), D=torch.zeros(H), state=torch.zeros(b, H, P, N))
    args[name] = change(args[name])
    with pytest.raises(ValueError, match=msg):
        ssd.check_step_args(**args)
