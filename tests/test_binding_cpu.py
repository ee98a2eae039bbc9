"""CPU tests of the Python binding's argument checks (they run before any device call)."""
import pytest
import torch

import selective_state_space_57_amd as ssm


def _args(b=2, D=3, L=5, N=4, dt=torch.bfloat16):
    return dict(x=torch.zeros(b, D, L, dtype=dt), dt=torch.zeros(b, D, L, dtype=dt), A=torch.zeros(D, N),
                B=torch.zeros(b, N, L, dtype=dt), C=torch.zeros(b, N, L, dtype=dt))


def test_y_dtype_follows_given_output():
    a = _args()
    with pytest.raises(TypeError, match="does not match"):
        ssm.scan_fwd(**a, y=torch.zeros(2, 3, 5), y_dtype=torch.bfloat16)


@pytest.mark.parametrize("key,bad", [("dt", torch.zeros(2, 3, 6, dtype=torch.bfloat16)),
                                     ("B", torch.zeros(2, 5, 5, dtype=torch.bfloat16)),
                                     ("A", torch.zeros(3, 4, dtype=torch.float64)),
                                     ("C", torch.zeros(2, 4, 5))])
def test_shape_and_dtype_checks(key, bad):
    a = _args()
    a[key] = bad
    with pytest.raises((ValueError, TypeError)):
        ssm.scan_fwd(**a)


def test_non_contiguous_rejected():
    a = _args()
    a["x"] = torch.zeros(2, 5, 3, dtype=torch.bfloat16).transpose(1, 2)
    with pytest.raises(ValueError, match="contiguous"):
        ssm.scan_fwd(**a)


def test_unsupported_dtype():
    a = _args(dt=torch.float16)
    with pytest.raises(TypeError):
        ssm.scan_fwd(**a)
