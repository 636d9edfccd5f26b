"""Pins for the oracle's forward and backward of the QLoRA linear (CPU only).

* A hand-computed 1x2 example fixes the equation's terms and the alpha/r
  factor (llm-compass "QLoRA", 方法与公式).
* X = I reads the operand layout back: Y = W^T + s (B A)^T.
* The backward is pinned to the forward by exact directional derivatives
  (the loss <dY, Y> is linear in A, in B and in X) and by fp64 torch autograd.
* Only the adapters receive gradients: B = 0 removes the adapter term and
  makes dA zero; A = 0 makes dB zero.
* The SiLU glue is pinned to torch.nn.functional.silu and its autograd.
"""
import numpy as np
import pytest

import oracle


def _case(seed=0, M=7, K=12, N=5, r=3):
    g = np.random.default_rng(seed)
    return (g.standard_normal((M, K)), g.standard_normal((N, K)),
            g.standard_normal((r, K)), g.standard_normal((N, r)),
            g.standard_normal((M, N)))


def test_scale_from_pages():
    assert oracle.lora_scale(32, 16) == 2.0       # r=16, alpha=32 on every page listing
    assert oracle.lora_scale(16, 8) == 2.0
    assert oracle.lora_scale(3, 7) == float(np.float32(3) / np.float32(7))


def test_forward_hand_example():
    X = np.array([[1.0, 2.0]])
    W = np.array([[3.0, -1.0]])           # N=1, K=2
    A = np.array([[0.5, 0.25]])           # r=1
    B = np.array([[4.0]])
    Y, T = oracle.forward(X, W, A, B, alpha=2.0, r=1)    # s = 2
    # base: 3 - 2 = 1 ; lora: A x = 1.0, B (A x) = 4, times s = 8 -> 9
    assert T.tolist() == [[1.0]] and Y.tolist() == [[9.0]]


def test_forward_identity_reads_layout():
    _, W, A, B, _ = _case(M=12, K=12)
    Y, _ = oracle.forward(np.eye(12), W, A, B, alpha=6.0, r=3)
    assert np.allclose(Y, W.T + 2.0 * (B @ A).T, rtol=0, atol=1e-12)


def test_directional_derivatives_are_exact():
    X, W, A, B, dY = _case(1)
    alpha, r = 5.0, 3
    dX, dA, dB = oracle.backward(dY, X, W, A, B, alpha, r)
    L = lambda X_, A_, B_: float(np.sum(dY * oracle.forward(X_, W, A_, B_, alpha, r)[0]))
    g = np.random.default_rng(9)
    for _ in range(3):
        E = g.standard_normal(A.shape)
        assert abs(L(X, A + E, B) - L(X, A, B) - np.sum(dA * E)) < 1e-9
        E = g.standard_normal(B.shape)
        assert abs(L(X, A, B + E) - L(X, A, B) - np.sum(dB * E)) < 1e-9
        E = g.standard_normal(X.shape)
        # L is quadratic in X only through nothing: it is linear in X as well
        assert abs(L(X + E, A, B) - L(X, A, B) - np.sum(dX * E)) < 1e-9


def test_backward_matches_torch_autograd():
    torch = pytest.importorskip("torch")
    X, W, A, B, dY = _case(2, M=9, K=16, N=11, r=4)
    alpha, r = 8.0, 4
    dX, dA, dB = oracle.backward(dY, X, W, A, B, alpha, r)
    tX = torch.tensor(X, requires_grad=True)
    tA = torch.tensor(A, requires_grad=True)
    tB = torch.tensor(B, requires_grad=True)
    tW = torch.tensor(W)
    Y = torch.nn.functional.linear(tX, tW) + (alpha / r) * torch.nn.functional.linear(
        torch.nn.functional.linear(tX, tA), tB)
    Y.backward(torch.tensor(dY))
    assert np.allclose(dX, tX.grad.numpy(), atol=1e-12)
    assert np.allclose(dA, tA.grad.numpy(), atol=1e-12)
    assert np.allclose(dB, tB.grad.numpy(), atol=1e-12)
    Yo, _ = oracle.forward(X, W, A, B, alpha, r)
    assert np.allclose(Yo, Y.detach().numpy(), atol=1e-12)


def test_adapter_only_special_cases():
    X, W, A, B, dY = _case(3)
    Y0, _ = oracle.forward(X, W, A, np.zeros_like(B), 4.0, 3)
    assert np.allclose(Y0, X @ W.T, atol=1e-12)
    _, dA, _ = oracle.backward(dY, X, W, A, np.zeros_like(B), 4.0, 3)
    assert np.all(dA == 0)
    _, _, dB = oracle.backward(dY, X, W, np.zeros_like(A), B, 4.0, 3)
    assert np.all(dB == 0)


def test_one_hot_grad_reads_a_weight_row():
    X, W, A, B, _ = _case(4)
    dY = np.zeros((X.shape[0], W.shape[0]))
    dY[2, 4] = 1.0
    dX, _, _ = oracle.backward(dY, X, W, A, B, 6.0, 3)
    assert np.allclose(dX[2], W[4] + 2.0 * B[4] @ A, atol=1e-12)
    assert np.all(dX[[0, 1, 3, 4, 5, 6]] == 0)


def test_silu_glue_against_torch():
    torch = pytest.importorskip("torch")
    g = np.random.default_rng(6)
    G, U, dH = (g.standard_normal((5, 33)) * 3 for _ in range(3))
    H = oracle.silu_mul_forward(G, U)
    tG = torch.tensor(G, requires_grad=True)
    tU = torch.tensor(U, requires_grad=True)
    tH = torch.nn.functional.silu(tG) * tU
    assert np.allclose(H, tH.detach().numpy(), atol=1e-12)
    tH.backward(torch.tensor(dH))
    dG, dU = oracle.silu_mul_backward(dH, G, U)
    assert np.allclose(dG, tG.grad.numpy(), atol=1e-12)
    assert np.allclose(dU, tU.grad.numpy(), atol=1e-12)


def test_mlp_backward_against_torch():
    torch = pytest.importorskip("torch")
    g = np.random.default_rng(8)
    M, K, F = 6, 10, 14
    mk = lambda N, Kin, r: dict(W_hat=g.standard_normal((N, Kin)), A=g.standard_normal((r, Kin)),
                                B=g.standard_normal((N, r)), alpha=4.0, r=2)
    gate, up, down = mk(F, K, 2), mk(F, K, 2), mk(K, F, 2)
    X, dY = g.standard_normal((M, K)), g.standard_normal((M, K))
    Y, saved = oracle.mlp_forward(X, gate, up, down)
    dX, grads = oracle.mlp_backward(dY, X, saved, gate, up, down)
    t = {k: {n: torch.tensor(v, requires_grad=(n in "AB")) if isinstance(v, np.ndarray) else v
             for n, v in d.items()} for k, d in dict(gate=gate, up=up, down=down).items()}
    tX = torch.tensor(X, requires_grad=True)
    lin = lambda x, p: x @ p["W_hat"].T + 2.0 * (x @ p["A"].T) @ p["B"].T
    tY = lin(torch.nn.functional.silu(lin(tX, t["gate"])) * lin(tX, t["up"]), t["down"])
    tY.backward(torch.tensor(dY))
    assert np.allclose(Y, tY.detach().numpy(), atol=1e-10)
    assert np.allclose(dX, tX.grad.numpy(), atol=1e-10)
    for k in ("gate", "up", "down"):
        assert np.allclose(grads[k][0], t[k]["A"].grad.numpy(), atol=1e-10)
        assert np.allclose(grads[k][1], t[k]["B"].grad.numpy(), atol=1e-10)
