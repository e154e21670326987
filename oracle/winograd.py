"""fp64 Winograd F(2x2, 3x3) for stride-1 3x3 conv2d -- TEST INFRASTRUCTURE ONLY.

The tensorcore "Conv2D" page ("What's not done in v0.1") names a Winograd
path for 3x3 stride-1 layers as a later priority and expects it to be about
twice as fast.  F(2x2, 3x3) is Lavin and Gray's minimal filtering algorithm
("Fast Algorithms for Convolutional Neural Networks", 2016): each 2x2 block
of outputs is computed from a 4x4 input tile d and a 3x3 filter g as

    Y = A^T [ (G g G^T) (.) (B^T d B) ] A

where (.) is the elementwise product and the sum over input channels is
taken on the 4x4 transformed values.  The matrices are the published ones:

    B^T = [[1, 0,-1, 0], [0, 1, 1, 0], [0,-1, 1, 0], [0, 1, 0,-1]]
    G   = [[1, 0, 0], [1/2, 1/2, 1/2], [1/2,-1/2, 1/2], [0, 0, 1]]
    A^T = [[1, 1, 1, 0], [0, 1,-1,-1]]

This module follows those steps in fp64 with numpy einsum as the only
primitive, so the algorithm can be checked against the direct definition
(the oracle's ``fprop``): the two agree to rounding for any input.  It also
gives, per output, the sum of the absolute values of every term the
algorithm adds, S = sum |A^T_ya A^T_xb| |U| |V| over the 16 transformed
points and the input channels, which bounds the error that rounding the
transformed operands to a 16-bit type introduces (see ``error_bound``).

Only stride 1, dilation 1, 3x3, groups 1.  Tensors are float64 numpy arrays
x [N,H,W,C], w [K,3,3,C], y [N,P,Q,K].
"""
import numpy as np

BT = np.array([[1, 0, -1, 0], [0, 1, 1, 0], [0, -1, 1, 0], [0, 1, 0, -1]], dtype=np.float64)
G = np.array([[1, 0, 0], [0.5, 0.5, 0.5], [0.5, -0.5, 0.5], [0, 0, 1]], dtype=np.float64)
AT = np.array([[1, 1, 1, 0], [0, 1, -1, -1]], dtype=np.float64)


def _check_prob(prob):
    if not (prob["R"] == 3 and prob["S"] == 3 and prob["stride_h"] == 1 and prob["stride_w"] == 1
            and prob["dil_h"] == 1 and prob["dil_w"] == 1 and prob["groups"] == 1):
        raise ValueError("Winograd F(2x2,3x3) covers stride-1, dilation-1, 3x3, groups-1 problems only")
    P = prob["H"] + 2 * prob["pad_h"] - 2
    Q = prob["W"] + 2 * prob["pad_w"] - 2
    if P < 1 or Q < 1:
        raise ValueError("empty output")
    return P, Q


def _tiles(prob, x):
    """Input tiles d[n, tp, tq, i, j, c]: the 4x4 input window of the 2x2
    output block (2tp.., 2tq..), zeros outside the image."""
    P, Q = _check_prob(prob)
    N, H, W, C = x.shape
    TP, TQ = (P + 1) // 2, (Q + 1) // 2
    ph, pw = prob["pad_h"], prob["pad_w"]
    xp = np.zeros((N, 2 * TP + 2, 2 * TQ + 2, C), dtype=np.float64)
    h1, w1 = min(H, 2 * TP + 2 - ph), min(W, 2 * TQ + 2 - pw)
    xp[:, ph:ph + h1, pw:pw + w1, :] = x[:, :h1, :w1, :]
    d = np.empty((N, TP, TQ, 4, 4, C), dtype=np.float64)
    for i in range(4):
        for j in range(4):
            d[:, :, :, i, j, :] = xp[:, i:i + 2 * TP:2, j:j + 2 * TQ:2, :]
    return d, P, Q


def transforms(prob, x, w):
    """U[k, a, b, c] = (G g_kc G^T)[a, b] and V[n, tp, tq, a, b, c] = (B^T d B)[a, b]."""
    d, P, Q = _tiles(prob, x)
    U = np.einsum("ar,krsc,bs->kabc", G, np.asarray(w, dtype=np.float64), G)
    V = np.einsum("ai,ntqijc,bj->ntqabc", BT, d, BT)
    return U, V, P, Q


def fprop(prob, x, w, bias=None, relu=False):
    """y = A^T [sum_c U (.) V] A per 2x2 block, then bias and ReLU (no rounding)."""
    U, V, P, Q = transforms(prob, x, w)
    M = np.einsum("kabc,ntqabc->ntqabk", U, V)
    Yb = np.einsum("ya,ntqabk,xb->ntqyxk", AT, M, AT)
    N, TP, TQ = Yb.shape[:3]
    y = Yb.transpose(0, 1, 3, 2, 4, 5).reshape(N, 2 * TP, 2 * TQ, -1)[:, :P, :Q, :]
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)
    if relu:
        y = np.maximum(y, 0.0)
    return y


def abs_terms(prob, x, w):
    """S[n, p, q, k]: the sum over the 16 transformed points and the input
    channels of |A^T_ya A^T_xb| |U| |V| for output (p, q) = (2tp+y, 2tq+x)."""
    U, V, P, Q = transforms(prob, x, w)
    Ma = np.einsum("kabc,ntqabc->ntqabk", np.abs(U), np.abs(V))
    Sb = np.einsum("ya,ntqabk,xb->ntqyxk", np.abs(AT), Ma, np.abs(AT))
    N, TP, TQ = Sb.shape[:3]
    return Sb.transpose(0, 1, 3, 2, 4, 5).reshape(N, 2 * TP, 2 * TQ, -1)[:, :P, :Q, :]


def error_bound(prob, x, w, u_op, u_acc=2.0 ** -24):
    """Per-output bound on |y_winograd - y| when U and V are each rounded
    once to a type of unit roundoff u_op and everything else runs in a type
    of unit roundoff u_acc (fp32): each term U*V then carries a relative
    error of at most 2 u_op + u_op^2, and the fp32 transforms and sums (at
    most 4 + 9 + 2C + 9 additions on any path) add at most (2C + 40) u_acc
    of S (first order, with a 1% margin on the whole)."""
    C = x.shape[-1]
    return 1.01 * ((2 * u_op + u_op * u_op) + (2 * C + 40) * u_acc) * abs_terms(prob, x, w)
