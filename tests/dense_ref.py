"""Dense brute-force mass matrix for tiny periodic grids (numpy).

Independent of ``oracle/``: it never finds a "first support node". It
evaluates the 1D B-spline at the wrapped distance from the particle to every
node, builds the dense interpolation matrix W [np, nnodes] and forms
M^{ij} = W^T diag(sigma * w * alpha^{ij}) W (the tensor-contraction form of
Pennati & Markidis, Sec. 2.2 / Sec. 3.1 Eq. 14). alpha is obtained as the
matrix inverse of (I + beta [B]x), [B]x u = B x u, via numpy.
"""
import numpy as np


def bspline(order: int, t: np.ndarray) -> np.ndarray:
    a = np.abs(t)
    if order == 1:
        return np.where(a < 1.0, 1.0 - a, 0.0)
    if order == 2:
        inner = 0.75 - a * a
        outer = 0.5 * (1.5 - a) ** 2
        return np.where(a <= 0.5, inner, np.where(a < 1.5, outer, 0.0))
    raise ValueError(order)


def dense_W(order, n, origin, h, pos):
    n = np.asarray(n)
    pos = np.asarray(pos, dtype=np.float64).reshape(-1, 3)
    Wd = []
    for d in range(3):
        if d == 2 and n[2] == 1:  # 2D: one node plane, weight 1
            Wd.append(np.ones((pos.shape[0], 1)))
            continue
        u = (pos[:, d] - origin[d]) / h[d]
        nodes = np.arange(n[d], dtype=np.float64)
        t = u[:, None] - nodes[None, :]
        t = t - n[d] * np.floor(t / n[d] + 0.5)  # minimum image in [-n/2, n/2)
        Wd.append(bspline(order, t))
    W = (Wd[0][:, None, None, :] * Wd[1][:, None, :, None]) * Wd[2][:, :, None, None]
    return W.reshape(pos.shape[0], -1)  # node index = x + nx*(y + ny*z)


def alpha_inv(B, beta):
    B = np.asarray(B, dtype=np.float64)
    cross = np.array([np.cross(B, e) for e in np.eye(3)]).T  # cross @ u = B x u
    return np.linalg.inv(np.eye(3) + beta * cross)


def dense_M(order, n, origin, h, pos, w, B=None, beta=0.0, sigma=1.0):
    """Dense [ncomp, nnodes, nnodes] mass matrices."""
    W = dense_W(order, n, origin, h, pos)
    w = np.asarray(w, dtype=np.float64)
    if B is None:
        S = (sigma * w)[:, None]
    else:
        S = np.stack([(sigma * w[p]) * alpha_inv(B[p], beta).reshape(-1) for p in range(len(w))])
    return np.einsum("pg,pc,ph->cgh", W, S, W)


def dense_to_stencil(order, n, Md):
    R = order
    NO = 2 * R + 1
    nx, ny, nz = n
    ncomp = Md.shape[0]
    nn = nx * ny * nz
    RZ = 0 if nz == 1 else R  # 2D grids: no z offsets
    out = np.zeros((nn, NO * NO * (2 * RZ + 1), ncomp))
    g = np.arange(nn)
    gx, gy, gz = g % nx, (g // nx) % ny, g // (nx * ny)
    for oz in range(-RZ, RZ + 1):
        for oy in range(-R, R + 1):
            for ox in range(-R, R + 1):
                o = (ox + R) + NO * ((oy + R) + NO * (oz + RZ))
                g2 = ((gx + ox) % nx) + nx * (((gy + oy) % ny) + ny * ((gz + oz) % nz))
                out[:, o, :] = Md[:, g, g2].T
    return out


def stencil_bilinear(order, n, M, u, v):
    """sum_{g,o,i,j} u[g,i] M[g,o,(i,j)] v[g+o, j] (tensorial) or scalar analogue."""
    R = order
    NO = 2 * R + 1
    nx, ny, nz = n
    nn = nx * ny * nz
    g = np.arange(nn)
    gx, gy, gz = g % nx, (g // nx) % ny, g // (nx * ny)
    ncomp = M.shape[2]
    RZ = 0 if nz == 1 else R  # 2D grids: no z offsets
    total = 0.0
    for oz in range(-RZ, RZ + 1):
        for oy in range(-R, R + 1):
            for ox in range(-R, R + 1):
                o = (ox + R) + NO * ((oy + R) + NO * (oz + RZ))
                g2 = ((gx + ox) % nx) + nx * (((gy + oy) % ny) + ny * ((gz + oz) % nz))
                if ncomp == 1:
                    total += float(np.sum(u * M[:, o, 0] * v[g2]))
                else:
                    blk = M[:, o, :].reshape(nn, 3, 3)
                    total += float(np.einsum("gi,gij,gj->", u, blk, v[g2]))
    return total
