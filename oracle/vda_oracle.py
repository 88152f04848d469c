"""Plain float64 CPU oracle for the Video Delta Attention (VDA) forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or run
this module: only the tests, the smoke check and the benchmark's CPU-baseline
leg use it, to decide whether the GPU library is right and to time a baseline.
It shares no code with the GPU library.

What it computes (sources: the VDN-MiniMax-H3 pages -- the aiezz page, section 03
"technical principles", bullets "Video Delta Attention" and "dual text injection";
the laicaila page, section "technical principles", the same two bullets; the
comfyui-wiki page, section "how Video DeltaNet speeds up H3"; the model card's
introduction, bullet "hybrid architecture"):

* The linear branch keeps a recurrent state per head.  Per frame, all spatial
  tokens of that frame update the state together through the normal equations of
  a least-squares problem -- the frame-wise form of the token-wise delta rule.
  The pages give no formula.  The reading taken here is the regularised
  frame-level least squares

      X_f = argmin_X ||K_f X - V_f||_F^2 + lam ||X - X_prev||_F^2
          = (lam I + K_f^T K_f)^{-1} (lam X_prev + K_f^T V_f),

  with the state stored as X = S^T (d x dv), keys K_f (n x d), values V_f (n x dv).
* The text is written once into the state, at initialisation: the same update
  applied to a zero state with all T text tokens as one "frame".
* The state is bidirectional: a forward scan over frames 1..F and a backward scan
  over F..1, both starting from the text state.
* Each frame reads the state out with its queries.  Reading: inclusive states
  (after frame f's own update) and the mean of the two directions,
  O_f = Q_f (X_fwd_f + X_bwd_f) / 2.
* No feature map, no 1/sqrt(d) scaling, no decay and no gate inside the op.  The
  branch's gated fusion epilogue, applied to the op's output, is at the end of this
  module.

Every function works on float64 arrays and uses library linear algebra
(``numpy.linalg.solve``) for the solves, with no blocking or reordering beyond
the definition above.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "frame_statistics", "normal_equation_update", "text_state", "scan_from",
    "head_states", "readout", "vda_forward_head", "vda_forward",
    "gated_output", "vda_forward_gated_head", "vda_forward_gated",
    "vda_backward_head", "vda_backward",
]


def frame_statistics(K_f: np.ndarray, V_f: np.ndarray):
    """Normal-equation statistics of one frame: G = K_f^T K_f (d x d), B = K_f^T V_f (d x dv).
    All tokens of the frame enter together (the frame-wise joint solve of the
    "Video Delta Attention" bullet)."""
    K_f = np.asarray(K_f, dtype=np.float64)
    V_f = np.asarray(V_f, dtype=np.float64)
    return K_f.T @ K_f, K_f.T @ V_f


def normal_equation_update(X_prev: np.ndarray, K_f: np.ndarray, V_f: np.ndarray, lam: float):
    """One frame of the state update: solve (lam I + K_f^T K_f) X = lam X_prev + K_f^T V_f."""
    if not lam > 0:
        raise ValueError("lam must be > 0")
    G, Bm = frame_statistics(K_f, V_f)
    d = G.shape[0]
    A = lam * np.eye(d) + G
    R = lam * np.asarray(X_prev, dtype=np.float64) + Bm
    return np.linalg.solve(A, R)


def text_state(text_k: np.ndarray, text_v: np.ndarray, lam: float, d: int, dv: int):
    """The text written once into the state: the update applied to a zero state, with
    all text tokens as one frame ("dual text injection" bullet).  T = 0 gives zero."""
    text_k = np.asarray(text_k, dtype=np.float64).reshape(-1, d)
    text_v = np.asarray(text_v, dtype=np.float64).reshape(-1, dv)
    return normal_equation_update(np.zeros((d, dv)), text_k, text_v, lam)


def scan_from(X0: np.ndarray, K: np.ndarray, V: np.ndarray, lam: float):
    """Run the recurrence over frames in the order given.  K: [F,n,d], V: [F,n,dv].
    Returns the inclusive states [F,d,dv]: entry i is the state after frame i."""
    X = np.asarray(X0, dtype=np.float64)
    out = np.empty((K.shape[0],) + X.shape)
    for i in range(K.shape[0]):
        X = normal_equation_update(X, K[i], V[i], lam)
        out[i] = X
    return out


def head_states(k, v, text_k, text_v, lam):
    """Text state and both directional state sequences of one head.
    Returns (X_text [d,dv], X_fwd [F,d,dv], X_bwd [F,d,dv]); X_bwd[f] is the backward
    state after frame f (the backward scan runs f = F-1 .. 0)."""
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    d, dv = k.shape[-1], v.shape[-1]
    X_text = text_state(text_k, text_v, lam, d, dv)
    X_fwd = scan_from(X_text, k, v, lam)
    X_bwd = scan_from(X_text, k[::-1], v[::-1], lam)[::-1]
    return X_text, X_fwd, X_bwd


def readout(q, X_fwd, X_bwd):
    """O_f = Q_f (X_fwd_f + X_bwd_f) / 2 for every frame.  q: [F,n,d] -> [F,n,dv]."""
    q = np.asarray(q, dtype=np.float64)
    W = 0.5 * (X_fwd + X_bwd)
    return np.stack([q[f] @ W[f] for f in range(q.shape[0])]) if q.shape[0] else \
        np.zeros((0, q.shape[1], X_fwd.shape[-1]))


def vda_forward_head(q, k, v, text_k, text_v, lam):
    """VDA forward for one (batch, head): q,k [F,n,d], v [F,n,dv], text_k [T,d], text_v [T,dv]."""
    _, X_fwd, X_bwd = head_states(k, v, text_k, text_v, lam)
    return readout(q, X_fwd, X_bwd)


def vda_forward(q, k, v, text_k, text_v, lam):
    """VDA forward over [B,H,...] arrays; heads and batch entries are independent.
    Returns out [B,H,F,n,dv] in float64."""
    q = np.asarray(q, dtype=np.float64)
    Bsz, H = q.shape[:2]
    out = np.empty(q.shape[:-1] + (np.asarray(v).shape[-1],))
    for b in range(Bsz):
        for h in range(H):
            out[b, h] = vda_forward_head(q[b, h], k[b, h], v[b, h], text_k[b, h], text_v[b, h], lam)
    return out


# ---------------------------------------------------------------------------
# Gated fusion epilogue of the linear branch
# ---------------------------------------------------------------------------
# The pages (aiezz page, section 03, bullet "gated fusion"; laicaila page, section
# "technical principles", the same bullet) say the two attention branches have
# different output scales, so each branch gets a content-dependent sigmoid gate and
# an output projection of its own before the branches are merged.  For the linear
# branch alone this reads, per head and per token, with the branch output O (1 x dv)
# as the content the gate depends on:
#     Y = sigmoid(O W_g^T + b_g) * (O W_o^T)            (elementwise product)
# with W_g, W_o (dv x dv) stored as [output feature][input feature] and b_g (dv).
# Merging with the softmax branch is not part of this op.

def gated_output(O_rows, w_gate, b_gate, w_out):
    """Y = sigmoid(O W_g^T + b_g) * (O W_o^T) for rows O [..., dv]; w_gate, w_out [dv, dv]
    ([output][input]), b_gate [dv]."""
    O_rows = np.asarray(O_rows, dtype=np.float64)
    w_gate = np.asarray(w_gate, dtype=np.float64)
    w_out = np.asarray(w_out, dtype=np.float64)
    b_gate = np.asarray(b_gate, dtype=np.float64)
    g = O_rows @ w_gate.T + b_gate
    with np.errstate(over="ignore"):
        gate = 1.0 / (1.0 + np.exp(-g))
    return gate * (O_rows @ w_out.T)


def vda_forward_gated_head(q, k, v, text_k, text_v, lam, w_gate, b_gate, w_out):
    """The VDA output of one (batch, head) followed by the gated epilogue with that head's
    weights: w_gate, w_out [dv, dv], b_gate [dv]."""
    return gated_output(vda_forward_head(q, k, v, text_k, text_v, lam), w_gate, b_gate, w_out)


def vda_forward_gated(q, k, v, text_k, text_v, lam, w_gate, b_gate, w_out):
    """Gated VDA forward over [B,H,...] arrays with per-head weights w_gate, w_out [H, dv, dv]
    and b_gate [H, dv], shared by every batch entry."""
    out = vda_forward(q, k, v, text_k, text_v, lam)
    for h in range(out.shape[1]):
        out[:, h] = gated_output(out[:, h], w_gate[h], b_gate[h], w_out[h])
    return out


# ---------------------------------------------------------------------------
# Backward pass (gradients) of the forward op
# ---------------------------------------------------------------------------
# The pages train the branch (aiezz page, section 03, bullet "three-stage training
# adaptation"; laicaila page, the same bullet): layer-wise alignment of the linear
# branch, then end-to-end optimisation, then LoRA with the branch.  Training needs the
# gradient of the op.  Given dO = dL/dO for every frame, the chain rule through the
# definition above gives (A_f = lam I + K_f^T K_f, B_f = K_f^T V_f, W_f the readout
# state, all A_f symmetric):
#   readout:       dQ_f = dO_f W_f^T,   dW_f = Q_f^T dO_f,  each direction gets dW_f / 2
#   forward chain: U_f = A_f^{-1} (dW_f / 2 + lam U_{f+1}),  f = F..1,  U_{F+1} = 0
#   backward chain: V_f = A_f^{-1} (dW_f / 2 + lam V_{f-1}), f = 1..F,  V_0 = 0
#   frames:        dB_f = U_f + V_f,   dA_f = -(U_f X_fwd_f^T + V_f X_bwd_f^T)
#   text:          U_0 = A_0^{-1} lam (U_1 + V_F),  dB_0 = U_0,  dA_0 = -U_0 X_text^T
#   statistics:    dK += V dB^T + K (dA + dA^T),   dV += K dB
# (X_f = A_f^{-1} R_f gives dR_f = A_f^{-1} Gamma_f and dA_f = -A_f^{-1} Gamma_f X_f^T.)
# Each step is written out below in that order with library solves.

def vda_backward_head(q, k, v, text_k, text_v, lam, d_out):
    """Gradients of sum(d_out * O) for one (batch, head).  q,k [F,n,d], v [F,n,dv],
    text_k [T,d], text_v [T,dv], d_out [F,n,dv].  Returns (dq, dk, dv, d_text_k, d_text_v)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    d_out = np.asarray(d_out, dtype=np.float64)
    d, dv = k.shape[-1], v.shape[-1]
    text_k = np.asarray(text_k, dtype=np.float64).reshape(-1, d)
    text_v = np.asarray(text_v, dtype=np.float64).reshape(-1, dv)
    F = k.shape[0]
    X_text, X_fwd, X_bwd = head_states(k, v, text_k, text_v, lam)
    A = [lam * np.eye(d) + frame_statistics(k[f], v[f])[0] for f in range(F)]
    W = 0.5 * (X_fwd + X_bwd)
    dq = np.stack([d_out[f] @ W[f].T for f in range(F)]) if F else np.zeros_like(q)
    half_dW = [0.5 * (q[f].T @ d_out[f]) for f in range(F)]
    U = [None] * (F + 2)
    U[F + 1] = np.zeros((d, dv))
    for f in range(F, 0, -1):                      # frames are 1-based in the chains
        U[f] = np.linalg.solve(A[f - 1], half_dW[f - 1] + lam * U[f + 1])
    V = [None] * (F + 1)
    V[0] = np.zeros((d, dv))
    for f in range(1, F + 1):
        V[f] = np.linalg.solve(A[f - 1], half_dW[f - 1] + lam * V[f - 1])
    dk = np.empty_like(k)
    dvv = np.empty_like(v)
    for f in range(1, F + 1):
        dB = U[f] + V[f]
        dA = -(U[f] @ X_fwd[f - 1].T + V[f] @ X_bwd[f - 1].T)
        dk[f - 1] = v[f - 1] @ dB.T + k[f - 1] @ (dA + dA.T)
        dvv[f - 1] = k[f - 1] @ dB
    A0 = lam * np.eye(d) + text_k.T @ text_k
    gamma_text = lam * (U[1] + V[F]) if F else np.zeros((d, dv))
    U0 = np.linalg.solve(A0, gamma_text)
    dA0 = -(U0 @ X_text.T)
    d_text_k = text_v @ U0.T + text_k @ (dA0 + dA0.T)
    d_text_v = text_k @ U0
    return dq, dk, dvv, d_text_k, d_text_v


def vda_backward(q, k, v, text_k, text_v, lam, d_out):
    """Gradients over [B,H,...] arrays (heads and batch entries are independent)."""
    q = np.asarray(q, dtype=np.float64)
    Bsz, H = q.shape[:2]
    grads = [np.empty(np.shape(a), dtype=np.float64) for a in (q, k, v, text_k, text_v)]
    for b in range(Bsz):
        for h in range(H):
            res = vda_backward_head(q[b, h], k[b, h], v[b, h], text_k[b, h], text_v[b, h], lam,
                                    d_out[b, h])
            for g, r in zip(grads, res):
                g[b, h] = r
    return tuple(grads)
