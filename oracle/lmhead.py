"""Float64 lm_head backward (the step upstream of the layer stack).  TEST
INFRASTRUCTURE ONLY.

The entrenar trainer backpropagates "from lm_head through all FFN layers"
([ENT] wgpu_backward.rs, module doc; backward_through_layers takes the
grad_hidden "from lm_head backward") and keeps the lm_head weight with AdamW
moments (WgpuModelState lm_head, lm_head_m, lm_head_v: [vocab, hidden], in
its gradient-flow test).  The pages give no formula for that step; the plain
reading, used here and by the library:

  logits = h W^T                  h [S, hidden] the final hidden state,
                                  W [vocab, hidden] the lm_head weight
  loss   = (1/n) sum_s CE(logits_s, label_s),  CE(z, y) = logsumexp(z) - z_y
  dlogits = (softmax(logits) - onehot(labels)) / n
  grad_hidden = dlogits W          (the gradient handed to the top layer)
  dW     = dlogits^T h
  W, m, v <- AdamW(W, dW, m, v)    ([ENT] cpu_adamw, the adapters' form)

The logits are taken as saved by the forward (as the layer takes its saved
softmax weights).  A row whose label lies outside [0, vocab) (padding,
commonly -100) is ignored: it adds nothing to the loss or to any gradient,
and n counts the rows with a label in range (no rows: loss and gradients 0).
"""
import numpy as np

from .backward import adamw


def softmax_rows(z):
    z = np.asarray(z, np.float64)
    e = np.exp(z - z.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def label_rows(labels, vocab):
    """Mask of the rows whose label is a vocabulary index."""
    labels = np.asarray(labels)
    return (labels >= 0) & (labels < vocab)


def cross_entropy(logits, labels):
    """Mean over the labelled rows of logsumexp(z) - z[label]."""
    z = np.asarray(logits, np.float64)
    ok = label_rows(labels, z.shape[1])
    if not ok.any():
        return 0.0
    z = z[ok]
    mx = z.max(axis=-1)
    lse = mx + np.log(np.exp(z - mx[:, None]).sum(axis=-1))
    return float(np.mean(lse - z[np.arange(z.shape[0]), np.asarray(labels)[ok]]))


def lm_head_bwd(h, logits, labels, W, m, v, lr, beta1, beta2, eps, wd, step):
    """Returns dict(loss, dlogits, grad_hidden, dW, W, m, v) (updated W, m, v)."""
    h = np.asarray(h, np.float64)
    W = np.asarray(W, np.float64)
    p = softmax_rows(logits)
    ok = label_rows(labels, p.shape[1])
    rows = np.nonzero(ok)[0]
    y = np.zeros_like(p)
    y[rows, np.asarray(labels)[rows]] = 1.0
    p[~ok] = 0.0
    S = max(len(rows), 1)
    dlogits = (p - y) / S
    grad_hidden = dlogits @ W
    dW = dlogits.T @ h
    nW, nm, nv = adamw(W, dW, m, v, lr, beta1, beta2, eps, wd, step)
    return dict(loss=cross_entropy(logits, labels), dlogits=dlogits, grad_hidden=grad_hidden,
                dW=dW, W=nW, m=nm, v=nv)


def lm_head_sampled(h, logits, labels, W, rows, cols, chunk=64):
    """loss, grad_hidden[rows] and dW[cols] as lm_head_bwd defines them, for
    inputs too large to form the whole float64 dlogits: each row's softmax
    depends on that row alone (and on n, the labelled-row count), so dlogits
    is formed a block of rows at a time and only the requested rows and
    columns are kept.  W may be float32; it is widened a block at a time."""
    labels = np.asarray(labels)
    S, V = logits.shape
    ok = label_rows(labels, V)
    n = max(int(ok.sum()), 1)
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    loss = 0.0
    d_cols = np.zeros((S, len(cols)))
    d_rows = np.zeros((len(rows), V))
    for r0 in range(0, S, chunk):
        r1 = min(S, r0 + chunk)
        z = np.asarray(logits[r0:r1], np.float64)
        mx = z.max(axis=-1)
        lse = mx + np.log(np.exp(z - mx[:, None]).sum(axis=-1))
        p = np.exp(z - lse[:, None])
        for i in range(r1 - r0):
            s = r0 + i
            if ok[s]:
                loss += lse[i] - z[i, labels[s]]
                p[i, labels[s]] -= 1.0
            else:
                p[i] = 0.0
        p /= n
        d_cols[r0:r1] = p[:, cols]
        for j, s in enumerate(rows):
            if r0 <= s < r1:
                d_rows[j] = p[s - r0]
    grad_hidden = np.zeros((len(rows), W.shape[1]))
    for v0 in range(0, V, 8192):
        v1 = min(V, v0 + 8192)
        grad_hidden += d_rows[:, v0:v1] @ np.asarray(W[v0:v1], np.float64)
    dW = d_cols.T @ np.asarray(h, np.float64)
    return dict(loss=loss / n if ok.any() else 0.0, grad_hidden=grad_hidden, dW=dW)
