"""The SwiGLU expert FFN and the gate-weighted layer output (oracle; test infrastructure).

* Expert structure: gate, up and down projections; the down projection reads
  SiLU(gate) * up ([OSDI] section 4.3).  With weights stored [out, in]:
  FFN(x) = W_down (silu(W_gate x) * (W_up x)),  silu(a) = a / (1 + e^-a).
* Layer output: y_t = sum_j w_tj FFN_{id_tj}(x_t), the gate weight applied to
  each expert's output ([FT] "Graph 内的 CPU 执行分支": workers return
  gate-weighted per-token partial outputs).
* Split: the GPU sums the picks whose route was rewritten to a slot, the
  host sums the rest, and the two partial sums are added exactly ([FT]
  "q* 策略": CPU and GPU partial sums are merged without changing router,
  experts or precision).

Everything is float64 with exactly decoded weights; matrix products are
numpy's (a library primitive); no intermediate rounding.
"""
import numpy as np


def silu(a):
    a = np.asarray(a, dtype=np.float64)
    with np.errstate(over="ignore"):
        return a / (1.0 + np.exp(-a))


def expert_ffn(x, w_gate, w_up, w_down):
    """x [n, H]; w_gate, w_up [I, H]; w_down [H, I] (float64) -> [n, H]."""
    x = np.asarray(x, dtype=np.float64)
    g = x @ np.asarray(w_gate, np.float64).T
    u = x @ np.asarray(w_up, np.float64).T
    return (silu(g) * u) @ np.asarray(w_down, np.float64).T


def moe_partials(x, ids, w, expert, on_gpu=None):
    """Gate-weighted layer output split into (y_gpu, y_host).

    x float64 [T, H]; ids [T, k] expert keys; w [T, k] gate weights;
    expert(key) -> (w_gate, w_up, w_down) float64; on_gpu bool [T, k]
    (True where the route was rewritten to a slot; default all True).
    Each expert is evaluated once on the rows that picked it."""
    x = np.asarray(x, dtype=np.float64)
    ids = np.asarray(ids)
    w = np.asarray(w, dtype=np.float64)
    T, k = ids.shape
    if on_gpu is None:
        on_gpu = np.ones((T, k), bool)
    y_gpu = np.zeros((T, x.shape[1]))
    y_host = np.zeros((T, x.shape[1]))
    for key in sorted(set(ids.reshape(-1).tolist())):
        tt, jj = np.nonzero(ids == key)
        out = expert_ffn(x[tt], *expert(key))
        contrib = w[tt, jj][:, None] * out
        g = on_gpu[tt, jj]
        np.add.at(y_gpu, tt[g], contrib[g])
        np.add.at(y_host, tt[~g], contrib[~g])
    return y_gpu, y_host


def moe_output(x, ids, w, expert):
    y_gpu, y_host = moe_partials(x, ids, w, expert)
    return y_gpu + y_host
