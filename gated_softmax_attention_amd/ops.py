"""torch-facing wrappers with the C ABI's names: argument marshalling only."""
import torch

from . import _lib

MODES = {"none": _lib.GSA_GATE_NONE, "elementwise": _lib.GSA_GATE_ELEMENTWISE,
         "headwise": _lib.GSA_GATE_HEADWISE}
_DTYPES = {torch.float32: _lib.GSA_FP32, torch.bfloat16: _lib.GSA_BF16}


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dev(t: torch.Tensor, name: str):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _dtype(*ts):
    dt = ts[0].dtype
    if dt not in _DTYPES:
        raise TypeError(f"unsupported dtype {dt}; use float32 or bfloat16")
    for t in ts[1:]:
        if t.dtype != dt:
            raise TypeError("X/W or Q/K/V/Y tensors must share one dtype")
    return _DTYPES[dt]


def gate_width(layout, heads, D):
    """Gate columns per token row for a layout: heads·D (elementwise), heads
    (headwise) or D (shared: the head-mean of an elementwise gate)."""
    return {"elementwise": heads * D, "headwise": heads, "shared": D}[layout]


def _check_gate(G, layout, rows, heads, D, ref, name="G"):
    """The gate tensor the kernels will read: None exactly when layout is
    "none", else a contiguous float32 tensor on ref's device holding
    rows × gate_width(layout, heads, D) values.  Returns G (the caller takes its
    device pointer after every other check).
    The C ABI cannot see sizes, so this is where a gate of the wrong width or
    dtype is refused before any launch."""
    if layout == "none":
        if G is not None:
            raise ValueError(f"{name} must be None when there is no gate")
        return None
    if G is None:
        raise ValueError(f"{name} is required for the {layout!r} gate")
    if not isinstance(G, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if G.dtype != torch.float32:
        raise TypeError(f"{name} must be float32 (got {G.dtype})")
    if G.device != ref.device:
        raise ValueError(f"{name} is on {G.device}, the other tensors on {ref.device}")
    width = gate_width(layout, heads, D)
    if G.numel() != rows * width:
        raise ValueError(f"{name} has {G.numel()} values; the {layout!r} gate needs {rows} rows x {width}")
    return G


def _opt(t, name):
    return None if t is None else _dev(t, name)


def _out(Y, like, name="Y"):
    """A caller-supplied output must match `like` (shape, dtype, device); None allocates one."""
    if Y is None:
        return torch.empty_like(like)
    if not isinstance(Y, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(Y.shape) != tuple(like.shape) or Y.dtype != like.dtype or Y.device != like.device:
        raise ValueError(f"{name} must be {tuple(like.shape)} {like.dtype} on {like.device} "
                         f"(got {tuple(Y.shape)} {Y.dtype} on {Y.device})")
    return Y


def _same_device(ref, **ts):
    for n, t in ts.items():
        if isinstance(t, torch.Tensor) and t.device != ref.device:
            raise ValueError(f"{n} is on {t.device}, the other tensors on {ref.device}")


ACTIVATIONS = {"identity": _lib.GSA_ACT_IDENTITY, "sigmoid": _lib.GSA_ACT_SIGMOID,
               "ns_sigmoid": _lib.GSA_ACT_NS_SIGMOID, "silu": _lib.GSA_ACT_SILU}


def gate_logits_workspace_bytes(M, d_model, N, dtype=torch.bfloat16):
    return int(_lib.load().gsa_gate_logits_workspace_bytes(M, d_model, N, _DTYPES[dtype]))


def gate_logits(X, W, G=None, apply_sigmoid=True, activation=None, workspace=None, stream=None):
    """G = σ(X·W_θ) (or the logits Z when apply_sigmoid is False), float32 [M, N].
    ``activation`` ("identity", "sigmoid", "ns_sigmoid", "silu") overrides
    apply_sigmoid.  With ``workspace`` (a device tensor of at least
    gate_logits_workspace_bytes(M, d_model, N) bytes, or True to allocate one)
    shapes with few rows take the split-K path (gsa_gate_logits_ws).

    X: [..., d_model] (leading dims flattened to M rows); W: [d_model, N].
    """
    dm = X.shape[-1]
    M = X.numel() // dm
    N = W.shape[1]
    if W.shape[0] != dm:
        raise ValueError(f"W has {W.shape[0]} rows, X has d_model={dm}")
    _same_device(X, W=W)
    if G is None:
        G = torch.empty((M, N), dtype=torch.float32, device=X.device)
    elif not isinstance(G, torch.Tensor) or G.dtype != torch.float32 or G.numel() != M * N \
            or G.device != X.device:
        raise ValueError(f"G must be float32 with M*N = {M * N} elements on {X.device}")
    lib = _lib.load()
    if activation is None:
        act = _lib.GSA_ACT_SIGMOID if apply_sigmoid else _lib.GSA_ACT_IDENTITY
    elif activation in ACTIVATIONS:
        act = ACTIVATIONS[activation]
    else:
        raise ValueError(f"activation must be one of {list(ACTIVATIONS)}")
    if workspace is None:
        _lib.check(lib.gsa_gate_logits(_dev(X, "X"), _dev(W, "W"), _dev(G, "G"), M, dm, N,
                                       _dtype(X, W), act, _stream(stream)))
        return G
    need = int(lib.gsa_gate_logits_workspace_bytes(M, dm, N, _dtype(X, W)))
    if workspace is True:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=X.device) if need else None
    elif workspace.device != X.device:
        raise ValueError("the workspace must be on X's device")
    wp = None if workspace is None else _dev(workspace, "workspace")
    wb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _lib.check(lib.gsa_gate_logits_ws(_dev(X, "X"), _dev(W, "W"), _dev(G, "G"), M, dm, N, _dtype(X, W), act,
                                      wp, wb, _stream(stream)))
    return G


def _layout_of_mode(mode):
    _mode(mode)
    return mode


def _mode(mode):
    if mode not in MODES:
        raise ValueError(f"mode must be one of {list(MODES)}")
    return MODES[mode]


def forward(Q, K, V, G, mode, Y=None, stream=None):
    """Causal gated SDPA, Y' [B, S, Hq, D] from Q [B,S,Hq,D], K/V [B,S,Hkv,D] and G."""
    B, S, Hq, D = Q.shape
    Hkv = K.shape[2]
    if K.shape != (B, S, Hkv, D) or V.shape != K.shape:
        raise ValueError("K and V must be [B, S, Hkv, D] matching Q")
    _same_device(Q, K=K, V=V)
    G = _check_gate(G, _layout_of_mode(mode), B * S, Hq, D, Q)
    Y = _out(Y, Q)
    lib = _lib.load()
    _lib.check(lib.gsa_forward(_dev(Q, "Q"), _dev(K, "K"), _dev(V, "V"), _opt(G, "G"), _dev(Y, "Y"),
                               B, S, Hq, Hkv, D, _mode(mode), _dtype(Q, K, V, Y), _stream(stream)))
    return Y


def forward_lse(Q, K, V, G, mode, Y=None, LSE=None, stream=None):
    """forward() that also returns the per-row log-sum-exp LSE [B, Hq, S] float32."""
    B, S, Hq, D = Q.shape
    Hkv = K.shape[2]
    if K.shape != (B, S, Hkv, D) or V.shape != K.shape:
        raise ValueError("K and V must be [B, S, Hkv, D] matching Q")
    _same_device(Q, K=K, V=V, LSE=LSE)
    G = _check_gate(G, _layout_of_mode(mode), B * S, Hq, D, Q)
    Y = _out(Y, Q)
    if LSE is None:
        LSE = torch.empty((B, Hq, S), dtype=torch.float32, device=Q.device)
    elif LSE.dtype != torch.float32 or LSE.numel() != B * Hq * S:
        raise ValueError("LSE must be float32 with B*Hq*S elements")
    lib = _lib.load()
    _lib.check(lib.gsa_forward_lse(_dev(Q, "Q"), _dev(K, "K"), _dev(V, "V"), _opt(G, "G"), _dev(Y, "Y"),
                                   _dev(LSE, "LSE"), B, S, Hq, Hkv, D, _mode(mode),
                                   _dtype(Q, K, V, Y), _stream(stream)))
    return Y, LSE


def decode_num_splits(B, L, Hq, Hkv, D, num_splits=0):
    return int(_lib.load().gsa_decode_num_splits(B, L, Hq, Hkv, D, num_splits))


def decode_workspace_bytes(B, L, Hq, Hkv, D, num_splits=0):
    return int(_lib.load().gsa_decode_workspace_bytes(B, L, Hq, Hkv, D, num_splits))


def decode(Q, Kc, Vc, G, mode, num_splits=0, Y=None, workspace=None, stream=None):
    """One decode step: Q [B,1,Hq,D] against the cache Kc/Vc [B,L,Hkv,D]."""
    B, one, Hq, D = Q.shape
    if one != 1:
        raise ValueError("decode takes one query token per batch")
    L, Hkv = Kc.shape[1], Kc.shape[2]
    if Kc.shape != (B, L, Hkv, D) or Vc.shape != Kc.shape:
        raise ValueError("Kc and Vc must be [B, L, Hkv, D] matching Q")
    _same_device(Q, Kc=Kc, Vc=Vc, workspace=workspace)
    G = _check_gate(G, _layout_of_mode(mode), B, Hq, D, Q)
    Y = _out(Y, Q)
    need = decode_workspace_bytes(B, L, Hq, Hkv, D, num_splits)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=Q.device)
    wp = None if workspace is None else _dev(workspace, "workspace")
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    lib = _lib.load()
    _lib.check(lib.gsa_decode(_dev(Q, "Q"), _dev(Kc, "Kc"), _dev(Vc, "Vc"), _opt(G, "G"), _dev(Y, "Y"),
                              B, L, Hq, Hkv, D, _mode(mode), _dtype(Q, Kc, Vc, Y), num_splits,
                              wp, wbytes, _stream(stream)))
    return Y


def noalloc_scratch_bytes():
    return int(_lib.load().gsa_noalloc_scratch_bytes())


def decode_noalloc(Q, Kc, Vc, G, mode, Y, num_splits=0, stream=None):
    """decode() through gsa_decode_noalloc: the split partials live in the
    library's own device scratch, and nothing is allocated here either, so the
    caller passes the output Y [B,1,Hq,D].  Calls that overlap in time on one GPU
    race on that scratch."""
    B, one, Hq, D = Q.shape
    if one != 1:
        raise ValueError("decode takes one query token per batch")
    L, Hkv = Kc.shape[1], Kc.shape[2]
    if Kc.shape != (B, L, Hkv, D) or Vc.shape != Kc.shape:
        raise ValueError("Kc and Vc must be [B, L, Hkv, D] matching Q")
    if Y is None:
        raise ValueError("decode_noalloc allocates nothing: pass the output Y")
    _same_device(Q, Kc=Kc, Vc=Vc)
    G = _check_gate(G, _layout_of_mode(mode), B, Hq, D, Q)
    Y = _out(Y, Q)
    lib = _lib.load()
    _lib.check(lib.gsa_decode_noalloc(_dev(Q, "Q"), _dev(Kc, "Kc"), _dev(Vc, "Vc"), _opt(G, "G"), _dev(Y, "Y"),
                                      B, L, Hq, Hkv, D, _mode(mode), _dtype(Q, Kc, Vc, Y), num_splits,
                                      _stream(stream)))
    return Y


def backward_workspace_bytes(B, S, Hq, Hkv, D, d_model, mode):
    return int(_lib.load().gsa_backward_workspace_bytes(B, S, Hq, Hkv, D, d_model, _mode(mode)))


def backward(X, W, G, Q, K, V, Y, LSE, dY, mode, workspace=None, stream=None):
    """Gradients of the gated forward for the upstream gradient dY of Y'.

    X [..., d_model] and W [d_model, N] are the gate projection's inputs, G its
    float32 output (from gate_logits), Y and LSE the outputs of forward_lse.  For
    mode "none" X, W and G are None.  Returns a dict with dQ, dK, dV (shapes of
    Q, K, V, bf16), dX (shape of X, bf16) and dW (float32 [d_model, N]); the
    last two are None without a gate.
    """
    B, S, Hq, D = Q.shape
    Hkv = K.shape[2]
    if K.shape != (B, S, Hkv, D) or V.shape != K.shape:
        raise ValueError("K and V must be [B, S, Hkv, D] matching Q")
    if Y.shape != Q.shape or dY.shape != Q.shape:
        raise ValueError("Y and dY must have Q's shape")
    if LSE.dtype != torch.float32 or LSE.numel() != B * Hq * S:
        raise ValueError("LSE must be float32 with B*Hq*S elements")
    gated = _mode(mode) != _lib.GSA_GATE_NONE
    _same_device(Q, K=K, V=V, Y=Y, LSE=LSE, dY=dY, X=X, W=W, workspace=workspace)
    _check_gate(G, mode, B * S, Hq, D, Q)
    if not gated and (X is not None or W is not None):
        raise ValueError("X and W must be None without a gate")
    d_model = X.shape[-1] if gated else 0
    if gated and (W.dim() != 2 or W.shape[0] != d_model or X.numel() != B * S * d_model
                  or W.shape[1] != gate_width(mode, Hq, D)):
        raise ValueError(f"X must hold B*S = {B * S} rows of d_model and W must be [d_model, "
                         f"{gate_width(mode, Hq, D)}] for the {mode!r} gate")
    need = backward_workspace_bytes(B, S, Hq, Hkv, D, d_model, mode)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=Q.device)
    dQ, dK, dV = torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V)
    dX = torch.empty_like(X) if gated else None
    dW = torch.empty(tuple(W.shape), dtype=torch.float32, device=Q.device) if gated else None
    p = lambda t, n: None if t is None else _dev(t, n)
    lib = _lib.load()
    _lib.check(lib.gsa_backward(
        p(X, "X"), p(W, "W"), p(G, "G"), _dev(Q, "Q"), _dev(K, "K"), _dev(V, "V"), _dev(Y, "Y"),
        _dev(LSE, "LSE"), _dev(dY, "dY"), p(dX, "dX"), p(dW, "dW"), _dev(dQ, "dQ"), _dev(dK, "dK"),
        _dev(dV, "dV"), B, S, Hq, Hkv, D, d_model, _mode(mode), _dtype(Q, K, V, Y, dY),
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream(stream)))
    return {"dQ": dQ, "dK": dK, "dV": dV, "dX": dX, "dW": dW}


LAYOUTS = {"none": _lib.GSA_GATE_NONE, "elementwise": _lib.GSA_GATE_ELEMENTWISE,
           "headwise": _lib.GSA_GATE_HEADWISE, "shared": _lib.GSA_GATE_SHARED}


def forward_variant(Q, K, V, G, layout, combine="mul", norm=None, Y=None, LSE=None, stream=None):
    """Causal SDPA with a design-space gate: combine(norm(Y), G) with G already
    activated (gate_logits' activation), layout in LAYOUTS, combine "mul" or
    "add", norm None or "rms".  Returns Y' (and LSE when an LSE tensor is given)."""
    B, S, Hq, D = Q.shape
    Hkv = K.shape[2]
    if K.shape != (B, S, Hkv, D) or V.shape != K.shape:
        raise ValueError("K and V must be [B, S, Hkv, D] matching Q")
    if layout not in LAYOUTS or combine not in ("mul", "add") or norm not in (None, "rms"):
        raise ValueError("layout, combine or norm not recognised")
    _same_device(Q, K=K, V=V, LSE=LSE)
    G = _check_gate(G, layout, B * S, Hq, D, Q)
    Y = _out(Y, Q)
    if LSE is not None and (LSE.dtype != torch.float32 or LSE.numel() != B * Hq * S):
        raise ValueError("LSE must be float32 with B*Hq*S elements")
    lib = _lib.load()
    _lib.check(lib.gsa_forward_variant(
        _dev(Q, "Q"), _dev(K, "K"), _dev(V, "V"), _opt(G, "G"), _dev(Y, "Y"),
        None if LSE is None else _dev(LSE, "LSE"), B, S, Hq, Hkv, D, LAYOUTS[layout],
        _lib.GSA_COMBINE_ADD if combine == "add" else _lib.GSA_COMBINE_MUL,
        _lib.GSA_NORM_RMS if norm == "rms" else _lib.GSA_NORM_NONE, _dtype(Q, K, V, Y), _stream(stream)))
    return Y if LSE is None else (Y, LSE)


def decode_variant(Q, Kc, Vc, G, layout, combine="mul", norm=None, num_splits=0, Y=None, workspace=None,
                   stream=None):
    """One decode step with a design-space gate at the merge: combine(norm(Y), G)
    with G [B, N] already activated, layout in LAYOUTS, combine "mul" or "add",
    norm None or "rms"; other arguments as decode."""
    B, one, Hq, D = Q.shape
    if one != 1:
        raise ValueError("decode takes one query token per batch")
    L, Hkv = Kc.shape[1], Kc.shape[2]
    if Kc.shape != (B, L, Hkv, D) or Vc.shape != Kc.shape:
        raise ValueError("Kc and Vc must be [B, L, Hkv, D] matching Q")
    if layout not in LAYOUTS or combine not in ("mul", "add") or norm not in (None, "rms"):
        raise ValueError("layout, combine or norm not recognised")
    _same_device(Q, Kc=Kc, Vc=Vc, workspace=workspace)
    G = _check_gate(G, layout, B, Hq, D, Q)
    Y = _out(Y, Q)
    need = decode_workspace_bytes(B, L, Hq, Hkv, D, num_splits) if Q.dtype == torch.bfloat16 else 0
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=Q.device)
    wp = None if workspace is None else _dev(workspace, "workspace")
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    lib = _lib.load()
    _lib.check(lib.gsa_decode_variant(
        _dev(Q, "Q"), _dev(Kc, "Kc"), _dev(Vc, "Vc"), _opt(G, "G"), _dev(Y, "Y"),
        B, L, Hq, Hkv, D, LAYOUTS[layout], _lib.GSA_COMBINE_ADD if combine == "add" else _lib.GSA_COMBINE_MUL,
        _lib.GSA_NORM_RMS if norm == "rms" else _lib.GSA_NORM_NONE, _dtype(Q, Kc, Vc, Y), num_splits, wp, wbytes,
        _stream(stream)))
    return Y


def forward_value_gated(Q, K, V, Gv, layout, Y=None, LSE=None, stream=None):
    """Causal SDPA over the G2-gated values V ⊙ Gv (Gv = σ(X·W_v) per key/value
    head and dim, [B*S, Hkv*D], or per key/value head, [B*S, Hkv], float32),
    gated as the kernel stages the value tiles.  Returns Y (and LSE when an LSE
    tensor is given)."""
    B, S, Hq, D = Q.shape
    Hkv = K.shape[2]
    if K.shape != (B, S, Hkv, D) or V.shape != K.shape:
        raise ValueError("K and V must be [B, S, Hkv, D] matching Q")
    if layout not in ("elementwise", "headwise"):
        raise ValueError("the value gate's layout is 'elementwise' or 'headwise'")
    _same_device(Q, K=K, V=V, LSE=LSE)
    Gv = _check_gate(Gv, layout, B * S, Hkv, D, Q, name="Gv")
    Y = _out(Y, Q)
    if LSE is not None and (LSE.dtype != torch.float32 or LSE.numel() != B * Hq * S):
        raise ValueError("LSE must be float32 with B*Hq*S elements")
    lib = _lib.load()
    _lib.check(lib.gsa_forward_value_gated(
        _dev(Q, "Q"), _dev(K, "K"), _dev(V, "V"), _dev(Gv, "Gv"), _dev(Y, "Y"),
        None if LSE is None else _dev(LSE, "LSE"), B, S, Hq, Hkv, D, LAYOUTS[layout], _dtype(Q, K, V, Y),
        _stream(stream)))
    return Y if LSE is None else (Y, LSE)


def value_gate(V, G, layout, Vout=None, stream=None):
    """G2: V ⊙ G per key/value head (elementwise G [B*S, Hkv*D]) or per head
    (headwise G [B*S, Hkv]); returns the gated values, V's shape and dtype."""
    B, S, Hkv, D = V.shape
    if layout not in ("elementwise", "headwise"):
        raise ValueError("the value gate's layout is 'elementwise' or 'headwise'")
    G = _check_gate(G, layout, B * S, Hkv, D, V)
    Vout = _out(Vout, V, "Vout")
    lib = _lib.load()
    _lib.check(lib.gsa_value_gate(_dev(V, "V"), _opt(G, "G"), _dev(Vout, "Vout"), B, S, Hkv, D,
                                  LAYOUTS[layout], _dtype(V, Vout), _stream(stream)))
    return Vout


def project_qkvg(X, Wcat, Hq, Hkv, D, n_gate, stream=None):
    """Q [.., Hq, D], K and V [.., Hkv, D] (bf16) and G = σ(Z) [M, n_gate] float32
    (None when n_gate is 0) from X [..., d_model] and Wcat = [W_Q | W_K | W_V | W_θ]."""
    dm = X.shape[-1]
    M = X.numel() // dm
    lead = tuple(X.shape[:-1])
    if Wcat.shape != (dm, (Hq + 2 * Hkv) * D + n_gate):
        raise ValueError("Wcat must be [d_model, Hq*D + 2*Hkv*D + n_gate]")
    Q = torch.empty(lead + (Hq, D), dtype=X.dtype, device=X.device)
    K = torch.empty(lead + (Hkv, D), dtype=X.dtype, device=X.device)
    V = torch.empty(lead + (Hkv, D), dtype=X.dtype, device=X.device)
    G = torch.empty((M, n_gate), dtype=torch.float32, device=X.device) if n_gate > 0 else None
    lib = _lib.load()
    _lib.check(lib.gsa_project_qkvg(_dev(X, "X"), _dev(Wcat, "Wcat"), _dev(Q, "Q"), _dev(K, "K"), _dev(V, "V"),
                                    None if G is None else _dev(G, "G"), M, dm, Hq, Hkv, D, n_gate,
                                    _dtype(X, Wcat), _stream(stream)))
    return Q, K, V, G


def first_token_attention(Q, K, LSE, with_means=True, stream=None):
    """Share of attention each query row gives token 0, F [B, Hq, S] float32, from
    the LSE of forward_lse on the same Q and K.  With with_means also returns the
    per-head means over batches and rows followed by their mean (Hq + 1 floats)."""
    B, S, Hq, D = Q.shape
    Hkv = K.shape[2]
    if K.shape != (B, S, Hkv, D):
        raise ValueError("K must be [B, S, Hkv, D] matching Q")
    if LSE.dtype != torch.float32 or LSE.numel() != B * Hq * S:
        raise ValueError("LSE must be float32 with B*Hq*S elements")
    F = torch.empty((B, Hq, S), dtype=torch.float32, device=Q.device)
    means = torch.empty(Hq + 1, dtype=torch.float32, device=Q.device) if with_means else None
    lib = _lib.load()
    _lib.check(lib.gsa_first_token_attention(_dev(Q, "Q"), _dev(K, "K"), _dev(LSE, "LSE"), _dev(F, "F"),
                                             None if means is None else _dev(means, "head_mean"),
                                             B, S, Hq, Hkv, D, _dtype(Q, K), _stream(stream)))
    return (F, means) if with_means else F


def _check_gate_inputs(X, W, rows, Hq, D, mode):
    """X must hold `rows` token rows and W_θ must have the gate width of `mode`."""
    if _mode(mode) == _lib.GSA_GATE_NONE:
        return
    if X is None or W is None:
        raise ValueError(f"X and W are required for the {mode!r} gate")
    dm = X.shape[-1]
    if X.numel() != rows * dm:
        raise ValueError(f"X must hold {rows} token rows of d_model (got shape {tuple(X.shape)})")
    if W.dim() != 2 or W.shape[0] != dm or W.shape[1] != gate_width(mode, Hq, D):
        raise ValueError(f"W must be [d_model={dm}, {gate_width(mode, Hq, D)}] for the {mode!r} gate "
                         f"(got {tuple(W.shape)})")


def gate_head_mean(G, Hq, D, Gs=None, stream=None):
    """Head-shared gate scores Gs [M, D] = the mean over the Hq heads of the
    activated elementwise scores G [M, Hq·D] (float32)."""
    if not isinstance(G, torch.Tensor) or G.dtype != torch.float32:
        raise TypeError("G must be a float32 torch.Tensor")
    if G.numel() % (Hq * D) != 0:
        raise ValueError(f"G must hold rows of Hq*D = {Hq * D} values")
    M = G.numel() // (Hq * D)
    if Gs is None:
        Gs = torch.empty((M, D), dtype=torch.float32, device=G.device)
    elif Gs.dtype != torch.float32 or Gs.numel() != M * D or Gs.device != G.device:
        raise ValueError(f"Gs must be float32 with M*D = {M * D} values on {G.device}")
    lib = _lib.load()
    _lib.check(lib.gsa_gate_head_mean(_dev(G, "G"), _dev(Gs, "Gs"), M, Hq, D, _stream(stream)))
    return Gs


def gated_attention(X, W, Q, K, V, mode, stream=None):
    """The whole prefill path: gate projection + sigmoid, then causal gated SDPA."""
    B, S, Hq, D = Q.shape
    _check_gate_inputs(X, W, B * S, Hq, D, mode)
    G = None if mode == "none" else gate_logits(X, W, stream=stream)
    return forward(Q, K, V, G, mode, stream=stream)


def gated_decode_workspace_bytes(B, L, Hq, Hkv, D, d_model, mode, dtype=torch.bfloat16, num_splits=0):
    return int(_lib.load().gsa_gated_decode_workspace_bytes(B, L, Hq, Hkv, D, d_model, _mode(mode), _DTYPES[dtype],
                                                             num_splits))


def gated_decode(X, W, Q, Kc, Vc, mode, num_splits=0, Y=None, workspace=None, stream=None):
    """The whole decode path in one call (gsa_gated_decode): the gate σ(X·W_θ) of
    the B new tokens (split-K for few rows) and the decode of Q [B,1,Hq,D]
    against Kc/Vc [B,L,Hkv,D], with one workspace for both."""
    B, one, Hq, D = Q.shape
    if one != 1:
        raise ValueError("decode takes one query token per batch")
    L, Hkv = Kc.shape[1], Kc.shape[2]
    if Kc.shape != (B, L, Hkv, D) or Vc.shape != Kc.shape:
        raise ValueError("Kc and Vc must be [B, L, Hkv, D] matching Q")
    _check_gate_inputs(X, W, B, Hq, D, mode)
    gated = _mode(mode) != _lib.GSA_GATE_NONE
    if not gated and (X is not None or W is not None):
        raise ValueError("X and W must be None without a gate")
    _same_device(Q, Kc=Kc, Vc=Vc, X=X, W=W, workspace=workspace)
    if gated:
        _dtype(Q, Kc, Vc, X, W)
    Y = _out(Y, Q)
    dm = X.shape[-1] if gated else 0
    need = gated_decode_workspace_bytes(B, L, Hq, Hkv, D, dm, mode, Q.dtype, num_splits)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=Q.device)
    wp = None if workspace is None else _dev(workspace, "workspace")
    wb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    lib = _lib.load()
    _lib.check(lib.gsa_gated_decode(None if X is None else _dev(X, "X"), None if W is None else _dev(W, "W"),
                                    _dev(Q, "Q"), _dev(Kc, "Kc"), _dev(Vc, "Vc"), _dev(Y, "Y"), B, L, Hq, Hkv, D, dm,
                                    _mode(mode), _dtype(Q, Kc, Vc, Y), num_splits, wp, wb, _stream(stream)))
    return Y


def gated_attention_variant(X, W, Q, K, V, layout, activation="sigmoid", combine="mul", norm=None, stream=None):
    """A design-space point of the whole prefill path: G = act(X·W_θ), then for
    the head-shared layout the mean over the heads (W_θ is Hq·D wide, as for
    elementwise), then the variant forward combine(norm(Y), G)."""
    B, S, Hq, D = Q.shape
    if layout == "none":
        return forward_variant(Q, K, V, None, "none", combine, norm, stream=stream)
    _check_gate_inputs(X, W, B * S, Hq, D, "elementwise" if layout == "shared" else layout)
    G = gate_logits(X, W, activation=activation, stream=stream)
    if layout == "shared":
        G = gate_head_mean(G, Hq, D, stream=stream)
    return forward_variant(Q, K, V, G, layout, combine, norm, stream=stream)
