"""One SmoothQuant W8A8 linear layer on one GPU: its device buffers and the
sequence of C-ABI calls that make up the path.

The record kept per layer follows ADR-010's SmoothQuantLinear (int8 weight
with a per-row scale, a per-tensor activation scale, per-input-channel
smoothing factors), with fp32 scales, or with every scale stored in fp16 as
the ADR's "Consequences" section has it (scales="f16": float16 tensors, the
_f16 entry points, no stored 1/s). PyTorch only allocates the buffers and
supplies the stream; all arithmetic is in libsq.so.

    step(x_calib, x) = calibrate(x_calib) -> prepare() -> forward(x)
      calibrate: act_max  = max |x_calib| per input channel   (sq_calib_absmax)
      prepare:   w_max    = max |W| per input channel          (sq_calib_absmax)
                 s, 1/s, act_scale                             (sq_smooth_factors)
                 Wq, w_scale = per-row int8 of W diag(s)       (sq_quant_weight)
      forward:   Xq = per-tensor int8 of x * (1/s)             (sq_smooth_quant_act)
                 Y  = dequant(Xq Wq^T)                         (sq_w8a8_gemm)
      forward_dynamic: the same with the per-tensor scale taken from x itself
                 (sq_dynamic_quant_act; pwwt.cn §2.3 dynamic mode)

prepare_block(layers, calib) does calibrate + prepare for the projections of
one transformer block with the batched entry points: every statistic (the
calibration inputs' and the weights') in one launch, the smoothing factors in
two, the weight codes in one per row-length class; forward_block(layers, xs)
quantizes every input in one launch (an input shared by several projections
is read once) and runs the products in one grouped launch. Results are
identical to the per-layer calls.
"""
from __future__ import annotations

from . import capi


def _fresh(shape, dtype, device, *streams):
    """A new buffer for kernels that run on `streams`: torch's caching
    allocator ties a block to the stream that allocated it, so the block is
    also recorded on every other stream that reads or writes it; otherwise,
    once the caller drops the tensor, the block could be handed to a new
    allocation on the current stream while those kernels still use it."""
    import torch
    t = torch.empty(shape, dtype=dtype, device=device)
    cur = torch.cuda.current_stream(device)
    for s in streams:
        if s is not None and s != cur:
            t.record_stream(s)
    return t


class W8A8Linear:
    def __init__(self, w, alpha: float = 0.5, max_tokens: int = 0, out_dtype=None, scales: str = "f32"):
        import torch
        if scales not in ("f32", "f16"):
            raise ValueError(f"scales must be 'f32' or 'f16', got {scales!r}")
        self.w = w
        self.alpha = float(alpha)
        self.scales = scales
        self.n, self.k = w.shape
        d = w.device
        f32 = torch.float32
        sd = torch.float16 if scales == "f16" else f32
        self.act_max = torch.zeros(self.k, dtype=f32, device=d)
        self.w_max = torch.empty(self.k, dtype=f32, device=d)
        self.s = torch.empty(self.k, dtype=sd, device=d)
        # fp16 storage keeps no 1/s: the kernels form fl(1 / s) from the stored s
        self.inv_s = torch.empty(self.k, dtype=f32, device=d) if scales == "f32" else None
        self.act_scale = torch.empty(16 // sd.itemsize, dtype=sd, device=d)  # one value, padded to 16 bytes
        self.wq = torch.empty((self.n, self.k), dtype=torch.int8, device=d)
        self.w_scale = torch.empty(self.n, dtype=sd, device=d)
        self.live_max = torch.empty(self.k, dtype=f32, device=d)  # dynamic mode: the batch statistic
        self.dyn_scale = torch.empty(4, dtype=f32, device=d)      # dynamic mode: the batch's scale
        self.out_dtype = out_dtype if out_dtype is not None else torch.bfloat16
        self.xq = torch.empty((max_tokens, self.k), dtype=torch.int8, device=d) if max_tokens else None
        self.y = torch.empty((max_tokens, self.n), dtype=self.out_dtype, device=d) if max_tokens else None

    def calibrate(self, x, accumulate: bool = False, stream=None):
        capi.sq_calib_absmax(x, self.act_max, accumulate, stream)

    def prepare(self, stream=None):
        capi.sq_calib_absmax(self.w, self.w_max, False, stream)
        if self.scales == "f16":
            capi.sq_smooth_factors_f16(self.act_max, self.w_max, self.alpha, self.s, self.act_scale, stream)
            capi.sq_quant_weight_f16(self.w, self.s, self.wq, self.w_scale, stream)
            return
        capi.sq_smooth_factors(self.act_max, self.w_max, self.alpha, self.s, self.inv_s, self.act_scale, stream)
        capi.sq_quant_weight(self.w, self.s, self.wq, self.w_scale, stream)

    def quantize_input(self, x, xq=None, stream=None):
        import torch
        m = x.shape[0]
        if xq is None:
            xq = self.xq[:m] if self.xq is not None and self.xq.shape[0] >= m else \
                _fresh((m, self.k), torch.int8, x.device, stream)
        if self.scales == "f16":
            capi.sq_smooth_quant_act_f16(x, self.s, self.act_scale, xq, stream)
        else:
            capi.sq_smooth_quant_act(x, self.inv_s, self.act_scale, xq, stream)
        return xq

    def quantize_input_dynamic(self, x, xq=None, stream=None):
        import torch
        if self.scales != "f32":
            raise ValueError("the dynamic scale mode keeps fp32 scales")
        m = x.shape[0]
        if xq is None:
            xq = self.xq[:m] if self.xq is not None and self.xq.shape[0] >= m else \
                _fresh((m, self.k), torch.int8, x.device, stream)
        capi.sq_dynamic_quant_act(x, self.inv_s, self.live_max, self.dyn_scale, xq, stream)
        return xq

    def matmul(self, xq, y=None, acc_out=None, stream=None, act_scale=None):
        import torch
        m = xq.shape[0]
        if y is None:
            y = self.y[:m] if self.y is not None and self.y.shape[0] >= m else \
                _fresh((m, self.n), self.out_dtype, xq.device, stream)
        a = self.act_scale if act_scale is None else act_scale
        if self.scales == "f16":
            capi.sq_w8a8_gemm_f16(xq, self.wq, a, self.w_scale, y, acc_out, stream)
        else:
            capi.sq_w8a8_gemm(xq, self.wq, a, self.w_scale, y, acc_out, stream)
        return y

    def forward(self, x, y=None, xq=None, acc_out=None, stream=None):
        return self.matmul(self.quantize_input(x, xq, stream), y, acc_out, stream)

    def forward_dynamic(self, x, y=None, xq=None, acc_out=None, stream=None):
        return self.matmul(self.quantize_input_dynamic(x, xq, stream), y, acc_out, stream, act_scale=self.dyn_scale)

    def step(self, x_calib, x, stream=None):
        self.calibrate(x_calib, False, stream)
        self.prepare(stream)
        return self.forward(x, stream=stream)


MAX_BATCH = 16  # SQ_MAX_BATCH, the most items one batched call takes


def _chunks(seq):
    return [seq[i:i + MAX_BATCH] for i in range(0, len(seq), MAX_BATCH)]


def _storage(layers):
    """The scale storage shared by every layer of a block call."""
    kinds = {l.scales for l in layers}
    if len(kinds) > 1:
        raise ValueError("the layers of one block call must share their scale storage")
    return kinds.pop() if kinds else "f32"


def prepare_block(layers, calib=(), stream=None):
    """calibrate + prepare for several W8A8Linear layers in few launches.
    calib: (x, act_max) pairs; act_max is overwritten with the column max of
    |x| (layers that share an input hold the same act_max tensor)."""
    f16 = _storage(layers) == "f16"
    stats = [(x, a) for x, a in calib] + [(l.w, l.w_max) for l in layers]
    for part in _chunks(stats):
        capi.sq_calib_absmax_batched([x for x, _ in part], [a for _, a in part], False, stream)
    for part in _chunks(list(layers)):
        if f16:
            capi.sq_smooth_factors_f16_batched([l.act_max for l in part], [l.w_max for l in part],
                                               [l.alpha for l in part], [l.s for l in part],
                                               [l.act_scale for l in part], stream)
            capi.sq_quant_weight_f16_batched([l.w for l in part], [l.s for l in part], [l.wq for l in part],
                                             [l.w_scale for l in part], stream)
            continue
        capi.sq_smooth_factors_batched([l.act_max for l in part], [l.w_max for l in part], [l.alpha for l in part],
                                       [l.s for l in part], [l.inv_s for l in part], [l.act_scale for l in part],
                                       stream)
        capi.sq_quant_weight_batched([l.w for l in part], [l.s for l in part], [l.wq for l in part],
                                     [l.w_scale for l in part], stream)


def forward_block(layers, xs, stream=None, gemm_stream=None, between=None):
    """forward for several layers: xs[i] feeds layers[i] (the same tensor for
    layers that share an input). The activation codes are made on `stream`,
    the products on `gemm_stream` (default: the same stream; a different one
    must already be ordered after `stream` by the caller via `between`, a
    callable run between the two launches). Returns the outputs."""
    import torch
    f16 = _storage(layers) == "f16"
    quant = capi.sq_smooth_quant_act_f16_batched if f16 else capi.sq_smooth_quant_act_batched
    gemm = capi.sq_w8a8_gemm_f16_batched if f16 else capi.sq_w8a8_gemm_batched
    xqs, ys = [], []
    gs = gemm_stream if gemm_stream is not None else stream
    for l, x in zip(layers, xs):
        m = x.shape[0]
        xqs.append(l.xq[:m] if l.xq is not None and l.xq.shape[0] >= m else
                   _fresh((m, l.k), torch.int8, x.device, stream, gs))
        ys.append(l.y[:m] if l.y is not None and l.y.shape[0] >= m else
                  _fresh((m, l.n), l.out_dtype, x.device, gs))
    for part in _chunks(list(range(len(layers)))):
        quant([xs[i] for i in part], [layers[i].s if f16 else layers[i].inv_s for i in part],
              [layers[i].act_scale for i in part], [xqs[i] for i in part], stream)
    if between is not None:
        between()
    # products in reverse order of preparation: the codes written last are the
    # ones still in the 256 MB Infinity Cache when the products start
    # (measured on the 13B block: the grouped launch 602 -> 591 us with
    # 256 x 160 tiles, 546 -> 536 us with 256 x 256)
    for part in _chunks(list(range(len(layers)))[::-1]):
        gemm([xqs[i] for i in part], [layers[i].wq for i in part], [layers[i].act_scale for i in part],
             [layers[i].w_scale for i in part], [ys[i] for i in part], None, gs)
    return ys


def forward_block_dynamic(layers, xs, stream=None):
    """forward_dynamic for several layers in four launches (plus the zero
    fill of the statistics): the live max of each distinct input (one batched
    reduction; layers that share an input tensor share its statistic), every
    layer's dynamic act scale (one launch), the activation codes (one launch)
    and the products (one grouped launch, newest-first as in forward_block).
    Every layer's dyn_scale holds its batch scale, as after forward_dynamic;
    the batch statistic is written to the live_max of the first layer that
    reads each input (the others' live_max are left as they were). Returns
    the outputs."""
    import torch
    if _storage(layers) != "f32":
        raise ValueError("the dynamic scale mode keeps fp32 scales")
    distinct, owner = [], {}
    for l, x in zip(layers, xs):
        if id(x) not in owner:
            owner[id(x)] = l
            distinct.append((x, l.live_max))
    for part in _chunks(distinct):
        capi.sq_calib_absmax_batched([x for x, _ in part], [a for _, a in part], False, stream)
    live = [owner[id(x)].live_max for x in xs]
    for part in _chunks(list(range(len(layers)))):
        capi.sq_act_scale_batched([live[i] for i in part], [layers[i].inv_s for i in part],
                                  [layers[i].dyn_scale for i in part], stream)
    xqs, ys = [], []
    for l, x in zip(layers, xs):
        m = x.shape[0]
        xqs.append(l.xq[:m] if l.xq is not None and l.xq.shape[0] >= m else
                   _fresh((m, l.k), torch.int8, x.device, stream))
        ys.append(l.y[:m] if l.y is not None and l.y.shape[0] >= m else
                  _fresh((m, l.n), l.out_dtype, x.device, stream))
    for part in _chunks(list(range(len(layers)))):
        capi.sq_smooth_quant_act_batched([xs[i] for i in part], [layers[i].inv_s for i in part],
                                         [layers[i].dyn_scale for i in part], [xqs[i] for i in part], stream)
    for part in _chunks(list(range(len(layers)))[::-1]):
        capi.sq_w8a8_gemm_batched([xqs[i] for i in part], [layers[i].wq for i in part],
                                  [layers[i].dyn_scale for i in part], [layers[i].w_scale for i in part],
                                  [ys[i] for i in part], None, stream)
    return ys


class PhasedBlock:
    """A block's projections split into phases that share no input, run on
    two streams: each phase's preparation (statistics of its inputs and
    weights, smoothing factors, weight and activation codes) on `prep`, its
    products on `gemm` once that preparation is done. The HBM-bound
    preparation of phase i + 1 thereby runs beside the products of phase i,
    and the next pass's phase i beside this pass's later products: a phase's
    preparation waits only for the products of the same phase in the previous
    pass (the last readers of its buffers).

    phases: list of (layers, calib, xs) as for prepare_block / forward_block;
    layers of different phases must not share act_max tensors or inputs that
    a phase writes."""

    def __init__(self, phases):
        self.phases = phases
        self.done = [None] * len(phases)

    def step(self, prep, gemm, on_gemm=None):
        """Enqueue one pass. on_gemm(i, before): called with before=True just
        before phase i's product launch is enqueued on `gemm` and with
        before=False just after (for timing events). Returns the outputs."""
        import torch
        outs = []
        for i, (layers, calib, xs) in enumerate(self.phases):
            if self.done[i] is not None:
                prep.wait_event(self.done[i])
            prepare_block(layers, calib, prep)
            ready = torch.cuda.Event()

            def between(i=i, ready=ready):
                ready.record(prep)
                gemm.wait_event(ready)
                if on_gemm is not None:
                    on_gemm(i, True)

            outs += forward_block(layers, xs, prep, gemm, between)
            if on_gemm is not None:
                on_gemm(i, False)
            done = torch.cuda.Event()
            done.record(gemm)
            self.done[i] = done
        return outs
