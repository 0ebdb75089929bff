"""Benchmark: one MoE/linear layer step (quantization + grouped GEMMs) on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic inputs
already resident in HBM: every quantization call and grouped GEMM of the
layer's forward, dgrad and wgrad, in the order a training step issues them,
on preallocated buffers (no allocation, no host sync inside the step).

Default workload: the dense Llama3-8B-shaped linear (X [8192, 4096], W [14336,
4096], dY [8192, 14336]; E = 1), FP8 rowwise recipe with colwise-quantized
backward operands and FP8 wgrad.  --config selects the other workloads:
1 tiny MoE (fwd only), 3 DeepSeek-MoE-16B-shaped layer, 4 DeepSeek-V3-shaped
one-GPU expert share, 5 Llama4-Scout-shaped MXFP8 layer; --gw adds the BF16
weight-gradient variant of config 2 as its own line item.

Prints ONE JSON line.  `value` is microseconds per layer step (lower is
better).  Every input has 4 device copies and step s reads copy s % 4, so no
step finds its inputs in the 256 MB last-level cache (reuse between launches
inside a step stays).  Also reported: aggregate quantization GB/s (algorithmic
bytes: 2 B read + 1 B written per element + scale bytes), aggregate GEMM
TFLOP/s (2 * sum_e M_e * N * K), per-kernel averages from HIP events on the
launch stream over the timed steps, the roofline of the dominant kernel, each
launch alone after a 1 GiB cache-evicting read (median, p10, p90 of 20
repeats after 5 warm-ups), the peaks used, the shader clock rocm-smi reports
while untimed steps run, and the CPU oracle timed on a bounded sample of the
same workload (a reported baseline, not a target).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E
PEAK_FP8_TFLOPS = 5000.0       # dense FP8 / MXFP8 MFMA
PEAK_BF16_TFLOPS = 2500.0      # dense bf16 MFMA


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=5, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--gw", action="store_true", help="config 2: add the BF16 wgrad variant")
    ap.add_argument("--experts-only", action="store_true",
                    help="configs 3-5: time only the expert GEMMs and their quantizations (synthetic operands), "
                         "not the whole MoE layer")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--swiglu", action="store_true",
                    help="configs 3/4: also time the fused SwiGLU + rowwise quantization (forward and backward) "
                         "on the layer's A2/dH1 shapes, outside the layer step")
    ap.add_argument("--tensorwise", action="store_true",
                    help="config 2: the tensorwise recipe (one scale per tensor for X, W and dY) in place of "
                         "rowwise + colwise")
    ap.add_argument("--blockwise", action="store_true",
                    help="config 2: also time the blockwise recipe's launches (1x128 / 128x128 tiles, 128-token "
                         "blocks for the weight gradient, the three blockwise GEMMs) outside the layer step")
    ap.add_argument("--route", action="store_true",
                    help="configs 3/4: also time the routing kernels (route, permute of X into the grouped layout, "
                         "combine of the grouped output) on the layer's routing and hidden size, outside the layer step")
    ap.add_argument("--no-per-kernel", action="store_true",
                    help="skip the flushed per-kernel pass and the clock sample (kernel traces of the steps alone)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (calibrates HBM byte counters)")
    ap.add_argument("--only", default=None, metavar="ITEM",
                    help="profiling aid: warm up the whole step, then time only launch ITEM (e.g. 'gemm fwd'), "
                         "after a marker kernel so counter passes can isolate its dispatches")
    ap.add_argument("--write-traffic", nargs=4, default=None,
                    metavar=("FETCH_DB", "WRITE_DB", "COPY_FETCH_DB", "COPY_WRITE_DB"),
                    help="write profiles/traffic.json for --only ITEM of --config from rocprofv3 --pmc "
                         "FETCH_SIZE / WRITE_SIZE databases of an --only run and of a --copy-probe run")
    ap.add_argument("--copy-mib", type=int, default=512, help="size of the --copy-probe run behind the calibration")
    return ap.parse_args()


# ---------------------------------------------------------------------- layer plan

def progress(msg: str) -> None:
    """A progress line on stderr (stdout carries only the JSON result)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


N_ROTATE = 4   # device copies of every input; step s reads copy s % N_ROTATE


class Step:
    """A list of launches; each item: (name, kind, fn, work, hbm) with kind 'quant' (work = hbm =
    algorithmic bytes) or 'gemm' / 'gemm_bf16' (work = flops, hbm = algorithmic bytes: operands and
    scales read once, output written once).  Launches read their inputs through getters that pick
    copy `rot[0]`, so consecutive steps read inputs that the caches do not hold.  `specs[name]`
    says what a launch computes (operation, named host inputs, device outputs), so a parity test
    can check every launch of exactly this step against the oracle."""

    def __init__(self):
        self.items = []
        self.rot = [0]
        self.specs = {}
        self.outputs = {}

    def add(self, name, kind, fn, work, hbm=None, spec=None):
        self.items.append((name, kind, fn, work, work if hbm is None else hbm))
        if spec is not None:
            self.specs[name] = spec

    def run(self):
        for it in self.items:
            it[2]()


def build_step(cfg: int, gw: bool, tensorwise: bool = False, n_rotate: int = N_ROTATE, keep_host: bool = False,
               dev: str = "cuda:0", experts_only: bool = False):
    """The layer step of workload `cfg` on preallocated device buffers.  Returns (step, host): host
    holds the bf16 inputs as numpy bit patterns (X, DY and W always; with keep_host every input,
    named as in Step.specs).

    For the MoE workloads (3, 4, 5) the step is the whole MoE layer, forward and backward, from
    the tokens' expert ids to the tokens' input gradient (see moe_layer below); experts_only keeps
    only the expert GEMMs and their quantizations, on synthetic inputs for every operand."""
    import torch
    import mxfp8_quantized_moe_amd as fm
    from mxfp8_quantized_moe_amd import synth

    w = synth.WORKLOADS[cfg]

    def dv(bits):
        """n_rotate device copies of a bf16 input; returns a getter of the current one."""
        t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)
        copies = [t] + [t.clone() for _ in range(n_rotate - 1)]
        return lambda: copies[step.rot[0]]

    u8 = lambda *s: torch.empty(s, dtype=torch.uint8, device=dev)
    f32 = lambda *s: torch.empty(s, dtype=torch.float32, device=dev)
    bf = lambda *s: torch.empty(s, dtype=torch.bfloat16, device=dev)
    step = Step()
    host = {}

    E, M, H = w.E, w.M, w.H
    offs_np = w.offs
    offs = torch.from_numpy(offs_np.astype(np.int32)).to(dev)
    counts = np.diff(np.concatenate([[0], offs_np]))
    nonempty = int((counts > 0).sum())

    def qbytes(n_elem, n_scale, scale_bytes=4):
        return 3 * n_elem + scale_bytes * n_scale

    def q_row(name, src, x, rows, cols):
        q, s = u8(rows, cols), f32(rows)
        step.add(name, "quant", lambda: fm.quantize_rowwise(x().view(rows, cols), 0, q=q, scale=s),
                 qbytes(rows * cols, rows), spec=dict(op="q_row", src=src, shape=(rows, cols), q=q, s=s))
        return q, s

    def q_col_grouped(name, src, x, rows, cols):
        ld = (rows + 15) // 16 * 16
        q, s = u8(cols, ld), f32(E, cols)
        step.add(name, "quant", lambda: fm.quantize_colwise(x(), offs, 0, q_t=q, scale=s, ld_q=ld),
                 qbytes(rows * cols, E * cols), spec=dict(op="q_col_grouped", src=src, offs=offs_np, q=q, s=s))
        return q, s, ld

    def q_col_batched(name, src, x, B, R, C):
        q, s = u8(B, C, R), f32(B, C)
        step.add(name, "quant", lambda: fm.quantize_colwise(x(), None, 0, q_t=q, scale=s, ld_q=R),
                 qbytes(B * R * C, B * C), spec=dict(op="q_col_batched", src=src, shape=(B, R, C), q=q, s=s))
        return q, s

    def gemm_bytes(a_elems, b_elems, out_elems, a_rows, b_rows, sk):
        # fp8 operands + bf16 output; fp32 scales per row (per group row for the weight side) or
        # one e8m0 byte per 32 operand bytes
        sc = (a_elems + b_elems) / 32 if sk in (fm.SCALE_E8M0, fm.SCALE_E8M0_K4) else 4 * (a_rows + b_rows)
        return a_elems + b_elems + 2 * out_elems + sc

    def g_m(name, qa, sa, qb, sb, Mr, N, K, sk=fm.SCALE_F32):
        # the weight operand of an expert with no rows is never read: only non-empty experts count
        o = bf(Mr, N)
        step.add(name, "gemm", lambda: fm.grouped_mm_scaled(fm.GROUPED_M, qa, 0, sa, qb, 0, sb, sk, offs, E,
                                                            Mr, N, K, out=o), 2.0 * M * N * K,
                 gemm_bytes(M * K, nonempty * N * K, M * N, M, nonempty * N, sk),
                 spec=dict(op="g_m", qa=qa, sa=sa, qb=qb, sb=sb, sk=sk, offs=offs_np, M=Mr, N=N, K=K, out=o))
        return o

    def g_k(name, qa, sa, qb, sb, Mc, N, K, sk=fm.SCALE_F32, offs_t=None):
        o = bf(E, N, K)
        og = offs if offs_t is None else offs_t
        step.add(name, "gemm", lambda: fm.grouped_mm_scaled(fm.GROUPED_K, qa, 0, sa, qb, 0, sb, sk, og, E,
                                                            Mc, N, K, out=o), 2.0 * M * N * K,
                 gemm_bytes(N * M, K * M, E * N * K, E * N, E * K, sk),
                 spec=dict(op="g_k", qa=qa, sa=sa, qb=qb, sb=sb, sk=sk, offs=offs_np if offs_t is None else offs_t,
                           M=Mc, N=N, K=K, out=o))
        return o

    # MXFP8: e8m0 scales written by the quantizer in the K4 layout the GEMM reads per stage
    rule = fm.MX_FLOOR_OCP
    Mp = fm.quantize_mx_rows_bound(M, E)
    K4 = fm.MX_LAYOUT_K4

    def mx_last(name, src, x, rows, cols):
        q, s = u8(rows, cols), u8(*fm.mx_k4_shape(rows, cols // 32))
        step.add(name, "quant", lambda: fm.quantize_mx(x().view(rows, cols), axis=1, rule=rule, q=q, scale=s,
                                                       layout=K4),
                 qbytes(rows * cols, rows * cols // 32, 1),
                 spec=dict(op="mx_last", src=src, shape=(rows, cols), rule=rule, q=q, s=s))
        return q, s

    def mx_rows_b(name, src, x, B, R, C):
        q, s = u8(B, C, R), u8(*fm.mx_k4_shape(B * C, R // 32))
        step.add(name, "quant", lambda: fm.quantize_mx(x(), axis=0, rule=rule, q=q, scale=s, layout=K4),
                 qbytes(B * R * C, B * C * R // 32, 1),
                 spec=dict(op="mx_rows_b", src=src, shape=(B, R, C), rule=rule, q=q, s=s))
        return q, s

    op = torch.empty(E, dtype=torch.int32, device=dev)

    def mx_rows_g(name, src, x, rows, cols):
        q, s = u8(cols, Mp), u8(*fm.mx_k4_shape(cols, Mp // 32))
        step.add(name, "quant", lambda: fm.quantize_mx(x(), axis=0, offs=offs, rule=rule, rows_pad=Mp, q=q, scale=s,
                                                       offs_pad=op, layout=K4),
                 qbytes(rows * cols, cols * rows // 32, 1),
                 spec=dict(op="mx_rows_g", src=src, offs=offs_np, rows_pad=Mp, rule=rule, q=q, s=s, offs_pad=op))
        return q, s

    def mx_dual_b(name, src, x, B, R, C):
        """Both MX forms of a batched tensor (weights) from one read."""
        q, s = u8(B * R, C), u8(*fm.mx_k4_shape(B * R, C // 32))
        qt, st = u8(B, C, R), u8(*fm.mx_k4_shape(B * C, R // 32))
        step.add(name, "quant", lambda: fm.quantize_mx_dual(x(), rule=rule, q=q, scale=s, q_t=qt, scale_t=st, layout=K4),
                 4 * B * R * C + 2 * (B * R * C // 32),
                 spec=dict(op="mx_dual", src=src, shape=(B, R, C), rule=rule, q=q, s=s, qt=qt, st=st))
        return q, s, qt, st

    def mx_dual_g(name, src, x, rows, cols):
        """Both MX forms of a grouped tensor (activations) from one read; row blocks padded per group."""
        q, s = u8(rows, cols), u8(*fm.mx_k4_shape(rows, cols // 32))
        qt, st = u8(cols, Mp), u8(*fm.mx_k4_shape(cols, Mp // 32))
        step.add(name, "quant", lambda: fm.quantize_mx_dual(x(), offs=offs, rule=rule, rows_pad=Mp, q=q, scale=s,
                                                            q_t=qt, scale_t=st, offs_pad=op, layout=K4),
                 4 * rows * cols + 2 * (rows * cols // 32),
                 spec=dict(op="mx_dual", src=src, shape=(rows, cols), offs=offs_np, rows_pad=Mp, rule=rule, q=q, s=s,
                           qt=qt, st=st, offs_pad=op))
        return q, s, qt, st

    def moe_layer():
        """The MoE layer as one stream-ordered step with no host synchronisation [P1 Details, MoE
        paragraph; P4 "MoE"]: route the tokens' expert ids into offsets, gather the token rows into
        the grouped layout (with the FP8 rowwise recipe quantized in the same pass), W1, SwiGLU
        (fused with the next quantization), W2, the weighted combine back to tokens; then the
        mirror backward: combine's backward (routed-row gradients, fused with their rowwise
        quantization, and the router weights' gradients), dgrad and wgrad of W2, SwiGLU's backward,
        dgrad and wgrad of W1, and the sum of each token's routed input gradients.  Every GEMM
        reads the device-computed offsets; intermediate tensors are the previous launches' own
        outputs.  Kind 'moe' marks the memory-bound launches that are not quantizations alone."""
        nonlocal offs
        F, F2 = w.F, w.F2
        T, k = synth.tokens_topk(cfg)
        ids, RW = synth.routing_ids(cfg), synth.router_weights(cfg)
        S = T * k
        rows = fm.moe_route_rows_bound(S, E, 1)
        assert rows == M, "the routing reproduces the workload's routed rows"
        import concurrent.futures as cf
        with cf.ThreadPoolExecutor(4) as ex:
            X, DY, W1, W2 = ex.map(lambda f: f(w), [synth.make_tokens, synth.make_dy_tokens, synth.make_w1,
                                                    synth.make_w2])
        host.update(X=X, DY=DY, W=W1.reshape(E * F2, H), IDS=ids, RW=RW)
        if keep_host:
            host.update(W1=W1, W2=W2)
        Xd, DYd, W1d, W2d = dv(X), dv(DY), dv(W1), dv(W2)
        idsd = torch.from_numpy(ids).to(dev)
        rwd = torch.from_numpy(RW).to(dev)
        i32 = lambda n: torch.empty(n, dtype=torch.int32, device=dev)
        r_counts, r_offs, r_dest, r_src = i32(E), i32(E), i32(S), i32(rows)
        ws = u8(max(fm.moe_route_workspace_bytes(S, E), 1))
        offs = r_offs                        # every launch below reads the routed offsets
        step.add("route", "moe",
                 lambda: fm.moe_route(idsd, E, 1, out=(r_counts, r_offs, r_dest, r_src), workspace=ws),
                 4 * S + 4 * S + 4 * rows + 8 * E,
                 spec=dict(op="route", ids="IDS", E=E, pad=1, out=(r_counts, r_offs, r_dest, r_src)))
        def mx_gather(name, x, x_name, wts, w_name):
            """Both MX forms of the token rows x gathered into the grouped layout (times the router
            weights when given) in one launch: the gathered tensor never goes to memory."""
            q, s = u8(rows, H), u8(*fm.mx_k4_shape(rows, H // 32))
            qt, st = u8(H, Mp), u8(*fm.mx_k4_shape(H, Mp // 32))
            step.add(name, "quant",
                     lambda: fm.moe_permute_quantize_mx_dual(x(), r_src, k, offs, weights=wts, rule=rule,
                                                             rows_pad=Mp, q=q, scale=s, q_t=qt, scale_t=st,
                                                             offs_pad=op, layout=K4),
                     2 * T * H + 2 * rows * H + 2 * (rows * H // 32) + 4 * rows + (4 * S if wts is not None else 0),
                     spec=dict(op="permute_mx_dual", x=x_name, rsrc=r_src, dest=r_dest, topk=k, w=w_name,
                               shape=(rows, H), offs=offs_np, rows_pad=Mp, rule=rule, q=q, s=s, qt=qt, st=st,
                               offs_pad=op))
            return q, s, qt, st

        xg = dyg = None                      # the gathered bf16 rows: neither recipe forms them in memory

        def q_col_gathered(name, x, x_name, wts, w_name):
            """The colwise quantization of the token rows x gathered into the grouped layout (times the
            router weights when given): the gathered rows are formed at load time."""
            ld = (rows + 15) // 16 * 16
            q, s = u8(H, ld), f32(E, H)
            step.add(name, "quant",
                     lambda: fm.moe_permute_quantize_colwise(x(), r_src, k, offs, weights=wts, codec=0, q_t=q,
                                                             scale=s, ld_q=ld),
                     2 * T * H + rows * H + 4 * E * H + 4 * rows + (4 * S if wts is not None else 0),
                     spec=dict(op="permute_q_col", x=x_name, rsrc=r_src, dest=r_dest, topk=k, w=w_name, offs=offs_np,
                               q=q, s=s))
            return q, s, ld

        if w.mx:
            qx, sx, qxt, sxt = mx_gather("permute+mx Xg (both forms)", Xd, "X", None, None)
            qw1, sw1, qw1t, sw1t = mx_dual_b("mx W1 (both forms)", "W1", W1d, E, F2, H)
            h1 = g_m("gemm fwd W1", qx, sx, qw1, sw1, rows, F2, H, sk=fm.SCALE_E8M0_K4)
        else:
            # the gathered rows' bf16 copy is not kept: the weight gradient's colwise operand is gathered again
            qx, sx = u8(rows, H), f32(rows)
            step.add("permute+q X", "moe",
                     lambda: fm.moe_permute_rowwise(Xd(), r_src, k, 0, keep_bf16=False, qg=qx, scale_g=sx),
                     3 * rows * H + 8 * rows,
                     spec=dict(op="permute_rowwise", src="X", topk=k, rsrc=r_src, xg=None, q=qx, s=sx))
            qw1, sw1 = q_row("q_row W1", "W1", W1d, E * F2, H)
            h1 = g_m("gemm fwd W1", qx, sx, qw1, sw1, rows, F2, H)
        if w.mx:
            # SwiGLU computed inside the quantizer: A2 itself never goes to memory
            qa2, sa2 = u8(rows, F), u8(*fm.mx_k4_shape(rows, F // 32))
            qa2t, sa2t = u8(F, Mp), u8(*fm.mx_k4_shape(F, Mp // 32))
            step.add("swiglu+mx A2 (both forms)", "quant",
                     lambda: fm.swiglu_quantize_mx_dual(h1, offs, rule=rule, rows_pad=Mp, q=qa2, scale=sa2, q_t=qa2t,
                                                        scale_t=sa2t, offs_pad=op, layout=K4),
                     2 * rows * F2 + 2 * rows * F + 2 * (rows * F // 32),
                     spec=dict(op="swiglu_mx", h1=h1, da2=None, F=F, offs=offs_np, rows_pad=Mp, rule=rule, q=qa2,
                               s=sa2, qt=qa2t, st=sa2t, offs_pad=op))
            qw2, sw2, qw2t, sw2t = mx_dual_b("mx W2 (both forms)", "W2", W2d, E, H, F)
            yg = g_m("gemm fwd W2", qa2, sa2, qw2, sw2, rows, H, F, sk=fm.SCALE_E8M0_K4)
        else:
            a2 = bf(rows, F)
            qa2, sa2 = u8(rows, F), f32(rows)
            step.add("swiglu+q", "moe", lambda: fm.swiglu_quantize_rowwise(h1, 0, a2=a2, q=qa2, scale=sa2),
                     2 * rows * F2 + 3 * rows * F + 4 * rows,
                     spec=dict(op="swiglu", h1=h1, F=F, a2=a2, q=qa2, s=sa2))
            qw2, sw2 = q_row("q_row W2", "W2", W2d, E * H, F)
            yg = g_m("gemm fwd W2", qa2, sa2, qw2, sw2, rows, H, F)
        y = bf(T, H)
        step.add("combine", "moe", lambda: fm.moe_combine(yg, r_dest, rwd, k, y=y), 2 * S * H + 2 * T * H + 8 * S,
                 spec=dict(op="combine", yg=yg, dest=r_dest, w="RW", topk=k, out=y))
        # backward
        dw = f32(S)
        if w.mx:
            # the router weights' gradients only; the routed-row gradients are formed inside the quantizer
            step.add("combine bwd (dw)", "moe",
                     lambda: fm.moe_combine_backward(DYd(), yg, r_dest, r_src, rwd, k, 0, codes=False,
                                                     rows_out=False, dweights=dw),
                     2 * T * H + 2 * rows * H + 16 * S,
                     spec=dict(op="combine_bwd", dy="DY", yg=yg, dest=r_dest, src=r_src, w="RW", topk=k, dyg=None,
                               q=None, s=None, dw=dw))
            qdy, sdy, qdyt, sdyt = mx_gather("permute+mx dYg (both forms)", DYd, "DY", rwd, "RW")
            da2 = g_m("gemm dgrad W2", qdy, sdy, qw2t, sw2t, rows, F, H, sk=fm.SCALE_E8M0_K4)
            g_k("gemm wgrad W2", qdyt, sdyt, qa2t, sa2t, Mp, H, F, sk=fm.SCALE_E8M0_K4, offs_t=op)
        else:
            # routed-row gradients quantized rowwise in the combine backward; their colwise operand is
            # gathered from dY again, so the grouped bf16 dYg never goes to memory
            qdy, sdy = u8(rows, H), f32(rows)
            step.add("combine bwd+q", "moe",
                     lambda: fm.moe_combine_backward(DYd(), yg, r_dest, r_src, rwd, k, 0, rows_out=False, q=qdy,
                                                     scale=sdy, dweights=dw),
                     2 * T * H + 3 * rows * H + 4 * rows + 16 * S,
                     spec=dict(op="combine_bwd", dy="DY", yg=yg, dest=r_dest, src=r_src, w="RW", topk=k, dyg=None,
                               q=qdy, s=sdy, dw=dw))
            qw2t, sw2t = q_col_batched("q_col W2", "W2", W2d, E, H, F)
            da2 = g_m("gemm dgrad W2", qdy, sdy, qw2t, sw2t, rows, F, H)
            qdyt, sdyt, ld = q_col_gathered("q_col dYg (gathered)", DYd, "DY", rwd, "RW")
            qa2t, sa2t, _ = q_col_grouped("q_col A2", a2, lambda: a2, rows, F)
            g_k("gemm wgrad W2", qdyt, sdyt, qa2t, sa2t, ld, H, F)
        if w.mx:
            qdh, sdh = u8(rows, F2), u8(*fm.mx_k4_shape(rows, F2 // 32))
            qdht, sdht = u8(F2, Mp), u8(*fm.mx_k4_shape(F2, Mp // 32))
            step.add("swiglu bwd+mx dH1 (both forms)", "quant",
                     lambda: fm.swiglu_backward_quantize_mx_dual(da2, h1, offs, rule=rule, rows_pad=Mp, q=qdh,
                                                                 scale=sdh, q_t=qdht, scale_t=sdht, offs_pad=op,
                                                                 layout=K4),
                     2 * rows * F + 2 * rows * F2 + 2 * rows * F2 + 2 * (rows * F2 // 32),
                     spec=dict(op="swiglu_mx", h1=h1, da2=da2, F=F, offs=offs_np, rows_pad=Mp, rule=rule, q=qdh,
                               s=sdh, qt=qdht, st=sdht, offs_pad=op))
            dxg = g_m("gemm dgrad W1", qdh, sdh, qw1t, sw1t, rows, H, F2, sk=fm.SCALE_E8M0_K4)
            g_k("gemm wgrad W1", qdht, sdht, qxt, sxt, Mp, F2, H, sk=fm.SCALE_E8M0_K4, offs_t=op)
        else:
            dh1 = bf(rows, F2)
            qdh, sdh = u8(rows, F2), f32(rows)
            step.add("swiglu bwd+q", "moe",
                     lambda: fm.swiglu_backward_quantize_rowwise(da2, h1, 0, dh1=dh1, q=qdh, scale=sdh),
                     2 * rows * F + 5 * rows * F2 + 4 * rows,
                     spec=dict(op="swiglu_bwd", da2=da2, h1=h1, F=F, dh1=dh1, q=qdh, s=sdh))
            qw1t, sw1t = q_col_batched("q_col W1", "W1", W1d, E, F2, H)
            dxg = g_m("gemm dgrad W1", qdh, sdh, qw1t, sw1t, rows, H, F2)
            qdht, sdht, _ = q_col_grouped("q_col dH1", dh1, lambda: dh1, rows, F2)
            qxt, sxt, _ = q_col_gathered("q_col Xg (gathered)", Xd, "X", None, None)
            g_k("gemm wgrad W1", qdht, sdht, qxt, sxt, ld, F2, H)
        dx = bf(T, H)
        step.add("combine dX", "moe", lambda: fm.moe_combine(dxg, r_dest, None, k, y=dx), 2 * S * H + 2 * T * H + 4 * S,
                 spec=dict(op="combine", yg=dxg, dest=r_dest, w=None, topk=k, out=dx))
        step.outputs = dict(y=y, dx=dx, dw=dw, xg=xg, h1=h1, yg=yg, dyg=dyg, da2=da2, dxg=dxg,
                            route=(r_counts, r_offs, r_dest, r_src))
        return step, host

    if cfg in (3, 4, 5) and not experts_only:
        return moe_layer()

    if cfg == 2 and tensorwise:
        # one scale per tensor: each of X, W, dY quantized once into both layouts, its scale broadcast
        # into a vector long enough for both of its GEMM uses; the GEMM launches are the rowwise ones
        F2 = w.F2
        X, W1, DY = synth.make_x(w), synth.make_w1(w), synth.make_dy(w)
        host.update(X=X, W=W1.reshape(F2, H), DY=DY)
        Xd, Wd, DYd = dv(X), dv(W1), dv(DY)

        def q_tw(name, x, R, C):
            ld = (R + 15) // 16 * 16
            q, qt, sc, ws = u8(R, C), u8(1, C, ld), f32(max(R, C)), u8(4096)
            step.add(name, "quant", lambda: fm.quantize_tensorwise(x().view(R, C), 0, rowmajor=True, transposed=True,
                                                                   ld_q=ld, n_scale=max(R, C), q=q, q_t=qt, scale=sc,
                                                                   workspace=ws),
                     4 * R * C + 4 * max(R, C))   # read once, both layouts written, the scale vector
            return q, qt.view(C, ld), sc, ld

        qx, qxt, sx, ld = q_tw("q_tw X", Xd, M, H)
        qw, qwt, sw, _ = q_tw("q_tw W", Wd, F2, H)
        g_m("gemm fwd", qx, sx, qw, sw, M, F2, H)
        qdy, qdyt, sdy, _ = q_tw("q_tw dY", DYd, M, F2)
        g_m("gemm dgrad", qdy, sdy, qwt.view(1, H, F2), sw, M, H, F2)
        g_k("gemm wgrad", qdyt, sdy, qxt, sx, ld, F2, H)
        return step, host

    if cfg in (1, 2):
        F2 = w.F2
        X, W1 = synth.make_x(w), synth.make_w1(w)
        host.update(X=X, W=W1.reshape(E * F2, H), W1=W1)
        Xd, Wd = dv(X), dv(W1)
        qx, sx = q_row("q_row X", "X", Xd, M, H)
        qw, sw = q_row("q_row W", "W1", Wd, E * F2, H)
        g_m("gemm fwd", qx, sx, qw, sw, M, F2, H)
        if cfg == 2:
            DY = synth.make_dy(w)
            host.update(DY=DY)
            DYd = dv(DY)
            qdy, sdy = q_row("q_row dY", "DY", DYd, M, F2)
            qwt, swt = q_col_batched("q_col W", "W1", Wd, 1, F2, H)
            g_m("gemm dgrad", qdy, sdy, qwt, swt, M, H, F2)
            qdyt, sdyt, ld = q_col_grouped("q_col dY", "DY", DYd, M, F2)
            qxt, sxt, _ = q_col_grouped("q_col X", "X", Xd, M, H)
            g_k("gemm wgrad", qdyt, sdyt, qxt, sxt, ld, F2, H)
            if gw:
                o = bf(1, F2, H)
                step.add("gemm wgrad bf16", "gemm_bf16",
                         lambda: fm.grouped_mm_scaled(fm.GROUPED_K, DYd(), fm.OPD_BF16, None, Xd(), fm.OPD_BF16, None,
                                                      fm.SCALE_NONE, offs, 1, M, F2, H, out=o), 2.0 * M * F2 * H,
                         2 * (M * F2 + M * H + F2 * H),
                         spec=dict(op="g_k_bf16", a="DY", b="X", offs=offs_np, out=o))
        return step, host

    F, F2 = w.F, w.F2
    import concurrent.futures as cf
    with cf.ThreadPoolExecutor(6) as ex:      # independent seeded streams: the values do not depend on this
        X, A2, DY, DH1, W1, W2 = ex.map(lambda f: f(w), [synth.make_x, synth.make_a2, synth.make_dy,
                                                         synth.make_dh1, synth.make_w1, synth.make_w2])
    host.update(X=X, W=W1.reshape(E * F2, H), DY=DY)
    if keep_host:
        host.update(A2=A2, DH1=DH1, W1=W1, W2=W2)
    Xd, A2d, DYd, DH1d, W1d, W2d = dv(X), dv(A2), dv(DY), dv(DH1), dv(W1), dv(W2)
    del W1, W2
    if cfg in (3, 4):
        qx, sx = q_row("q_row X", "X", Xd, M, H)
        qw1, sw1 = q_row("q_row W1", "W1", W1d, E * F2, H)
        g_m("gemm fwd W1", qx, sx, qw1, sw1, M, F2, H)
        qa2, sa2 = q_row("q_row A2", "A2", A2d, M, F)
        qw2, sw2 = q_row("q_row W2", "W2", W2d, E * H, F)
        g_m("gemm fwd W2", qa2, sa2, qw2, sw2, M, H, F)
        qdy, sdy = q_row("q_row dY", "DY", DYd, M, H)
        qw2t, sw2t = q_col_batched("q_col W2", "W2", W2d, E, H, F)
        g_m("gemm dgrad W2", qdy, sdy, qw2t, sw2t, M, F, H)
        qdyt, sdyt, ld = q_col_grouped("q_col dY", "DY", DYd, M, H)
        qa2t, sa2t, _ = q_col_grouped("q_col A2", "A2", A2d, M, F)
        g_k("gemm wgrad W2", qdyt, sdyt, qa2t, sa2t, ld, H, F)
        qdh, sdh = q_row("q_row dH1", "DH1", DH1d, M, F2)
        qw1t, sw1t = q_col_batched("q_col W1", "W1", W1d, E, F2, H)
        g_m("gemm dgrad W1", qdh, sdh, qw1t, sw1t, M, H, F2)
        qdht, sdht, _ = q_col_grouped("q_col dH1", "DH1", DH1d, M, F2)
        qxt, sxt, _ = q_col_grouped("q_col X", "X", Xd, M, H)
        g_k("gemm wgrad W1", qdht, sdht, qxt, sxt, ld, F2, H)
        return step, host

    # cfg 5: MXFP8
    qx, sx = mx_last("mx X", "X", Xd, M, H)
    qw1, sw1 = mx_last("mx W1", "W1", W1d, E * F2, H)
    g_m("gemm fwd W1", qx, sx, qw1, sw1, M, F2, H, sk=fm.SCALE_E8M0_K4)
    qa2, sa2 = mx_last("mx A2", "A2", A2d, M, F)
    qw2, sw2 = mx_last("mx W2", "W2", W2d, E * H, F)
    g_m("gemm fwd W2", qa2, sa2, qw2, sw2, M, H, F, sk=fm.SCALE_E8M0_K4)
    qdy, sdy = mx_last("mx dY", "DY", DYd, M, H)
    qw2t, sw2t = mx_rows_b("mx W2^T", "W2", W2d, E, H, F)
    g_m("gemm dgrad W2", qdy, sdy, qw2t, sw2t, M, F, H, sk=fm.SCALE_E8M0_K4)
    qdyt, sdyt = mx_rows_g("mx dY^T", "DY", DYd, M, H)
    qa2t, sa2t = mx_rows_g("mx A2^T", "A2", A2d, M, F)
    g_k("gemm wgrad W2", qdyt, sdyt, qa2t, sa2t, Mp, H, F, sk=fm.SCALE_E8M0_K4, offs_t=op)
    qdh, sdh = mx_last("mx dH1", "DH1", DH1d, M, F2)
    qw1t, sw1t = mx_rows_b("mx W1^T", "W1", W1d, E, F2, H)
    g_m("gemm dgrad W1", qdh, sdh, qw1t, sw1t, M, H, F2, sk=fm.SCALE_E8M0_K4)
    qdht, sdht = mx_rows_g("mx dH1^T", "DH1", DH1d, M, F2)
    qxt, sxt = mx_rows_g("mx X^T", "X", Xd, M, H)
    g_k("gemm wgrad W1", qdht, sdht, qxt, sxt, Mp, F2, H, sk=fm.SCALE_E8M0_K4, offs_t=op)
    return step, host


# ---------------------------------------------------------------------- CPU oracle baseline

def cpu_model():
    """The host CPU's model name (lscpu), or None."""
    import subprocess
    try:
        r = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=30)
        for line in r.stdout.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except Exception:
        return None
    return None


def _k4_rows(k4, R, NB):
    """e8m0 scales in the K4 layout [ceil(NB/4), R, 4] as row-major [R, NB] (a layout change only)."""
    return np.ascontiguousarray(k4.transpose(1, 0, 2).reshape(R, 4 * k4.shape[0])[:, :NB])


def cpu_baseline(step, host: dict):
    """The oracle timed on a bounded sample of every launch of the step, each scaled linearly to its
    full size (us per layer step):
      * quantization: a slice of whole rows (rowwise, MX last-dim blocks) or whole columns (colwise,
        MX row blocks) of about 2M elements, single-threaded numpy;
      * GEMMs: a block of up to 1024 output rows x 4096 output columns of the largest group, over the
        whole contraction, on the step's own operands copied to the host, fp64 BLAS; scaled by flops;
      * the MoE layer's routing (whole), gathers, SwiGLU and combines: about 2M output elements of
        whole rows (tokens for the combines), single-threaded numpy.
    Inputs that the step computes (the MoE layer's intermediate tensors) are copied from the device
    as the last step left them."""
    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits
    total_us = 0.0
    pieces = []
    QS = 1 << 21

    def timed(fn, threads=None):
        if threads == 1:
            with threadpool_limits(1):
                t0 = time.perf_counter()
                fn()
                return time.perf_counter() - t0
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    def add(name, secs, factor):
        nonlocal total_us
        total_us += secs * factor * 1e6
        pieces.append(f"{name} x{factor:.0f}")

    def h(t):
        import torch
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).cpu().numpy().view(np.uint16)
        return t.cpu().numpy()

    dev_cache = {}

    def src(name):
        if not isinstance(name, str):               # a device tensor the step computes
            if id(name) not in dev_cache:
                dev_cache[id(name)] = h(name)
            return dev_cache[id(name)]
        return host["W1"] if name == "W1" else host[name]

    from oracle import route as o_route, swiglu as o_swiglu

    def gathered(sp, x, s_rows, cols):
        """The oracle's gather of rows s_rows (first `cols` columns) of the token rows x, or with router
        weights the routed-row gradients of its combine backward."""
        xs, k = np.ascontiguousarray(x[:, :cols]), sp["topk"]
        if sp["w"] is None:
            return o_route.permute(xs, s_rows, k)
        T = x.shape[0]
        return o_route.combine_backward(xs, np.zeros((s_rows.size, cols), np.uint16), s_rows,
                                        np.full(T * k, -1, np.int32), host[sp["w"]], T, k)[0]

    for name, kind, *_ in step.items:
        sp = step.specs.get(name)
        if sp is None:
            continue
        op = sp["op"]
        if op in ("q_row", "mx_last"):
            R, C = sp["shape"]
            x = src(sp["src"]).reshape(R, C)
            r = max(1, min(R, QS // max(C, 1)))
            f = (lambda: oracle.quantize_rowwise(x[:r], 0)) if op == "q_row" else \
                (lambda: oracle.quantize_mx_lastdim(x[:r], sp["rule"]))
            add(name, timed(f, 1), R / r)
        elif op in ("q_col_grouped", "mx_rows_g"):
            x = src(sp["src"])
            M, C = x.shape
            c = max(8, min(C, QS // max(M, 1)) // 8 * 8)
            xs = np.ascontiguousarray(x[:, :c])
            f = (lambda: oracle.quantize_colwise_grouped(xs, sp["offs"], 0)) if op == "q_col_grouped" else \
                (lambda: oracle.quantize_mx_rows_grouped(xs, sp["offs"], sp["rule"], sp["rows_pad"]))
            add(name, timed(f, 1), C / c)
        elif op in ("q_col_batched", "mx_rows_b"):
            B, R, C = sp["shape"]
            x = src(sp["src"]).reshape(B, R, C)
            c = max(8, min(C, QS // max(B * R, 1)) // 8 * 8)
            xs = np.ascontiguousarray(x[:, :, :c])
            f = (lambda: oracle.quantize_colwise_batched(xs, 0)) if op == "q_col_batched" else \
                (lambda: oracle.quantize_mx_rows_batched(xs, sp["rule"]))
            add(name, timed(f, 1), C / c)
        elif op == "g_m":
            M, N, K = sp["M"], sp["N"], sp["K"]
            offs = sp["offs"]
            lo, hi = oracle.group_bounds(offs, M)
            e = int(np.argmax(hi - lo))
            m, n = min(1024, int(hi[e] - lo[e])), min(4096, N)
            rows = slice(int(lo[e]), int(lo[e]) + m)
            qa = h(sp["qa"][rows])
            qb = h(sp["qb"].view(len(offs), N, K)[e, :n])[None]
            one = np.array([m], np.int32)
            if sp["sk"] == 0:
                sa, sb = h(sp["sa"][rows]), h(sp["sb"].view(len(offs), N)[e, :n])[None]
                f = lambda: oracle.mm_grouped_m(qa, sa, qb, sb, one, 0, 0)
            else:
                sa = _k4_rows(h(sp["sa"]), M, K // 32)[rows]
                sb = _k4_rows(h(sp["sb"]), len(offs) * N, K // 32).reshape(len(offs), N, K // 32)[e:e + 1, :n]
                f = lambda: oracle.mm_grouped_m_mx(qa, sa, qb, sb, one)
            full = 2.0 * float((hi - lo).sum()) * N * K
            add(name, timed(f), full / (2.0 * m * n * K))
        elif op == "g_k":
            Mc, N, K = sp["M"], sp["N"], sp["K"]
            offs = sp["offs"] if isinstance(sp["offs"], np.ndarray) else h(sp["offs"])
            lo, hi = oracle.group_bounds(offs, Mc)
            e = int(np.argmax(hi - lo))
            n, k = min(1024, N), min(4096, K)
            cols = slice(int(lo[e]), int(hi[e]))
            qa, qb = h(sp["qa"][:n])[:, cols], h(sp["qb"][:k])[:, cols]
            one = np.array([int(hi[e] - lo[e])], np.int32)
            if sp["sk"] == 0:
                sa, sb = h(sp["sa"][e:e + 1, :n]), h(sp["sb"][e:e + 1, :k])
                f = lambda: oracle.mm_grouped_k(np.ascontiguousarray(qa), sa, np.ascontiguousarray(qb), sb, one, 0, 0)
            else:
                sa = _k4_rows(h(sp["sa"]), N, Mc // 32)[:n, int(lo[e]) // 32:int(hi[e]) // 32]
                sb = _k4_rows(h(sp["sb"]), K, Mc // 32)[:k, int(lo[e]) // 32:int(hi[e]) // 32]
                f = lambda: oracle.mm_grouped_k_mx(np.ascontiguousarray(qa), sa, np.ascontiguousarray(qb), sb, one)
            full = 2.0 * float((hi - lo).sum()) * N * K
            add(name, timed(f), full / (2.0 * n * k * float(hi[e] - lo[e])))
        elif op == "mx_dual":
            x = src(sp["src"])
            if "offs" in sp:
                M, C = sp["shape"]
                x = x.reshape(M, C)
                r = max(1, min(M, QS // max(C, 1)))
                c = max(8, min(C, QS // max(M, 1)) // 32 * 32)
                xs = np.ascontiguousarray(x[:, :c])
                # the two halves scale differently: rows sampled for one, columns for the other
                t_l = timed(lambda: oracle.quantize_mx_lastdim(x[:r], sp["rule"]), 1) * (M / r)
                t_r = timed(lambda: oracle.quantize_mx_rows_grouped(xs, sp["offs"], sp["rule"], sp["rows_pad"]), 1) * (C / c)
            else:
                B, R, C = sp["shape"]
                x = x.reshape(B, R, C)
                r = max(1, min(B * R, QS // max(C, 1)))
                c = max(8, min(C, QS // max(B * R, 1)) // 8 * 8)
                xs = np.ascontiguousarray(x[:, :, :c])
                t_l = timed(lambda: oracle.quantize_mx_lastdim(x.reshape(B * R, C)[:r], sp["rule"]), 1) * (B * R / r)
                t_r = timed(lambda: oracle.quantize_mx_rows_batched(xs, sp["rule"]), 1) * (C / c)
            add(name, t_l + t_r, 1.0)
        elif op == "permute_mx_dual":
            x, rsrc = host[sp["x"]], src(sp["rsrc"])
            M, C = sp["shape"]
            r = max(1, min(M, QS // max(C, 1)))
            c = max(32, min(C, QS // max(M, 1)) // 32 * 32)
            t_l = timed(lambda: oracle.quantize_mx_lastdim(gathered(sp, x, rsrc[:r], C), sp["rule"]), 1) * (M / r)
            t_r = timed(lambda: oracle.quantize_mx_rows_grouped(gathered(sp, x, rsrc, c), sp["offs"], sp["rule"],
                                                                sp["rows_pad"]), 1) * (C / c)
            add(name, t_l + t_r, 1.0)
        elif op == "permute_q_col":
            x, rsrc = host[sp["x"]], src(sp["rsrc"])
            M, C = rsrc.size, x.shape[1]
            c = max(8, min(C, QS // max(M, 1)) // 8 * 8)
            add(name, timed(lambda: oracle.quantize_colwise_grouped(gathered(sp, x, rsrc, c), sp["offs"], 0), 1),
                C / c)
        elif op == "swiglu_mx":
            h1 = src(sp["h1"])
            R, F = h1.shape[0], sp["F"]
            C = F if sp["da2"] is None else 2 * F
            r = max(1, min(R, QS // max(C, 1)))
            if sp["da2"] is None:
                t_r = timed(lambda: oracle.quantize_mx_lastdim(o_swiglu.swiglu_fwd(h1[:r], F), sp["rule"]), 1)
            else:
                da2 = src(sp["da2"])
                t_r = timed(lambda: oracle.quantize_mx_lastdim(o_swiglu.swiglu_bwd(da2[:r], h1[:r], F), sp["rule"]), 1)
            # the row-block form costs what the last-dim form does per element (one more pass over the tensor)
            add(name, 2.0 * t_r, R / r)
        elif op == "route":
            ids = host[sp["ids"]]
            add(name, timed(lambda: o_route.route(ids, sp["E"], sp["pad"]), 1), 1.0)
        elif op in ("permute", "permute_rowwise"):
            x, rsrc = src(sp["src"]), src(sp["rsrc"])
            R, C = rsrc.size, x.shape[1]
            r = max(1, min(R, QS // max(C, 1)))
            sub = rsrc[:r]
            f = (lambda: o_route.permute(x, sub, sp["topk"])) if op == "permute" else \
                (lambda: oracle.quantize_rowwise(o_route.permute(x, sub, sp["topk"]), 0))
            add(name, timed(f, 1), R / r)
        elif op in ("swiglu", "swiglu_bwd"):
            h1 = src(sp["h1"])
            R, F = h1.shape[0], sp["F"]
            r = max(1, min(R, QS // max(2 * F, 1)))
            if op == "swiglu":
                f = (lambda: o_swiglu.swiglu_fwd(h1[:r], F)) if sp["q"] is None else \
                    (lambda: o_swiglu.swiglu_quantize_rowwise(h1[:r], F, 0))
            else:
                da2 = src(sp["da2"])
                f = (lambda: o_swiglu.swiglu_bwd(da2[:r], h1[:r], F)) if sp["q"] is None else \
                    (lambda: o_swiglu.swiglu_backward_quantize_rowwise(da2[:r], h1[:r], F, 0))
            add(name, timed(f, 1), R / r)
        elif op in ("combine", "combine_bwd"):
            yg, dest, k = src(sp["yg"]), src(sp["dest"]), sp["topk"]
            T, C = dest.size // k, yg.shape[1]
            t = max(1, min(T, QS // max(C * k, 1)))
            d = dest[:t * k]
            yg_sub = yg[np.clip(d, 0, None)]
            d_sub = np.where(d >= 0, np.arange(t * k), -1).astype(np.int32)
            wts = None if sp["w"] is None else host[sp["w"]][:t]
            if op == "combine":
                f = lambda: o_route.combine(yg_sub, d_sub, wts, t, k)
            else:
                dy = host[sp["dy"]][:t]
                s_sub = np.arange(t * k, dtype=np.int32)
                f = lambda: o_route.combine_backward(dy, yg_sub, s_sub, d_sub, wts, t, k)
            add(name, timed(f, 1), T / t)
        elif op == "g_k_bf16":
            a, b = host[sp["a"]], host[sp["b"]]
            Mt, N = a.shape
            K = b.shape[1]
            n, k = min(1024, N), min(4096, K)
            an, bk = np.ascontiguousarray(a[:, :n]), np.ascontiguousarray(b[:, :k])
            add(name, timed(lambda: oracle.mm_grouped_k_bf16(an, bk, sp["offs"])), (N * K) / (n * k))
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": round(total_us, 1), "unit": "us/layer", "cores": int(threads), "kind": "oracle",
            "cpu_model": cpu_model(), "cpu_count": os.cpu_count(),
            "sample": f"numpy oracle on a bounded sample of every launch of the step, each scaled linearly to its "
                      f"full size (quantization: about {QS} elements of whole rows or columns, one thread; GEMMs: up "
                      f"to 1024 x 4096 outputs of the largest group over the whole contraction, fp64 BLAS with "
                      f"{threads} threads, scaled by flops): " + ", ".join(pieces)}


# ---------------------------------------------------------------------- traffic evidence

# The sources that define the grouped-GEMM kernels and their launch configuration, whose counters
# profiles/traffic.json holds (the entry-point and declaration files change with every new entry point).
TRAFFIC_SOURCES = ("gemm_grouped.hip", "gemm_common.hpp", "device_common.hpp")


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mxfp8_quantized_moe_amd", "csrc")
    for f in TRAFFIC_SOURCES:
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def _dispatch_counters(db: str, counter: str):
    """[(dispatch_id, kernel_name, value)] of one PMC counter, in dispatch order (value summed
    over the counter's instances)."""
    import sqlite3
    cur = sqlite3.connect(db).cursor()
    acc = {}
    for name, cn, val, disp in cur.execute(
            "select kernel_name, counter_name, value, dispatch_id from counters_collection"):
        if cn != counter:
            continue
        k = acc.setdefault(disp, [name, 0.0])
        k[1] += val
    return [(d, acc[d][0], acc[d][1]) for d in sorted(acc)]


def _item_kib(db: str, counter: str, steps: int) -> float:
    """Counter KiB per launch of the --only item: the run of library dispatches after the last
    dispatch of any other kernel (the marker), divided by the number of timed launches."""
    rows = _dispatch_counters(db, counter)
    tail = []
    for d, name, v in reversed(rows):
        if "fp8moe::" not in name:
            break
        tail.append(v)
    if not tail:
        raise SystemExit(f"{db}: no library dispatches after the marker")
    return sum(tail) / steps


def _copy_factor(db: str, counter: str, nbytes: int) -> float:
    rows = _dispatch_counters(db, counter)
    vals = sorted((v for _, _, v in rows), reverse=True)[:3]
    return nbytes / (float(np.mean(vals)) * 1024.0)


def write_traffic(args):
    fdb, wdb, cfdb, cwdb = args.write_traffic
    if not args.only:
        raise SystemExit("--write-traffic needs --only ITEM (the item the databases were taken for)")
    nbytes = args.copy_mib << 20
    ff, fw = _copy_factor(cfdb, "FETCH_SIZE", nbytes), _copy_factor(cwdb, "WRITE_SIZE", nbytes)
    fetch = _item_kib(fdb, "FETCH_SIZE", args.steps) * 1024.0 * ff
    write = _item_kib(wdb, "WRITE_SIZE", args.steps) * 1024.0 * fw
    p = os.path.join(ROOT, "profiles", "traffic.json")
    d = json.load(open(p)) if os.path.exists(p) else {}
    if d.get("source_digest") != kernel_source_digest():
        d = {"source_digest": kernel_source_digest(), "per_launch_bytes": {}, "detail": {}}
    key = f"cfg{args.config}:{args.only}"
    d["per_launch_bytes"][key] = round(fetch + write)
    d["detail"][key] = {"fetch_bytes": round(fetch), "write_bytes": round(write),
                        "fetch_scale": round(ff, 4), "write_scale": round(fw, 4),
                        "timed_launches": args.steps,
                        "counter_runs": f"rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) -- python bench.py --config "
                                        f"{args.config} --only '{args.only}' --steps {args.steps} --warmup 1 "
                                        f"--no-cpu-baseline; calibration: the same counters on "
                                        f"python bench.py --copy-probe {args.copy_mib}"}
    with open(p, "w") as f:
        json.dump(d, f, indent=1, sort_keys=True)
    print(json.dumps({key: d["detail"][key], "per_launch_bytes": d["per_launch_bytes"][key]}))


def traffic_for(kernel_item: str, cfg: int):
    """HBM bytes per launch measured by rocprofv3 PMC (profiles/traffic.json), or None
    if absent or taken on a different kernel source."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
    except ValueError:
        return None
    if d.get("source_digest") != kernel_source_digest():
        return None
    return d.get("per_launch_bytes", {}).get(f"cfg{cfg}:{kernel_item}")


# ---------------------------------------------------------------------- per-kernel protocol

FLUSH_BYTES = 1 << 30   # read before each flushed repeat: more than the 256 MB last-level cache and the L2s


def per_kernel_flushed(step, stream, warmup=5, repeats=20):
    """Each launch of the step alone: `warmup` untimed launches, then `repeats` timed ones, each after
    a 1 GiB device read that evicts the last-level cache and the L2s (outside the timed events).  A
    read, not a write: a write would leave up to 256 MB of dirty lines whose write-back then falls
    inside the timed launch.  Returns {name: (median, p10, p90)} in microseconds."""
    import torch
    flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda:0")
    res = {}
    step.rot[0] = 0
    for name, _, fn, _, _ in step.items:
        for _ in range(warmup):
            fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(repeats)]
        for r in range(repeats):
            flush.sum()
            ev[r][0].record(stream)
            fn()
            ev[r][1].record(stream)
        torch.cuda.synchronize()
        t = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
        res[name] = tuple(round(float(np.percentile(t, p)), 1) for p in (50, 10, 90))
    del flush
    return res


def _smi_sclk():
    import subprocess
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True, timeout=30)
        d = json.loads(r.stdout)
        for card in d.values():
            for k, v in card.items():
                if "sclk" in k.lower() and "speed" in k.lower():
                    digits = "".join(ch for ch in str(v).split("Mhz")[0] if ch.isdigit() or ch == ".")
                    return float(digits) if digits else None
    except Exception:
        return None
    return None


def observed_sclk(step, seconds=1.5):
    """Shader clock (MHz) that rocm-smi reports while untimed steps run back to back, or None."""
    import threading
    import torch
    box = {}

    def sample():
        time.sleep(seconds / 3)
        box["mhz"] = _smi_sclk()

    th = threading.Thread(target=sample)
    t_end = time.perf_counter() + seconds
    th.start()
    k = 0
    while time.perf_counter() < t_end or th.is_alive():
        step.rot[0] = k % N_ROTATE
        for it in step.items:
            it[2]()
        torch.cuda.synchronize()
        k += 1
        if k > 100000:
            break
    th.join()
    return box.get("mhz")


def swiglu_extras(cfg: int, stream):
    """The fused SwiGLU kernels on the layer's shapes (H1 [M, 2F], dA2 [M, F]; seeded normal inputs),
    timed like kernels_flushed.  Not part of the layer step's call list."""
    import torch
    import mxfp8_quantized_moe_amd as fm
    from mxfp8_quantized_moe_amd import synth
    w = synth.WORKLOADS[cfg]
    M, F = w.M, w.F
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(1000 * cfg + 7)
    h1 = (torch.randn(M, 2 * F, device="cuda:0", generator=gen) * 2).to(torch.bfloat16)
    da2 = (torch.randn(M, F, device="cuda:0", generator=gen) * 1e-3).to(torch.bfloat16)
    a2 = torch.empty(M, F, dtype=torch.bfloat16, device="cuda:0")
    qa = torch.empty(M, F, dtype=torch.uint8, device="cuda:0")
    sa = torch.empty(M, dtype=torch.float32, device="cuda:0")
    dh1 = torch.empty(M, 2 * F, dtype=torch.bfloat16, device="cuda:0")
    qd = torch.empty(M, 2 * F, dtype=torch.uint8, device="cuda:0")
    sd = torch.empty(M, dtype=torch.float32, device="cuda:0")
    st = Step()
    # algorithmic bytes: inputs read once, bf16 result and FP8 codes written once, one fp32 scale per row
    st.add("swiglu+q A2", "quant", lambda: fm.swiglu_quantize_rowwise(h1, 0, a2=a2, q=qa, scale=sa),
           M * (4 * F + 2 * F + F) + 4 * M)
    st.add("swiglu bwd+q dH1", "quant", lambda: fm.swiglu_backward_quantize_rowwise(da2, h1, 0, dh1=dh1, q=qd,
                                                                                    scale=sd),
           M * (2 * F + 4 * F + 4 * F + 2 * F) + 4 * M)
    t = per_kernel_flushed(st, stream)
    out = {}
    for name, _, _, work, _ in st.items:
        med, p10, p90 = t[name]
        out[name] = {"median_us": med, "p10_us": p10, "p90_us": p90, "GBps": round(work / med / 1e3, 1),
                     "frac": round(work / med / 1e3 / PEAK_HBM_GBPS, 4), "rows": M, "F": F}
    return out


def blockwise_extras(stream):
    """The blockwise recipe's launches on the Llama3-8B linear layer (M = 8192, H = 4096, F = 14336), timed
    like kernels_flushed: X and dY in 1 x 128 tiles, W and W^T in 128 x 128 tiles, the token-major dY and X in
    128-token blocks for the weight gradient, and the three blockwise GEMMs.  Not the layer step (its W^T is a
    bf16 transpose made once outside the timing)."""
    import torch
    import mxfp8_quantized_moe_amd as fm
    M, K, N = 8192, 4096, 14336
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(2024)
    x = torch.randn(M, K, device="cuda:0", generator=gen).to(torch.bfloat16)
    w = (torch.randn(N, K, device="cuda:0", generator=gen) * 0.02).to(torch.bfloat16)
    dy = (torch.randn(M, N, device="cuda:0", generator=gen) * 1e-3).to(torch.bfloat16)
    wt = w.t().contiguous()
    offs = torch.tensor([M], dtype=torch.int32, device="cuda:0")
    qx, sx = fm.quantize_blockwise(x, 1)
    qw, sw = fm.quantize_blockwise(w.view(1, N, K), 128)
    qdy, sdy = fm.quantize_blockwise(dy, 1)
    qwt, swt = fm.quantize_blockwise(wt.view(1, K, N), 128)
    qdyt, sdyt = fm.quantize_blockwise_tokens(dy, offs)
    qxt, sxt = fm.quantize_blockwise_tokens(x, offs)
    o_f = torch.empty(M, N, dtype=torch.bfloat16, device="cuda:0")
    o_d = torch.empty(M, K, dtype=torch.bfloat16, device="cuda:0")
    o_w = torch.empty(1, N, K, dtype=torch.bfloat16, device="cuda:0")
    qb = lambda n_elem, n_scale: 3 * n_elem + 4 * n_scale
    st = Step()
    st.add("q_block X (1x128)", "quant", lambda: fm.quantize_blockwise(x, 1, q=qx, scale=sx), qb(M * K, M * K // 128))
    st.add("q_block W (128x128)", "quant", lambda: fm.quantize_blockwise(w.view(1, N, K), 128, q=qw, scale=sw),
           qb(N * K, N * K // 16384))
    st.add("gemm fwd blockwise", "gemm", lambda: fm.grouped_mm_blockwise(qx, sx.view(M, -1), qw, sw, offs, 1, M, N, K,
                                                                          out=o_f), 2.0 * M * N * K)
    st.add("q_block dY (1x128)", "quant", lambda: fm.quantize_blockwise(dy, 1, q=qdy, scale=sdy),
           qb(M * N, M * N // 128))
    st.add("q_block W^T (128x128)", "quant", lambda: fm.quantize_blockwise(wt.view(1, K, N), 128, q=qwt, scale=swt),
           qb(N * K, N * K // 16384))
    st.add("gemm dgrad blockwise", "gemm", lambda: fm.grouped_mm_blockwise(qdy, sdy.view(M, -1), qwt, swt, offs, 1, M,
                                                                            K, N, out=o_d), 2.0 * M * N * K)
    st.add("q_tokens dY", "quant", lambda: fm.quantize_blockwise_tokens(dy, offs, q_t=qdyt, scale=sdyt),
           qb(M * N, M * N // 128))
    st.add("q_tokens X", "quant", lambda: fm.quantize_blockwise_tokens(x, offs, q_t=qxt, scale=sxt),
           qb(M * K, M * K // 128))
    st.add("gemm wgrad blockwise", "gemm", lambda: fm.grouped_mm_blockwise_k(qdyt, sdyt, qxt, sxt, offs, M, out=o_w),
           2.0 * M * N * K)
    t = per_kernel_flushed(st, stream)
    res = {}
    for name, kind, _, work, _ in st.items:
        med, p10, p90 = t[name]
        if kind == "gemm":
            res[name] = {"median_us": med, "p10_us": p10, "p90_us": p90, "TFLOPs": round(work / med / 1e6, 1),
                         "frac": round(work / med / 1e6 / PEAK_FP8_TFLOPS, 4)}
        else:
            res[name] = {"median_us": med, "p10_us": p10, "p90_us": p90, "GBps": round(work / med / 1e3, 1),
                         "frac": round(work / med / 1e3 / PEAK_HBM_GBPS, 4)}
    res["sum_of_medians_us"] = round(sum(t[name][0] for name, *_ in st.items), 1)
    return res


def route_extras(cfg: int, stream):
    """The routing kernels on the layer's per-token routing (tokens x topk ids over E experts, no
    padding) and hidden size H: route, permute of X [T, H] into the grouped rows, combine of a grouped
    output [rows, H] back to [T, H]; timed like kernels_flushed.  Not part of the layer step."""
    import torch
    import mxfp8_quantized_moe_amd as fm
    from mxfp8_quantized_moe_amd import synth
    w = synth.WORKLOADS[cfg]
    ids_h = synth.routing_ids(cfg)
    T, k = ids_h.shape
    S, H, E = T * k, w.H, w.E
    ids = torch.from_numpy(ids_h).to("cuda:0")
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(1000 * cfg + 11)
    x = torch.randn(T, H, device="cuda:0", generator=gen).to(torch.bfloat16)
    wts = torch.rand(T, k, device="cuda:0", generator=gen)
    counts, offs, dest, src = fm.moe_route(ids, E, 1)
    R = src.numel()
    ws = torch.empty(max(int(fm._lib.lib().moe_route_workspace_bytes(S, E)), 4), dtype=torch.uint8, device="cuda:0")
    xg = fm.moe_permute(x, src, k)
    y = torch.empty(T, H, dtype=torch.bfloat16, device="cuda:0")
    q_tok, s_tok = fm.quantize_rowwise(x, 0)
    qg, sg = torch.empty(R, H, dtype=torch.uint8, device="cuda:0"), torch.empty(R, dtype=torch.float32,
                                                                                 device="cuda:0")
    q_rows, s_rows = torch.empty(R, H, dtype=torch.uint8, device="cuda:0"), torch.empty(R, dtype=torch.float32,
                                                                                        device="cuda:0")
    st = Step()
    # algorithmic bytes: ids read once, dest and src written once (plus counts and offsets)
    st.add("route", "route", lambda: fm.moe_route(ids, E, 1, out=(counts, offs, dest, src), workspace=ws),
           4 * S + 4 * S + 4 * R + 8 * E)
    # X read once, the grouped rows and src once
    st.add("permute X", "route", lambda: fm.moe_permute(x, src, k, xg=xg), 2 * T * H + 2 * R * H + 4 * R)
    # the two orders of gather and rowwise quantization for the first GEMM's operand:
    # bf16 gather (above) then quantizing the R grouped rows, or quantizing the T tokens then gathering codes
    st.add("q_row grouped X", "route", lambda: fm.quantize_rowwise(xg, 0, q=q_rows, scale=s_rows),
           3 * R * H + 4 * R)
    st.add("q_row tokens X", "route", lambda: fm.quantize_rowwise(x, 0, q=q_tok, scale=s_tok), 3 * T * H + 4 * T)
    st.add("permute q(X)", "route", lambda: fm.moe_permute_quantized(q_tok, s_tok, src, k, 0, qg=qg, scale_g=sg),
           T * H + R * H + 4 * R + 4 * T)
    # every grouped row read once, dest and weights once, Y written once
    st.add("combine Y", "route", lambda: fm.moe_combine(xg, dest, wts, k, y=y), 2 * R * H + 8 * S + 2 * T * H)
    t = per_kernel_flushed(st, stream)
    out = {}
    for name, _, _, work, _ in st.items:
        med, p10, p90 = t[name]
        out[name] = {"median_us": med, "p10_us": p10, "p90_us": p90, "GBps": round(work / med / 1e3, 1),
                     "frac": round(work / med / 1e3 / PEAK_HBM_GBPS, 4), "tokens": T, "topk": k, "E": E, "H": H}
    return out


# ---------------------------------------------------------------------- main

def main():
    args = parse()
    if args.write_traffic:
        write_traffic(args)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1",
                          "n_gpus_requested": args.gpus}))
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs an MI355X"
    if args.copy_probe:
        n = args.copy_probe << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        ev[0].record()
        for i in range(3):
            dst.copy_(src)
            ev[i + 1].record()
        torch.cuda.synchronize()
        us = [ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(1, 3)]   # the first launch warms up
        gbs = 2 * n / (sum(us) / len(us) * 1e-6) / 1e9                    # n bytes read + n written
        print(json.dumps({"copy_probe_bytes": n, "launches": 3, "us_per_copy": round(sum(us) / len(us), 1),
                          "GBps": round(gbs, 1), "frac_of_8TBps": round(gbs / 8000.0, 3)}), flush=True)
        return
    import mxfp8_quantized_moe_amd  # noqa: F401  (fails loudly if the HIP library is missing)
    from mxfp8_quantized_moe_amd import synth

    if args.tensorwise and args.config != 2:
        raise SystemExit("--tensorwise is built for config 2 (the Llama3-8B linear layer)")
    progress(f"config {args.config}: inputs")
    step, host = build_step(args.config, args.gw, args.tensorwise, keep_host=not args.no_cpu_baseline,
                            experts_only=args.experts_only)
    layer = args.config in (3, 4, 5) and not args.experts_only
    progress(f"config {args.config}: {len(step.items)} launches; warm-up")
    stream = torch.cuda.current_stream()
    names = [it[0] for it in step.items]
    for w_i in range(args.warmup):
        step.rot[0] = w_i % N_ROTATE
        for it in step.items:
            it[2]()
    torch.cuda.synchronize()
    if args.only is not None:
        sel = [it for it in step.items if it[0] == args.only]
        if not sel:
            raise SystemExit(f"--only: no launch named {args.only!r}; launches: {names}")
        step.items = sel
        torch.zeros(1, device="cuda:0").add_(1)      # marker dispatch for counter passes
        torch.cuda.synchronize()

    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in step.items]
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step.rot[0] = s % N_ROTATE
        for i, it in enumerate(step.items):
            ev[s][i][0].record(stream)
            it[2]()
            ev[s][i][1].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    per = {}
    for i, (name, kind, _, work, hbm) in enumerate(step.items):
        us = float(np.mean([ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(args.steps)])) * 1e3
        per[name] = (kind, work, us, hbm)
    q_bytes = sum(v[1] for v in per.values() if v[0] == "quant")
    q_us = sum(v[2] for v in per.values() if v[0] == "quant")
    m_bytes = sum(v[1] for v in per.values() if v[0] == "moe")
    m_us = sum(v[2] for v in per.values() if v[0] == "moe")
    g_flops = sum(v[1] for v in per.values() if v[0] == "gemm")
    g_us = sum(v[2] for v in per.values() if v[0] == "gemm")

    def roof(kind, work, us, hbm):
        """(bound, achieved, peak, unit): a GEMM is HBM-bound when moving its algorithmic bytes at
        peak bandwidth takes longer than its flops at peak MFMA rate."""
        if kind in ("quant", "moe"):
            return "hbm", work / us / 1e3, PEAK_HBM_GBPS, "GB/s"
        peak_f = PEAK_BF16_TFLOPS if kind == "gemm_bf16" else PEAK_FP8_TFLOPS
        if hbm / PEAK_HBM_GBPS / 1e3 > work / peak_f / 1e6:
            return "hbm", hbm / us / 1e3, PEAK_HBM_GBPS, "GB/s"
        return "mfma", work / us / 1e6, peak_f, "TFLOP/s"

    dom = max(per, key=lambda k: per[k][2])
    bound, achieved, peak, unit = roof(*per[dom])
    fracs = {}
    for k, v in per.items():
        b, a, pk, _ = roof(*v)
        fracs[k] = {"bound": b, "frac": round(a / pk, 4)}

    progress(f"timed {args.steps} steps: {ms_per_step * 1e3:.1f} us per step")
    extras = args.only is None and not args.no_per_kernel
    flushed = per_kernel_flushed(step, stream) if extras else {}
    if extras:
        progress("per-kernel pass done")
    w = synth.WORKLOADS[args.config]
    out = {
        "metric": "quant HBM GB/s + grouped-GEMM TFLOP/s; us per MoE layer (quant+GEMM)",
        "value": round(ms_per_step * 1e3, 1),
        "unit": "us/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp8" if w.mx else "fp8",
        "data": "synthetic",
        "config": {"workload": w.name, "experts": w.E, "routed_rows": w.M, "hidden": w.H,
                   "w1_out": w.F2, "w2_in": w.F,
                   **({"tokens": synth.tokens_topk(args.config)[0], "topk": synth.tokens_topk(args.config)[1]}
                      if layer else {}),
                   "step": ("MoE layer fwd+bwd: route, permute, W1, SwiGLU, W2, combine; combine bwd, "
                            "W2 dgrad+wgrad, SwiGLU bwd, W1 dgrad+wgrad, input-gradient combine" if layer else
                            ("fwd" if args.config == 1 else "fwd+dgrad+wgrad") + ("+bf16 wgrad" if args.gw else "")),
                   "recipe": "mxfp8 (e8m0 per 1x32)" if w.mx else
                   "fp8 e4m3fn tensorwise (one scale per tensor)" if args.tensorwise else
                   "fp8 e4m3fn rowwise + colwise backward",
                   **({"only": args.only} if args.only else {})},
        "quant_GBps": round(q_bytes / q_us / 1e3, 1) if q_us else None,
        "quant_us": round(q_us, 1),
        **({"moe_ops_GBps": round(m_bytes / m_us / 1e3, 1), "moe_ops_us": round(m_us, 1)} if m_us else {}),
        "gemm_TFLOPs": round(g_flops / g_us / 1e6, 1) if g_us else None,
        "gemm_us": round(g_us, 1),
        "kernels_us": {k: round(v[2], 1) for k, v in per.items()},
        "roofline": {"kernel": dom, "bound": bound, "achieved": round(achieved, 1), "peak": peak, "unit": unit,
                     "frac": round(achieved / peak, 4), "traffic": traffic_for(dom, args.config)},
        "kernels_roofline": fracs,
        "kernels_flushed": {k: {"median_us": v[0], "p10_us": v[1], "p90_us": v[2],
                                "frac": round(roof(per[k][0], per[k][1], v[0], per[k][3])[1]
                                              / roof(per[k][0], per[k][1], v[0], per[k][3])[2], 4)}
                            for k, v in flushed.items()},
        "peaks": {"hbm_GBps": PEAK_HBM_GBPS, "fp8_TFLOPs": PEAK_FP8_TFLOPS, "bf16_TFLOPs": PEAK_BF16_TFLOPS},
        "sclk_MHz_under_load": observed_sclk(step) if extras else None,
        "inputs": f"{N_ROTATE} device copies of every input, step s reads copy s % {N_ROTATE}",
    }
    if args.swiglu and args.config in (3, 4):
        out["swiglu_fused"] = swiglu_extras(args.config, stream)
    if args.blockwise and args.config == 2:
        out["blockwise_recipe"] = blockwise_extras(stream)
    if args.route and args.config in (3, 4):
        out["routing"] = route_extras(args.config, stream)
    if not args.no_cpu_baseline and args.only is None and not args.tensorwise:
        progress("oracle baseline on the host")
        out["cpu_baseline"] = cpu_baseline(step, host)
    else:
        out["cpu_baseline"] = None      # the tensorwise recipe's launches carry no oracle spec
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
