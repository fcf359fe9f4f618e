"""One weight-streaming decode step over a stack of W12 layers, built from the library's
entry points only (every GEMM, rescale and the verification run in its HIP kernels).

Dataflow per layer (no nonlinearity; rms(v) = v / sqrt(mean(v^2)) per row):  q, k, v =
h W_q^T, h W_k^T, h W_v^T;  o = rms(q) W_o^T;  gate, up = rms(o) W_gate^T, rms(o)
W_up^T;  down = rms(up) W_down^T;  h <- rms(down).  k, v and gate are computed and not
fed forward.  By default every rms(v) W^T runs as one RMS GEMM (w12_gemm_rms /
w12_gemm_group_rms: (v W^T) / rms(v), the division on the FP32 accumulators), so the
next layer's q, k, v read the previous down directly and only the final h is rescaled
on its own (w12_rms_rescale, rounded to BF16); with fused_rms=False every rescale is its
own launch and the GEMMs read the rounded rescaled rows.  After the last layer the LM
head verifies a draft block greedily on the final h (exact-logit argmax per row,
accepted-prefix length), which is the verification step of greedy speculative decoding
in "StargazerX0/SpecPilot" (hotrepo.ai digest), section "Results and verification"; W12
weights are read inside the GEMMs as in "SpecPilot: an agent doubled speculative
decoding speed, and the 10.87x needs context", section "The mechanisms it found".
"""
from __future__ import annotations

from . import w12

MATS = ("q", "k", "v", "o", "gate", "up", "down")


class DecodeStack:
    """Layers: a list of dicts name -> W12Tensor (names as in MATS); head: W12Tensor of
    the LM head.  All activation buffers are allocated once for m rows."""

    def __init__(self, layers, head, m: int, fused_rms: bool = True):
        import torch
        if not layers:
            raise ValueError("empty layer stack")
        self.layers, self.head, self.m, self.fused_rms = layers, head, m, fused_rms
        hid = layers[0]["q"].k
        dev = head.device
        bf = dict(dtype=torch.bfloat16, device=dev)
        out = {name: torch.empty((m, layers[0][name].n), **bf) for name in MATS}
        self.out = out
        self.a = torch.empty((m, layers[0]["o"].k), **bf)       # rms(q): input of o
        self.b = torch.empty((m, layers[0]["gate"].k), **bf)    # rms(o): input of gate/up
        self.c = torch.empty((m, layers[0]["down"].k), **bf)    # rms(up): input of down
        self.h = torch.empty((m, hid), **bf)
        self.argmax = torch.empty(m, dtype=torch.int32, device=dev)
        self.accepted = torch.empty(1, dtype=torch.int32, device=dev)

    def _layer_calls(self, L, first: bool):
        o = self.out
        if self.fused_rms:
            # q, k, v read h (first layer) or the previous down through its RMS; o, gate/up
            # and down read q, o and up through theirs
            qkv_in = self.h if first else o["down"]
            return [w12.prepare_gemm_group(qkv_in, [L["q"], L["k"], L["v"]],
                                           [o["q"], o["k"], o["v"]], rms=not first),
                    w12.prepare_gemm(o["q"], L["o"], o["o"], rms=True),
                    w12.prepare_gemm_group(o["o"], [L["gate"], L["up"]], [o["gate"], o["up"]],
                                           rms=True),
                    w12.prepare_gemm(o["up"], L["down"], o["down"], rms=True)]
        # q, k, v read h and gate, up read rms(o): one grouped launch each
        return [w12.prepare_gemm_group(self.h, [L["q"], L["k"], L["v"]], [o["q"], o["k"], o["v"]]),
                w12.prepare_rms(o["q"], self.a),
                w12.prepare_gemm(self.a, L["o"], o["o"]),
                w12.prepare_rms(o["o"], self.b),
                w12.prepare_gemm_group(self.b, [L["gate"], L["up"]], [o["gate"], o["up"]]),
                w12.prepare_rms(o["up"], self.c),
                w12.prepare_gemm(self.c, L["down"], o["down"]),
                w12.prepare_rms(o["down"], self.h)]

    def prepare(self, draft):
        """Marshal every call of the step once (on the current stream): the layers read
        and write the stack's own buffers; the step starts from self.h."""
        self.calls = [self._layer_calls(L, li == 0) for li, L in enumerate(self.layers)]
        if self.fused_rms:   # the final h, rescaled on its own for the LM head
            self.calls[-1].append(w12.prepare_rms(self.out["down"], self.h))
        self.draft = draft
        self.verify_call = w12.prepare_verify(self.h, self.head, draft, self.argmax, self.accepted)

    def run(self):
        """One step from the current contents of self.h (after prepare)."""
        for calls in self.calls:
            for c in calls:
                c()
        self.verify_call()

    def step(self, h0, draft, capture=()):
        """Run every layer from h0 [m, hidden] and verify `draft` on the final h.
        capture: layer indices whose GEMM inputs and outputs are cloned and returned as
        {layer: {"in": {name: (input, rms applied)}, name: output for name in MATS}}.
        Returns (h, argmax, accepted, captured)."""
        self.prepare(draft)
        caps = {}
        self.h.copy_(h0)
        o = self.out
        for li, calls in enumerate(self.calls):
            if li in capture:
                x_qkv = (self.h if li == 0 or not self.fused_rms else o["down"]).clone()
            for c in calls:
                c()
            if li in capture:
                if self.fused_rms:
                    rq = li > 0
                    ins = {"q": (x_qkv, rq), "k": (x_qkv, rq), "v": (x_qkv, rq),
                           "o": (o["q"].clone(), True), "gate": (o["o"].clone(), True),
                           "up": (o["o"].clone(), True), "down": (o["up"].clone(), True)}
                else:
                    ins = {"q": (x_qkv, False), "k": (x_qkv, False), "v": (x_qkv, False),
                           "o": (self.a.clone(), False), "gate": (self.b.clone(), False),
                           "up": (self.b.clone(), False), "down": (self.c.clone(), False)}
                caps[li] = {"in": ins, **{k: v.clone() for k, v in o.items()}}
        self.verify_call()
        return self.h, self.argmax, self.accepted, caps

    def weight_bytes(self) -> int:
        return sum(t.nbytes() for L in self.layers for t in L.values()) + self.head.nbytes()

    def io_bytes(self) -> int:
        """Activation bytes the GEMMs, rescales and the verification read and write."""
        m = self.m
        total = 0
        for L in self.layers:
            for name in MATS:
                t = L[name]
                total += 2 * m * (t.k + t.n)
            if not self.fused_rms:
                for name in ("q", "o", "up", "down"):     # rescales: read + write
                    total += 2 * 2 * m * L[name].n
        if self.fused_rms:                                # the final h: read + write
            total += 2 * 2 * m * self.layers[-1]["down"].n
        t = self.head
        total += 2 * m * t.k + 2 * 16 * m * (t.n // 16) + 4 * m   # x, block records, argmax
        return total
