"""One weight-streaming decode step over a stack of W12 layers, built from the library's
entry points only (every GEMM, rescale and the verification run in its HIP kernels).

Dataflow per layer (no nonlinearity; rms(v) = v / sqrt(mean(v^2)) per row, rounded to
BF16):  q, k, v = h W_q^T, h W_k^T, h W_v^T;  o = rms(q) W_o^T;  gate, up = rms(o)
W_gate^T, rms(o) W_up^T;  down = rms(up) W_down^T;  h <- rms(down).  k, v and gate are
computed and not fed forward.  After the last layer the LM head verifies a draft block
greedily on the final h (exact-logit argmax per row, accepted-prefix length), which is
the verification step of greedy speculative decoding in "StargazerX0/SpecPilot"
(hotrepo.ai digest), section "Results and verification"; W12 weights are read inside
the GEMMs as in "SpecPilot: an agent doubled speculative decoding speed, and the 10.87x
needs context", section "The mechanisms it found".
"""
from __future__ import annotations

from . import w12

MATS = ("q", "k", "v", "o", "gate", "up", "down")


class DecodeStack:
    """Layers: a list of dicts name -> W12Tensor (names as in MATS); head: W12Tensor of
    the LM head.  All activation buffers are allocated once for m rows."""

    def __init__(self, layers, head, m: int):
        import torch
        if not layers:
            raise ValueError("empty layer stack")
        self.layers, self.head, self.m = layers, head, m
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

    def _layer_calls(self, L):
        o = self.out
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
        self.calls = [[c for c in self._layer_calls(L)] for L in self.layers]
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
        {layer: {"h", "a", "b", "c", *MATS}}.  Returns (h, argmax, accepted, captured)."""
        self.prepare(draft)
        caps = {}
        self.h.copy_(h0)
        for li, calls in enumerate(self.calls):
            if li in capture:
                h_in = self.h.clone()
            for c in calls:
                c()
            if li in capture:
                caps[li] = {"h": h_in, "a": self.a.clone(), "b": self.b.clone(),
                            "c": self.c.clone(), **{k: v.clone() for k, v in self.out.items()}}
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
            for name in ("q", "o", "up", "down"):         # rescales: read + write
                total += 2 * 2 * m * L[name].n
        t = self.head
        total += 2 * m * t.k + 8 * m * t.n + 4 * m        # x, logits written + read, argmax
        return total
