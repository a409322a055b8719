"""VBR degrade steps: re-encoding one (layer, side) tensor one rung down, and
the order in which the classic ladder moves tensors.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: the buun-llama-cpp page, "VBR -- Variable Bit-Rate KV Cache".  The
cache starts at f16 and, under budget pressure, degrades one (layer, side)
tensor at a time down a ladder of codecs, following a per-model price order.
The classic ladder is f16 -> q8_0 -> q4_0, taken band by band: no tensor
moves from q8_0 to q4_0 while a movable tensor is still at f16.  A side
pinned to a fixed type never degrades, and degrades stop at the last step
whose aggregate bits/value is still at or above the floor.

Readings (the page gives no arithmetic for a degrade step):

* A degrade step re-encodes the rows a tensor holds: each stored row is
  decoded to its values and encoded with the next codec, exactly as a new
  row with those values would be appended.  Only sources whose decoded values
  are exact in fp32 are re-encoded this way: f16 (an fp16 value), q8_0 (an
  int8 code times an fp16 scale: at most 8 + 11 significant bits) and q4_0
  (a code in -8..7 times an fp16 scale).  The encoders take fp32 input, so
  the step is well defined bit for bit.
* The destination is any codec with fewer bits per value than the source
  (f16 -> q8_0 / q4_0 / rot4, q8_0 -> q4_0 / rot4), rot4 standing in for the
  page's turbo4 rung.  The oracle also accepts the source's own codec, which
  makes the step an identity on stored rows (a pinned invariant).
* The price order is the caller's (the page measures it per model on KLD
  panels, which are not available); aggregate bits/value weighs equally sized
  tensors equally.
"""

import numpy as np

from . import codecs
from .bytes_model import BPV

EXACT_SOURCES = ("f16", "q8_0", "q4_0")
CLASSIC_LADDER = ("f16", "q8_0", "q4_0")


def transcode(src_codec, dst_codec, q_src, src_signs=None, dst_signs=None):
    """Re-encode stored rows: decode them with the source codec, then encode
    the values with the destination codec (``codecs.quantize``)."""
    assert src_codec in EXACT_SOURCES, f"{src_codec} rows do not decode exactly to fp32"
    assert BPV[dst_codec] <= BPV[src_codec], "a degrade step never adds bits"
    x = codecs.dequant(src_codec, q_src, src_signs)  # fp64
    x32 = x.astype(np.float32)
    assert np.array_equal(x32.astype(np.float64), x), "decoded values must be exact in fp32"
    return codecs.quantize(dst_codec, x32, dst_signs)


def aggregate_bpv(tensor_codecs):
    """Mean bits/value over equally sized (layer, side) tensors."""
    return sum(BPV[c] for c in tensor_codecs) / len(tensor_codecs)


def classic_next_step(tensor_codecs, price_order, movable=None, floor_bpv=None):
    """The next step of the classic ladder, as (tensor index, new codec), or
    None when no step is left.

    tensor_codecs: current codec of every (layer, side) tensor, each on the
    classic ladder; price_order: tensor indices, cheapest to degrade first;
    movable: False for pinned tensors (default: all movable); floor_bpv: the
    aggregate bits/value may not drop below it.

    Banding: the candidates are the movable tensors on the highest rung any
    movable tensor still occupies (so all of them leave f16 before any leaves
    q8_0); the first candidate in price order moves one rung down.
    """
    n = len(tensor_codecs)
    assert sorted(price_order) == list(range(n)), "price order must name every tensor once"
    movable = [True] * n if movable is None else list(movable)
    rung = [CLASSIC_LADDER.index(c) for c in tensor_codecs]
    open_rungs = [rung[i] for i in range(n) if movable[i] and rung[i] < len(CLASSIC_LADDER) - 1]
    if not open_rungs:
        return None
    top = min(open_rungs)  # the least degraded rung still held by a movable tensor
    for i in price_order:
        if movable[i] and rung[i] == top:
            new = CLASSIC_LADDER[top + 1]
            if floor_bpv is not None:
                after = list(tensor_codecs)
                after[i] = new
                if aggregate_bpv(after) < floor_bpv:
                    return None
            return i, new
    raise AssertionError("unreachable: a movable tensor holds the top open rung")


def classic_schedule(tensor_codecs, price_order, movable=None, floor_bpv=None):
    """Every step the classic ladder takes from this state, in order."""
    state = list(tensor_codecs)
    steps = []
    while True:
        st = classic_next_step(state, price_order, movable, floor_bpv)
        if st is None:
            return steps
        state[st[0]] = st[1]
        steps.append(st)
