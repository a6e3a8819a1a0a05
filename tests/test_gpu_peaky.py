"""GPU parity on peaky softmaxes (the HIP path through the C ABI against the
fp64 oracle, 3e-3 max-abs).

N(0,1) inputs give a flat softmax: after a chunk's first tile no score rises
far above the running max and no few keys dominate. Real heads are not like
that, so these cases plant logit structure (synth.plant_peaks): Q scaled up,
scores that rise along the path, late spikes in the root and the leaves, an
attention sink on the first token, and two near-equal dominant keys (with
independent values, and with opposite values). They drive

* the lazy rescale of the running max in the middle of a chunk, in every
  row path (single-wave MFMA items, LDS workgroup items, the fp32 GEMV path);
* the rounding of the softmax weights for the bf16 P V product, where a few
  large weights decide the output (the hi + lo split of large weights);
* the log-sum-exp merge of partials whose maxima lie far apart (a sink in one
  root chunk, spikes in leaves).

tests/test_peaky_inputs.py checks on the CPU that these inputs really raise
the running max mid-chunk by more than the rescale threshold.
"""
import pytest
import torch

import synth
from oracle import tree_attention as ta
from parity_util import check, log, run

pytestmark = pytest.mark.gpu

ROOT_LEN = 1100  # every query sees more than 1024 tokens


def peaky_tree(cls, kind, dtype, d, seed=0):
    """cls 'wave': every group has at most 16 rows (single-wave items only).
    cls 'workgroup': a 192-row root and 16-row leaves (leaf-local causal
    mask, qpl 4): workgroup items only; the root's 96-row blocks run 32-row
    tiles (32x32 matrix instruction), the leaves 16-row tiles."""
    if cls == "wave":
        par, lens, qpl = [-1, 0, 0, 0, 0], [ROOT_LEN, 60, 200, 350, 33], 1
    else:
        par = [-1] + [0] * 12
        lens = [ROOT_LEN] + [20 + 37 * i for i in range(12)]
        qpl = 4
    inst = synth.make_tree(par, lens, page_size=16, qpl=qpl, n_qheads=8, n_kvheads=2, head_dim=d, dtype=dtype,
                           seed=seed)
    synth.fill_tensors(inst, seed=100 + seed)
    if kind != "none":
        synth.plant_peaks(inst, kind, seed=200 + seed)
    return inst


@pytest.mark.parametrize("kind", ("none",) + synth.PEAK_KINDS)
@pytest.mark.parametrize("cls", ["wave", "workgroup"])
@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.bfloat16, 64), (torch.float32, 128),
                                     (torch.float32, 64)])
def test_peaky_softmax(kind, cls, dtype, d):
    log(f"peaky {kind} {cls} {dtype} d{d}")
    inst = peaky_tree(cls, kind, dtype, d)
    ref = ta.decode_instance(inst)
    check(run(inst), ref, f"peaky {kind} {cls} {str(dtype)[6:]} d{d}")
    # one chunk per group: the whole root in one stream, so the running max
    # is raised mid-stream many tiles after the first
    check(run(inst, split=False), ref, f"peaky {kind} {cls} {str(dtype)[6:]} d{d} no split")


@pytest.mark.parametrize("kind", synth.PEAK_KINDS)
def test_peaky_workloads(kind):
    """Peaky logits on the skewed long-context workload's shape (GQA 16,
    workgroup items over many root chunks whose partials are merged), with a
    shorter root so the oracle stays quick, and on a random radix tree."""
    inst = synth.make_tree([-1] + [0] * 10, [6000] + [400] * 10, page_size=16, qpl=1, n_qheads=64, n_kvheads=4,
                           head_dim=128, dtype=torch.bfloat16, seed=7)
    synth.fill_tensors(inst, seed=8)
    synth.plant_peaks(inst, kind, seed=9)
    check(run(inst), ta.decode_instance(inst), f"peaky {kind} skewed long context")
    inst = synth.random_small_tree(31, max_nodes=40, max_len=900, qpl=4, heads=(32, 8), head_dim=128,
                                   dtype=torch.bfloat16)
    synth.plant_peaks(inst, kind, seed=10)
    check(run(inst), ta.decode_instance(inst), f"peaky {kind} random tree")
