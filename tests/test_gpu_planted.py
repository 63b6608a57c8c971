"""GPU planted controls: builds of the library that each carry one deliberate
mistake (a test-only compile define; product builds never set one) must turn a
named parity test red, the CPU-side comparison with the oracle failing on their
results (TensorFold PR #2595 receipt: every planted control red as planted).

  combine_nan_to_zero   the log-sum-exp combine writes 0 where a NaN partial must
                        make the output NaN (HartsyInference PR #910 review item 1)
  alibi_before_softcap  the mask-mode kernel adds the ALiBi bias before the soft
                        cap instead of after it
  keep_repeats          the selected-key kernel visits a repeated block id once per
                        repeat instead of once (strix-llama.cpp PR #115)

Each named test also passes on the product build in the same process first.
"""

import contextlib
import os

import pytest
import torch

import split_flash_attention_amd as sa
from split_flash_attention_amd import build
from tests import test_gpu_parity as tp

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    sa.lib()


@contextlib.contextmanager
def planted(name):
    path = build.plant_path(name)
    if not os.path.exists(path):
        pytest.fail(f"{path} is not built (build() makes the planted variants)")
    product = sa.lib()
    sa._lib = sa.load(path)
    try:
        yield
    finally:
        sa._lib = product


CONTROLS = {
    "combine_nan_to_zero": ("test_decode_nan_propagation[work_group_bf16]",
                            lambda: tp.test_decode_nan_propagation("work_group_bf16")),
    "alibi_before_softcap": ("test_prefill_mask_softcap_then_alibi", tp.test_prefill_mask_softcap_then_alibi),
    "keep_repeats": ("test_prefill_selection_parity[bf16]", lambda: tp.test_prefill_selection_parity("bf16")),
}


@pytest.mark.parametrize("plant", sorted(CONTROLS))
def test_planted_mistake_turns_named_test_red(plant):
    what, run = CONTROLS[plant]
    run()                                         # green on the product build
    with planted(plant):
        with pytest.raises(AssertionError):
            run()                                 # red with the mistake planted
