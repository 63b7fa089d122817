"""GPU: the cross-workgroup message passing every notify and wait relies on
(device-coherent stores, each wave's store-completion wait, a workgroup
barrier, a relaxed device-scope atomic add; relaxed polls, a barrier,
device-coherent loads), run by the library's self-test between workgroup
pairs on different XCDs, every message word checked."""
import pytest

from gpu_util import announce

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("pairs,rounds", [(256, 400), (64, 2000)])
def test_message_passing_across_xcds(pairs, rounds):
    import torch
    from dynamic_moe_task_amd import binding as B
    announce(f"coherence self-test pairs={pairs} rounds={rounds}")
    nbytes = B.etc_coherence_selftest_bytes(pairs)
    assert nbytes > 0
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    bad, gave_up = B.etc_coherence_selftest(pairs, rounds, ws.data_ptr(), nbytes,
                                            torch.cuda.current_stream().cuda_stream)
    assert gave_up == 0
    assert bad == 0
