"""kvsel_read_probe: runs over buffers of several sizes (a single 16-byte
word, a ragged tail past the unrolled loop, 64 MiB) and writes nothing when
the data fold is not the sentinel (zeroed data folds to 0)."""
import pytest
import torch

from tests.parity_util import note

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n_words", [4, (1 << 18) + 4, 1 << 24])
def test_read_probe_reads_without_writing(n_words):
    import attention_score_guided_amd as K
    note(f"read probe over {n_words * 4} bytes")
    buf = torch.zeros(n_words, dtype=torch.int32, device="cuda")
    out = torch.full((1,), -5, dtype=torch.int32, device="cuda")
    K.read_probe(buf, out)
    torch.cuda.synchronize()
    assert int(out[0]) == -5
