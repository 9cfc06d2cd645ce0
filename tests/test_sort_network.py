"""The 12-input sorting network the float-key top-N kernel walks its cached candidates
with: by the 0-1 principle, a comparator network sorts every input iff it sorts every
input of zeros and ones, so all 4096 such inputs are run through the table as the
kernel source holds it."""
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _network():
    with open(os.path.join(ROOT, "binarized_qk_sparse_amd", "csrc", "topn_mfma.hip")) as f:
        text = f.read()
    m = re.search(r"constexpr int kSort12\[(\d+)\]\[2\] = \{(.*?)\};", text, re.S)
    assert m is not None
    pairs = [(int(a), int(b)) for a, b in re.findall(r"\{(\d+),\s*(\d+)\}", m.group(2))]
    assert len(pairs) == int(m.group(1))
    return pairs


def test_network_sorts_every_zero_one_input_descending():
    pairs = _network()
    assert all(0 <= i < j < 12 for i, j in pairs)
    for mask in range(1 << 12):
        v = [(mask >> k) & 1 for k in range(12)]
        for i, j in pairs:
            if v[i] < v[j]:
                v[i], v[j] = v[j], v[i]
        assert all(v[k] >= v[k + 1] for k in range(11)), mask


def test_a_broken_network_is_caught():
    # the same check on the network with one comparator dropped must fail somewhere
    pairs = _network()[:-1]
    failed = False
    for mask in range(1 << 12):
        v = [(mask >> k) & 1 for k in range(12)]
        for i, j in pairs:
            if v[i] < v[j]:
                v[i], v[j] = v[j], v[i]
        if any(v[k] < v[k + 1] for k in range(11)):
            failed = True
            break
    assert failed
