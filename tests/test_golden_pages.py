"""Values the pages print, with their citation (tests/golden/)."""
import json
import os

import numpy as np

import oracle.attention as orc
import mea_inputs as inp

HERE = os.path.dirname(os.path.abspath(__file__))


def test_scrapbox_single_query_agrees_with_last_row():
    g = json.load(open(os.path.join(HERE, "golden", "kv_cache_check_scrapbox.json")))
    last = np.array(g["full_product_last_row"])
    for key in ("single_query_first", "single_query_second"):
        assert np.allclose(np.array(g[key]), last, rtol=0, atol=10.0 ** -(g["printed_digits"] - 2))


def test_same_check_with_softmax_on_the_pages_shape():
    """The page's shape (1 batch, 1 head, 5 tokens, width 8) through the oracle:
    the newest query against the whole cache equals row 5 of causal attention."""
    c = inp.dense_case(2024, 1, 5, 5, 1, 1, 8, "fp16")
    full, _ = orc.fwd(c["q"], c["k"], c["v"], "fp16", 1.0 / np.sqrt(8), causal=True)
    dec = orc.decode(c["q"][:, 4], c["k"], c["v"], np.array([5], np.int32), "fp16", 1.0 / np.sqrt(8))
    assert np.max(np.abs(dec[0] - full[0, 4])) < 1e-12
