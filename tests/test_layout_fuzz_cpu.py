"""Property test of the library's host layout arithmetic against the oracle's, on random
geometries (all three layouts, token rows and page blocks, any alignment), plus the
descriptor check on random, often invalid, descriptors: it answers with a status and
never crashes.  CPU only: these entry points touch no GPU."""
import ctypes

import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from host_device_page_amd import binding as B
from oracle import oracle as O

LAYOUTS = [B.HC_LAYOUT_PAGE_FIRST, B.HC_LAYOUT_KV_SPLIT_SHARD, B.HC_LAYOUT_PAGE_FIRST_TOKEN_MAJOR]


@st.composite
def geometries(draw):
    L = draw(st.integers(1, 80))
    P = draw(st.integers(1, 128))
    nsub = draw(st.integers(1, 4))
    subs = [(draw(st.sampled_from([B.HC_TOKEN_ROWS, B.HC_PAGE_BLOCKS])), 16 * draw(st.integers(1, 600)))
            for _ in range(nsub)]
    H = draw(st.integers(1, 5000))
    S = P * draw(st.integers(1, 5000))
    layout = draw(st.sampled_from(LAYOUTS))
    align = 1 << draw(st.integers(4, 13))
    return L, P, subs, H, S, layout, align


@settings(max_examples=300, deadline=None, derandomize=True, suppress_health_check=[HealthCheck.too_slow])
@given(geometries(), st.data())
def test_host_offsets_match_the_oracle(geom, data):
    L, P, subs, H, S, layout, align = geom
    og = O.Geometry(L, P, subs, H, S, layout, align)
    d, _k = B.make_desc(layers=L, page_size=P, subs=[(g, e, [0x10000] * L) for g, e in subs], device_slots=S,
                        host_pages=H, layout=layout, shard_align=align)
    assert B.host_pool_bytes(d) == O.host_pool_bytes(og)
    assert B.staging_page_bytes(d) == (O.shard_bytes(og) if layout == B.HC_LAYOUT_KV_SPLIT_SHARD
                                       else O.page_payload_bytes(og))
    for _ in range(20):
        b = data.draw(st.integers(0, len(subs) - 1))
        p = data.draw(st.integers(0, H - 1))
        l = data.draw(st.integers(0, L - 1))
        r = data.draw(st.integers(0, P - 1))
        assert B.host_offset(d, b, p, l, r) == O.host_offset(og, b, p, l, r), (b, p, l, r)


@settings(max_examples=500, deadline=None, derandomize=True)
@given(layers=st.integers(-2, 1100), page_size=st.integers(-2, 1 << 21), nsub=st.integers(0, 5),
       elem=st.integers(-16, 1 << 17), gran=st.integers(-1, 2), slots=st.integers(-2, 1 << 62),
       pages=st.integers(-2, 1 << 62), layout=st.integers(-1, 3), align=st.integers(-1, 1 << 20),
       mode=st.integers(-1, 3), flags=st.integers(-1, 8), ctas=st.integers(-1, 70000))
def test_descriptor_check_answers_every_descriptor(layers, page_size, nsub, elem, gran, slots, pages, layout, align,
                                                    mode, flags, ctas):
    nl = max(0, min(layers, 1100))
    subs = [(gran, elem, [0x10000] * max(1, nl))] * max(1, min(nsub, 4))
    d, _k = B.make_desc(layers=layers, page_size=page_size, subs=subs, device_slots=slots, host_pages=pages,
                        layout=layout, shard_align=align, host_ptr=0x7f0000000000, host_bytes=1 << 62,
                        write_back_mode=mode, flags=flags, max_ctas=ctas)
    d.num_subbufs = nsub
    rc = B.lib.hc_desc_check(ctypes.byref(d))
    assert rc in (B.HC_OK, B.HC_ERR_INVALID, B.HC_ERR_UNSUPPORTED)
    if rc != B.HC_OK:
        assert B.lib.hc_last_error().decode()
    out = ctypes.c_int64()
    rc2 = B.lib.hc_host_pool_bytes(ctypes.byref(d), ctypes.byref(out))
    assert rc2 in (B.HC_OK, B.HC_ERR_INVALID, B.HC_ERR_UNSUPPORTED)
    if rc2 == B.HC_OK:
        assert 0 < out.value <= 1 << 62
