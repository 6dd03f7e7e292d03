"""Host-side checks of a plan's device image against what the matrix-core (cascade / extend)
kernel and the merge kernel will index: every access in bounds, and every partial slot a query
row's merge reads written by exactly one work item per query head."""

import numpy as np

NODE_INTS, MEMBER_INTS = 8, 3
INT32_MAX = 2**31 - 1


def check_plan_image(plan, num_q_heads, num_kv_heads, num_blocks):
    img, off, slots_max = plan.image()
    ROWS_PER_ITEM = plan.rows_per_item
    assert ROWS_PER_ITEM == (128 if hasattr(plan, "num_query_rows") else 64)
    group = num_q_heads // num_kv_heads
    nq = plan.num_query_rows if hasattr(plan, "num_query_rows") else plan.batch
    slots = max(slots_max, 1)
    row_info = img[off["row_info"]:off["nodes"]].reshape(-1, 2)
    assert row_info.shape[0] == nq
    nodes = img[off["nodes"]:off["blocks"]].reshape(-1, NODE_INTS)
    blocks = img[off["blocks"]:off["members"]]
    members = img[off["members"]:off["items"]].reshape(-1, MEMBER_INTS)
    seg = img[off["items"]:off["item_recs"]]
    items = seg[:len(seg) // 4 * 4].reshape(-1, 4)
    assert off["item_recs"] % 4 == 0 and off["item_recs"] - off["items"] - 4 * len(items) < 4
    ints = off["item_ints"]
    per_tile = ROWS_PER_ITEM // group
    assert ints == 16 + 4 * per_tile
    recs = img[off["item_recs"]:off["item_recs"] + ints * len(items)].reshape(-1, ints)
    assert len(recs) == len(items)
    written = {}
    for it, (node, hkv, row0, piece) in enumerate(items.tolist()):
        rec = recs[it].tolist()
        if node < 0:  # idle: no blocks, no member rows
            assert rec[:8] == [-1, 0, 0, 0, 0, 0, 0, 0] and rec[8:12] == [-1] * 4 and rec[12:16] == [0] * 4
            assert all(rec[16 + 4 * li: 20 + 4 * li] == [-1, 0, -1, 0] for li in range(per_tile))
            continue
        assert 0 <= node < len(nodes), (it, node)
        assert 0 <= hkv < num_kv_heads
        blk_off, nblocks, mem_off, nmem, pieces, piece_blocks, start_tok, valid = nodes[node].tolist()
        assert 0 <= piece < pieces and piece_blocks >= 1
        pb0 = piece * piece_blocks
        assert pb0 < nblocks
        nblk = min(piece_blocks, nblocks - pb0)
        assert 1 <= nblk <= 256
        assert 0 <= blk_off and blk_off + pb0 + nblk <= len(blocks)
        ids = blocks[blk_off + pb0: blk_off + pb0 + nblk]
        assert ((ids >= 0) & (ids < num_blocks)).all()
        R = nmem * group
        assert 0 <= row0 < R and row0 % ROWS_PER_ITEM == 0
        assert 0 <= mem_off and mem_off + nmem <= len(members)
        # the work item's record: the same item with its node's and members' fields inline
        assert rec[:8] == [hkv, row0, piece, blk_off + pb0, nblk, R, start_tok + 16 * pb0, valid - 16 * pb0], (it, rec[:8])
        assert rec[8:12] == [int(blocks[blk_off + pb0 + j]) if j < nblk else -1 for j in range(4)], (it, rec[8:12])
        assert rec[12:16] == [0, 0, 0, 0]
        for li in range(per_tile):
            e = rec[16 + 4 * li: 20 + 4 * li]
            m = row0 // group + li
            if m < nmem:
                qr, slot0, limit = members[mem_off + m].tolist()
                assert e == [qr, slot0 + piece, limit, 0], (it, li, e)
            else:
                assert e[0] == -1 and e[2] == -1, (it, li, e)
        for row in range(row0, min(row0 + ROWS_PER_ITEM, R)):
            qr, slot0, limit = members[mem_off + row // group].tolist()
            h = hkv * group + row % group
            assert 0 <= qr < nq
            slot = slot0 + piece
            assert 0 <= slot < row_info[qr, 1] <= slots, (it, row, qr, slot, row_info[qr, 1])
            key = (qr, h, slot)
            assert key not in written, f"slot written twice: {key}"
            written[key] = it
    for qr in range(nq):
        depth = int(row_info[qr, 1])
        for h in range(num_q_heads):
            for slot in range(depth):
                assert (qr, h, slot) in written, f"query row {qr} head {h} slot {slot} never written"
    return len(items), len(written)
